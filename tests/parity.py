"""Helpers shared by the GPU parity tests: run the HIP library and the
oracle on the same seeded batch and compare."""

from __future__ import annotations

import json
import os

import numpy as np
import torch

import paged_kv_cache_253_amd as pk
from oracle import paged
from workloads import extract_sequences, host_view

# Tolerances: |gpu - ref| <= atol + rtol * |ref| elementwise, plus a bar on
# each output row (one sequence, one query head): its largest error must stay
# below `norm` times its largest |ref|, so that the small outputs of long
# contexts cannot pass on atol alone.  bf16 output rounding alone reaches
# 2^-8 of a row's largest value; bf16 softmax weights in the matrix-core
# product add about 2^-9 of a value row.
TOL = {
    "f32": dict(atol=1e-5, rtol=1e-4, norm=1e-4),
    "bf16": dict(atol=5e-3, rtol=1e-2, norm=1e-2),
    "fp8_e4m3": dict(atol=2e-2, rtol=1e-2, norm=1e-2),
    "fp8_e5m2": dict(atol=2e-2, rtol=1e-2, norm=1e-2),   # same codes on both sides
    # The bf16 atol scaled by the INT4 values' magnitude: the stated 5e-3 is
    # for N(0, 1) data (rms 1); the INT4 caches hold codes uniform over
    # -8..7 (E[c^2] = 21.5) times scales uniform in [0.25, 0.5) (E[s^2] =
    # 7/48), rms sqrt(21.5 * 7/48) = 1.77, and every error term of the
    # kernels (bf16 softmax weights, bf16 output) is relative to the values
    # it weighs: 5e-3 * 1.77 = 8.85e-3, rounded up
    "int4": dict(atol=9e-3, rtol=1e-2, norm=1e-2),
}


def same_bits(a: np.ndarray, b: np.ndarray) -> bool:
    """Bit-for-bit equality of two raw arrays (NaN payloads and -0 included)."""
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    if a.dtype.kind == "f":
        view = {2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize]
        return np.array_equal(a.view(view), b.view(view))
    return np.array_equal(a, b)


def widen(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare(got: np.ndarray, ref: np.ndarray, cache_dtype: str, label: str = "") -> dict:
    tol = TOL[cache_dtype]
    err = np.abs(got - ref)
    bound = tol["atol"] + tol["rtol"] * np.abs(ref)
    big = np.abs(ref) >= 1e-2
    row_err = err.reshape(-1, err.shape[-1]).max(axis=1)
    row_ref = np.abs(ref).reshape(-1, ref.shape[-1]).max(axis=1)
    stats = {
        "max_abs": float(err.max()) if err.size else 0.0,
        "max_rel": float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0,
        "norm": float((row_err / np.maximum(row_ref, 1e-30)).max()) if err.size else 0.0,
        # the smallest atol that, with this rtol, would still pass
        "atol_needed": float((err - tol["rtol"] * np.abs(ref)).max()) if err.size else 0.0,
    }
    print(f"[parity] {label} {cache_dtype} max_abs={stats['max_abs']:.3e} "
          f"max_rel={stats['max_rel']:.3e} norm={stats['norm']:.3e}", flush=True)
    record = os.environ.get("PA_PARITY_RECORD")
    if record:  # one JSON line per comparison, for the committed margin tables
        with open(record, "a") as f:
            f.write(json.dumps({"label": label, "cache": cache_dtype, "rows": int(
                err.size // max(err.shape[-1], 1)), **tol, **stats}) + "\n")
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    bad = ~(err <= bound)
    assert not bad.any(), f"{label}: {int(bad.sum())} elements out of tolerance, worst {err.max():.3e}"
    assert stats["norm"] <= tol["norm"], f"{label}: normalised error {stats['norm']:.3e}"
    return stats


def gpu_write(batch) -> None:
    pk.kv_cache_write(batch.k_new, batch.v_new, batch.k_pool, batch.v_pool,
                      torch.from_numpy(batch.slot_mapping).to(batch.k_pool.device),
                      batch.k_scale, batch.v_scale, cache_dtype=batch.workload.cache_dtype)


def oracle_write(batch, k_host, v_host):
    w = batch.workload
    return paged.write_tokens(k_host, v_host, host_view(batch.k_new), host_view(batch.v_new),
                              batch.slot_mapping, w.block_size, w.src_dtype, w.cache_dtype,
                              None if batch.k_scale is None else batch.k_scale.cpu().numpy(),
                              None if batch.v_scale is None else batch.v_scale.cpu().numpy())


def device_tables(batch):
    dev = batch.k_pool.device
    return (torch.from_numpy(batch.block_tables).to(dev),
            torch.from_numpy(batch.context_lens).to(dev))


def gpu_decode(batch, partition_size=None, out=None):
    bt, cl = device_tables(batch)
    return pk.decode(batch.q, batch.k_pool, batch.v_pool, bt, cl, batch.max_context_len,
                     batch.scale, batch.k_scale, batch.v_scale, partition_size, out=out,
                     cache_dtype=batch.workload.cache_dtype)


def oracle_decode_host(batch, k_host: np.ndarray, v_host: np.ndarray, seqs) -> np.ndarray:
    """Oracle output of the listed sequences from host pools the oracle
    itself produced (e.g. by its own append).  Returns [len(seqs), Hq, D]."""
    w = batch.workload
    seqs = list(seqs)
    used = sorted({int(x) for b in seqs for x in batch.block_tables[b] if x >= 0})
    new_id = np.full(batch.num_blocks, -1, dtype=np.int64)
    new_id[used] = np.arange(len(used))
    tables = batch.block_tables[seqs].astype(np.int64)
    tables = np.where(tables >= 0, new_id[np.maximum(tables, 0)], -1).astype(np.int32)
    ks = None if batch.k_scale is None else batch.k_scale.cpu().numpy()
    vs = None if batch.v_scale is None else batch.v_scale.cpu().numpy()
    q_host, k_used, v_used = host_view(batch.q)[seqs], k_host[used], v_host[used]
    lens = batch.context_lens[seqs]
    if int(lens.sum()) < (1 << 20):
        return paged.decode(q_host, k_used, v_used, tables, lens, w.block_size, batch.scale,
                            w.q_dtype, w.cache_dtype, ks, vs)
    # long contexts: sequence by sequence, with a progress line each (the
    # oracle takes seconds per 131K-token sequence)
    out = np.zeros(q_host.shape, dtype=np.float64)
    for i in range(len(seqs)):
        out[i] = paged.decode(q_host[i:i + 1], k_used, v_used, tables[i:i + 1], lens[i:i + 1],
                              w.block_size, batch.scale, w.q_dtype, w.cache_dtype, ks, vs)[0]
        print(f"[oracle] sequence {i + 1}/{len(seqs)} ({int(lens[i])} tokens) decoded", flush=True)
    return out


def write_and_reference(batch):
    """Host copies of the pools, the oracle's append on them, then the GPU
    append on the device pools.  Returns the oracle's pools."""
    k_host, v_host = host_view(batch.k_pool), host_view(batch.v_pool)
    k_ref, v_ref = oracle_write(batch, k_host, v_host)
    del k_host, v_host
    gpu_write(batch)
    torch.cuda.synchronize()
    return k_ref, v_ref


def oracle_decode_seqs(batch, seqs) -> np.ndarray:
    """Oracle output of the listed sequences, from a host copy of only the
    blocks they use.  Returns [len(seqs), Hq, D]."""
    w = batch.workload
    sub = extract_sequences(batch, seqs)
    return paged.decode(sub["q"], sub["k_pool"], sub["v_pool"], sub["block_tables"],
                        sub["context_lens"], w.block_size, batch.scale, w.q_dtype, w.cache_dtype,
                        sub["k_scale"], sub["v_scale"])
