"""The balanced split merged inside the decode launch (PA_PARTITION_AUTO_MERGED)
on the GPU.

Its cut runs are merged by the wavefront that finishes a run's last piece,
with the merge routine the separate merge launch uses, so the output must be
bit for bit that of PA_PARTITION_AUTO followed by pa_decode_reduce, for every
cache kind, shape and kernel family, for runs cut into 2..4 pieces (the
merge's fast path), 5..64 and more than 64 pieces, over repeated calls on
one workspace (the counters must come back to zero), and for pa_decode as
well as pa_decode_append (whose append launch clears the counters).  The
full-size workloads are checked against the oracle in test_gpu_parity.py."""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_253_amd as pk
from workloads import WORKLOADS, host_view, make_batch

from .parity import compare, device_tables, gpu_write, oracle_decode_host, same_bits, widen, \
    write_and_reference

pytestmark = pytest.mark.gpu
DEV = "cuda"
AUTO, MERGED = pk.PARTITION_AUTO, pk.PARTITION_AUTO_MERGED

EDGE_LENS = [0, 1, 2, 15, 16, 17, 31, 32, 33, 64, 65, 100, 513, 1025, 4000, 3]
LONG_LENS = [30000, 1, 20000, 999]  # runs over many slices: > 64 pieces


def _batch(cache, head_dim, block, hq, hkv, lens, seed=11):
    base = WORKLOADS[2] if cache in ("bf16", "int4") else (
        WORKLOADS[5] if cache.startswith("fp8") else WORKLOADS[1])
    kw = dict(num_q_heads=hq, num_kv_heads=hkv, head_dim=head_dim, block_size=block,
              pool="exact", cache_dtype=cache)
    if cache == "int4":
        kw["q_dtype"] = "bf16"
    w = dataclasses.replace(base, **kw)
    return make_batch(w, seed=seed, device=DEV, lens=np.asarray(lens), poison=True)


def _decode(batch, p, workspace=None, append=False):
    bt, cl = device_tables(batch)
    kw = dict(scale=batch.scale, k_scale=batch.k_scale, v_scale=batch.v_scale,
              partition_size=p, workspace=workspace, cache_dtype=batch.workload.cache_dtype)
    if append:
        return pk.decode_append(batch.q, batch.k_new, batch.v_new, batch.k_pool, batch.v_pool,
                                bt, cl, batch.max_context_len, **kw)
    return pk.decode(batch.q, batch.k_pool, batch.v_pool, bt, cl, batch.max_context_len, **kw)


def _bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    return same_bits(host_view(a), host_view(b))


@pytest.mark.parametrize("cache", ["bf16", "fp8_e4m3", "fp8_e5m2", "int4"])
@pytest.mark.parametrize("head_dim,block", [(128, 16), (128, 32), (64, 16)])
@pytest.mark.parametrize("group", [2, 4, 8, 16])
def test_merged_equals_separate_merge(cache, head_dim, block, group):
    batch = _batch(cache, head_dim, block, 2 * group, 2, EDGE_LENS)
    print(f"[merged] {cache} d={head_dim} B={block} G={group}", flush=True)
    gpu_write(batch)
    ref = _decode(batch, AUTO).clone()
    got = _decode(batch, MERGED)
    torch.cuda.synchronize()
    assert _bits_equal(got, ref), f"{cache} d={head_dim} B={block} G={group}"


@pytest.mark.parametrize("cache,group,head_dim", [("f32", 1, 64), ("f32", 2, 128), ("f32", 8, 64),
                                                  ("bf16", 1, 128)])
def test_merged_vector_unit_paths(cache, group, head_dim):
    """f32 caches and G = 1 bf16 run the vector-unit kernel."""
    batch = _batch(cache, head_dim, 16, 2 * group, 2, EDGE_LENS)
    print(f"[merged] vector path {cache} G={group} d={head_dim}", flush=True)
    gpu_write(batch)
    ref = _decode(batch, AUTO).clone()
    got = _decode(batch, MERGED)
    torch.cuda.synchronize()
    assert _bits_equal(got, ref)


@pytest.mark.parametrize("cache,group", [("bf16", 4), ("bf16", 8), ("fp8_e4m3", 4), ("int4", 4),
                                         ("f32", 1), ("bf16", 1)])
def test_merged_runs_over_many_slices(cache, group):
    """Runs of 5..64 and of more than 64 pieces (the merge's general paths),
    and the oracle on every sequence."""
    head_dim = 64 if cache == "f32" else 128
    batch = _batch(cache, head_dim, 16, 2 * group, 2, LONG_LENS)
    print(f"[merged] long runs {cache} G={group}", flush=True)
    k_ref, v_ref = write_and_reference(batch)
    ref = _decode(batch, AUTO).clone()
    got = _decode(batch, MERGED)
    torch.cuda.synchronize()
    assert _bits_equal(got, ref)
    if cache != "int4":  # the INT4 oracle comparison is in test_gpu_int4.py
        want = oracle_decode_host(batch, k_ref, v_ref, range(len(LONG_LENS)))
        compare(widen(got), want, cache, f"merged long runs {cache}")


def test_counters_return_to_zero_over_repeated_calls():
    """pa_decode on one workspace, several calls in a row -- the same batch
    twice, then a smaller one, then one with many cut runs -- each equal to
    the separate merge; the counters are zero after every call."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(3)
    batches = [_batch("bf16", 128, 16, 8, 2, EDGE_LENS), None,
               _batch("bf16", 128, 16, 8, 2, [5, 40, 3]),
               _batch("bf16", 128, 16, 8, 2, rng.integers(1, 3000, size=40), seed=4)]
    batches[1] = batches[0]
    ws = pk.new_workspace(40, 8, 2, 128, 4000, MERGED, DEV)
    off = 256 + (16 * 8 * cus + 255) // 256 * 256
    counters = ws[off:off + 4 * 8 * cus].view(torch.int32)
    for i, batch in enumerate(batches):
        if i != 1:
            gpu_write(batch)
        ref = _decode(batch, AUTO).clone()
        got = _decode(batch, MERGED, workspace=ws)
        torch.cuda.synchronize()
        print(f"[merged] repeated call {i}", flush=True)
        assert _bits_equal(got, ref), f"call {i}"
        assert int(counters.abs().sum()) == 0, f"counters left nonzero after call {i}"


@pytest.mark.parametrize("cache", ["bf16", "fp8_e4m3", "int4"])
def test_decode_append_merged_clears_planted_counters(cache):
    """pa_decode_append clears the counters in its append launch: counters
    planted nonzero do not change the output, which equals the separate
    append, decode and merge, and the pools equal the separate append's."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    block = 32 if cache.startswith("fp8") else 16
    batch = _batch(cache, 128, block, 8, 2, EDGE_LENS)
    k2, v2 = batch.k_pool.clone(), batch.v_pool.clone()
    gpu_write(batch)
    ref = _decode(batch, AUTO).clone()
    ws = pk.new_workspace(len(EDGE_LENS), 8, 2, 128, batch.max_context_len, MERGED, DEV)
    off = 256 + (16 * 8 * cus + 255) // 256 * 256
    ws[off:off + 4 * 8 * cus].view(torch.int32).fill_(5)
    one = batch.replace(k_pool=k2, v_pool=v2)
    got = _decode(one, MERGED, workspace=ws, append=True)
    torch.cuda.synchronize()
    assert _bits_equal(k2, batch.k_pool) and _bits_equal(v2, batch.v_pool)
    assert _bits_equal(got, ref)
    assert int(ws[off:off + 4 * 8 * cus].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("idx", [2, 3])
def test_full_size_step_merged_equals_separate(idx):
    """The bench's step (pa_decode_append, merged) on the full 8B- and
    70B-shaped batches: bit for bit the separate append, decode and merge."""
    w = WORKLOADS[idx]
    print(f"[merged] full-size step, workload {idx} {w.name}", flush=True)
    batch = make_batch(w, device=DEV)
    k2, v2 = batch.k_pool.clone(), batch.v_pool.clone()
    gpu_write(batch)
    ref = _decode(batch, AUTO).clone()
    got = _decode(batch.replace(k_pool=k2, v_pool=v2), MERGED, append=True)
    torch.cuda.synchronize()
    assert _bits_equal(got, ref)
    assert torch.equal(k2.view(torch.int16), batch.k_pool.view(torch.int16))
    assert torch.equal(v2.view(torch.int16), batch.v_pool.view(torch.int16))


def test_many_launches_on_one_workspace_identical():
    """Twenty merged launches back to back on the full 8B-shaped batch (about
    500 cut runs, pieces on every XCD), one workspace: every output equals
    the separate merge's bit for bit, so no merge read a piece's state before
    it was visible."""
    w = WORKLOADS[2]
    batch = make_batch(w, device=DEV)
    ref = _decode(batch, AUTO).clone()
    s, hq, d = batch.q.shape
    ws = pk.new_workspace(s, hq, w.num_kv_heads, d, batch.max_context_len, MERGED, DEV)
    bt, cl = device_tables(batch)
    outs = [torch.empty_like(batch.q) for _ in range(20)]
    for o in outs:
        pk.decode(batch.q, batch.k_pool, batch.v_pool, bt, cl, batch.max_context_len, batch.scale,
                  partition_size=MERGED, out=o, workspace=ws)
    torch.cuda.synchronize()
    bad = [i for i, o in enumerate(outs) if not _bits_equal(o, ref)]
    assert not bad, f"launches {bad} differ from the separate merge"
