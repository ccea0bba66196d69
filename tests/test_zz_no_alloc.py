"""pa_decode_noalloc on the GPU, through the C ABI: the decode step for
callers that cannot allocate device memory.  Its output and pools must
equal, bit for bit, those of the existing entry point it varies --
pa_decode_append (or pa_decode) with the balanced split and a caller's
workspace, then pa_decode_reduce -- on two calls in a row, the second with
a smaller batch (the library's scratch array still holds the first call's
states), and match the oracle's append and decode within the stated
tolerance."""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_253_amd as pk
from workloads import WORKLOADS, host_view, make_batch

from .parity import compare, device_tables, oracle_decode_host, oracle_write, same_bits, widen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _workload(cache, group):
    base = WORKLOADS[5] if cache.startswith("fp8") else WORKLOADS[2]
    q = "f32" if cache == "f32" else "bf16"
    return dataclasses.replace(base, num_q_heads=8 * group, num_kv_heads=8, pool="exact",
                               cache_dtype=cache, q_dtype=q, name=f"noalloc-{cache}-g{group}")


def _one_call_pair(w, lens, seed, append):
    """(workspace entry point, no-alloc entry point) from the same start."""
    print(f"[noalloc] {w.name} seqs={len(lens)} append={append} seed={seed}", flush=True)
    batch = make_batch(w, seed=seed, device=DEV, lens=np.asarray(lens), poison=append)
    k0, v0 = host_view(batch.k_pool), host_view(batch.v_pool)
    ka, va = batch.k_pool.clone(), batch.v_pool.clone()
    bt, cl = device_tables(batch)
    rows = dict(k_new=batch.k_new, v_new=batch.v_new) if append else {}
    ref = pk.decode(batch.q, ka, va, bt, cl, batch.max_context_len, batch.scale, batch.k_scale,
                    batch.v_scale, pk.PARTITION_AUTO, cache_dtype=w.cache_dtype, **rows)
    got = pk.decode_noalloc(batch.q, batch.k_pool, batch.v_pool, bt, cl, batch.max_context_len,
                            batch.scale, batch.k_scale, batch.v_scale,
                            cache_dtype=w.cache_dtype, **rows)
    torch.cuda.synchronize()
    assert same_bits(host_view(got), host_view(ref)), f"{w.name}: out differs"
    assert same_bits(host_view(batch.k_pool), host_view(ka)), f"{w.name}: K pool differs"
    assert same_bits(host_view(batch.v_pool), host_view(va)), f"{w.name}: V pool differs"
    k_ref, v_ref = oracle_write(batch, k0, v0) if append else (k0, v0)
    seqs = list(range(len(lens)))
    compare(widen(got), oracle_decode_host(batch, k_ref, v_ref, seqs), w.cache_dtype,
            f"no-alloc {w.name}")


@pytest.mark.parametrize("cache,group,append", [
    ("bf16", 4, True),       # the decode kernel appends (matrix cores)
    ("bf16", 1, False),      # vector-unit kernels, no append
    ("fp8_e4m3", 4, True),   # append launch, then the decode
    ("f32", 2, True),        # float32 cache
    ("int4", 8, True),       # INT4 cache
])
def test_noalloc_equals_the_workspace_call_twice(cache, group, append):
    w = _workload(cache, group)
    rng = np.random.default_rng(77)
    big = rng.integers(512, 4097, size=48)
    small = np.array([0, 1, 17, 33, 250, 5])
    _one_call_pair(w, big, 101, append)
    _one_call_pair(w, small, 102, append)


def test_noalloc_rejects_a_half_given_append():
    w = _workload("bf16", 4)
    batch = make_batch(w, seed=3, device=DEV, lens=np.array([40, 70]))
    bt, cl = device_tables(batch)
    lib = pk.load()
    out = torch.empty_like(batch.q)
    st = lib.pa_decode_noalloc(pk._ptr(out), pk._ptr(batch.q), pk._ptr(batch.k_new), None,
                               pk._ptr(batch.k_pool), pk._ptr(batch.v_pool), pk._ptr(bt),
                               bt.shape[1], pk._ptr(cl), batch.max_context_len, 2,
                               w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                               batch.num_blocks, batch.scale, pk.PA_BF16, pk.PA_BF16,
                               pk.PA_BF16, None, None, None)
    assert st == 1  # PA_ERR_INVALID_ARG, nothing launched
