"""HIP library against the oracle on the GPU (through the C ABI).

Writes must match bit for bit over the whole pool; attention outputs must
meet the stated tolerance; layout invariances (block permutation, paged vs
contiguous, shared vs copied prefix), NaN-poisoned unused slots and repeated
runs must give identical bits.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_253_amd as pk
from oracle import paged
from workloads import (WORKLOADS, contiguous_layout, host_view, make_batch, permute_blocks,
                       unshare)

from .parity import (compare, device_tables, gpu_decode, gpu_write, oracle_decode_host,
                     oracle_decode_seqs, oracle_write, same_bits, widen, write_and_reference)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _sync():
    torch.cuda.synchronize()


def bits(t: torch.Tensor) -> torch.Tensor:
    """Integer view for bit-for-bit comparison (NaN-safe, sign of zero kept)."""
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------

# sequences the oracle checks one by one at full size: all of them (the
# 131K-token batch takes the oracle about a minute)
SAMPLE = {1: None, 2: None, 3: None, 4: None, 5: None}


def _sample(batch, spec):
    s = len(batch.context_lens)
    if spec is None:
        return list(range(s))
    if spec == "spread":
        order = np.argsort(batch.context_lens)
        pick = {int(order[0]), int(order[-1]), int(order[len(order) // 2])}
        pick |= set(np.random.default_rng(7).choice(s, 13, replace=False).tolist())
        return sorted(pick)
    return list(spec)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_workload_write_and_decode(idx):
    w = WORKLOADS[idx]
    print(f"[parity] workload {idx} {w.name}", flush=True)
    batch = make_batch(w, device=DEV, poison=True)
    k_ref, v_ref = write_and_reference(batch)
    # the append is bit-exact over the whole pool (untouched slots included)
    assert same_bits(host_view(batch.k_pool), k_ref), "K pool differs after the append"
    assert same_bits(host_view(batch.v_pool), v_ref), "V pool differs after the append"

    seqs = _sample(batch, SAMPLE[idx])
    ref = oracle_decode_host(batch, k_ref, v_ref, seqs)
    del k_ref, v_ref
    # -2: the balanced split merged inside the decode launch (the bench's step)
    splits = [w.partition_size, -1, -2] if w.partition_size else [-1, -2, 0, 512]
    for p in splits:
        out = gpu_decode(batch, p)
        _sync()
        compare(widen(out)[seqs], ref, w.cache_dtype, f"workload {idx} P={p}")


# ---------------------------------------------------------------------------
# layout invariances: identical bits
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("idx,p", [(2, 512), (2, 0), (2, -1), (1, 0), (1, -1), (4, 256), (4, -1)])
def test_block_permutation_and_contiguous_layout_bit_identical(idx, p):
    w = WORKLOADS[idx]
    batch = make_batch(w, device=DEV, num_seqs=8 if idx != 1 else None)
    base = gpu_decode(batch, p).clone()
    perm = np.random.default_rng(3).permutation(batch.num_blocks)
    moved = gpu_decode(permute_blocks(batch, perm), p)
    _sync()
    assert torch.equal(bits(base), bits(moved))
    if idx != 4:
        cont = gpu_decode(contiguous_layout(batch), p)
        _sync()
        assert torch.equal(bits(base), bits(cont))


@pytest.mark.parametrize("p", [0, 512, -1])
def test_shared_prefix_equals_private_copies(p):
    w = WORKLOADS[4]
    batch = make_batch(w, device=DEV)
    assert (batch.ref_counts[batch.block_tables[0, :128]] == 32).all()
    shared = gpu_decode(batch, p).clone()
    copied = gpu_decode(unshare(batch), p)
    _sync()
    assert torch.equal(bits(shared), bits(copied))


@pytest.mark.parametrize("idx", [2, 5])
def test_poisoned_unused_slots_do_not_change_bits(idx):
    w = WORKLOADS[idx]
    lens = None if idx == 2 else np.array([1000, 777])
    kw = dict(device=DEV, num_seqs=6 if idx == 2 else None, lens=lens)
    clean = make_batch(w, poison=False, **kw)
    dirty = make_batch(w, poison=True, **kw)
    gpu_write(clean)
    gpu_write(dirty)
    p = w.partition_size or 512
    a = gpu_decode(clean, p).clone()
    b = gpu_decode(dirty, p)
    _sync()
    assert torch.isfinite(b.float()).all()
    assert torch.equal(bits(a), bits(b))


@pytest.mark.parametrize("p", [512, -1])
def test_repeated_runs_identical(p):
    batch = make_batch(WORKLOADS[3], device=DEV, num_seqs=32)
    a = gpu_decode(batch, p).clone()
    b = gpu_decode(batch, p)
    _sync()
    assert torch.equal(bits(a), bits(b))


@pytest.mark.parametrize("cache,group", [("bf16", 4), ("bf16", 1), ("fp8_e4m3", 4), ("f32", 2),
                                         ("fp8_e5m2", 4), ("fp8_e5m2", 1)])
def test_balanced_split_cuts_and_empty_runs(cache, group):
    """Many short and a few long contexts with empty ones between them: the
    balanced slices cut long runs several times and start inside runs."""
    rng = np.random.default_rng(21)
    lens = rng.integers(1, 90, size=40)
    lens[[3, 17]] = 0
    lens[[5, 30]] = [5000, 2500]
    batch = _custom(cache, 128 if cache != "f32" else 64, 32 if cache.startswith("fp8") else 16,
                    2 * group, 2, lens)
    k_ref, v_ref = write_and_reference(batch)
    ref = oracle_decode_host(batch, k_ref, v_ref, range(len(lens)))
    out = gpu_decode(batch, -1)
    _sync()
    compare(widen(out), ref, cache, f"balanced {cache} G={group}")


@pytest.mark.parametrize("cache", ["bf16", "fp8_e4m3"])
def test_balanced_split_run_over_many_slices(cache):
    """One KV head and a 20,000-token context next to short ones: the long
    run is cut into well over 64 pieces (a slice is at least 4 steps), which
    the merge takes through its general loop rather than the one-batch
    path."""
    lens = np.array([20000, 37, 1, 300])
    batch = _custom(cache, 128, 32 if cache.startswith("fp8") else 16, 4, 1, lens)
    k_ref, v_ref = write_and_reference(batch)
    ref = oracle_decode_host(batch, k_ref, v_ref, range(len(lens)))
    out = gpu_decode(batch, -1)
    _sync()
    compare(widen(out), ref, cache, f"balanced, long run, {cache}")


def test_balanced_merge_records_written_every_launch():
    """The merge of the balanced split reads one record per slice that the
    decode writes on every launch, empty slices included.  Records planted in
    the workspace (each naming a real run as cut across two slices) must not
    reach the output: a long batch, then a short one whose slices are mostly
    empty, on the same workspace, both match the oracle."""
    rng = np.random.default_rng(5)
    long_lens = rng.integers(1, 90, size=40)
    long_lens[[5, 30]] = [5000, 2500]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ws = None
    for lens in (long_lens, np.array([3, 40, 0, 7])):
        batch = _custom("bf16", 128, 16, 8, 2, lens)
        k_ref, v_ref = write_and_reference(batch)
        ref = oracle_decode_host(batch, k_ref, v_ref, range(len(lens)))
        if ws is None:
            ws = pk.new_workspace(len(long_lens), 8, 2, 128, int(long_lens.max()), -1, DEV)
        recs = ws[256:256 + 16 * 8 * cus].view(torch.int32).view(-1, 4)
        recs.copy_(torch.tensor([0, 1, 2, 0], dtype=torch.int32, device=DEV).expand_as(recs))
        bt, cl = device_tables(batch)
        out = pk.decode(batch.q, batch.k_pool, batch.v_pool, bt, cl, batch.max_context_len,
                        batch.scale, batch.k_scale, batch.v_scale, -1, workspace=ws,
                        cache_dtype=batch.workload.cache_dtype)
        _sync()
        compare(widen(out), ref, "bf16", f"planted records, {len(lens)} seqs")


# ---------------------------------------------------------------------------
# shapes, groups, paths and edge cases on small batches
# ---------------------------------------------------------------------------

def _custom(cache, head_dim, block, hq, hkv, lens, seed=11, poison=True):
    base = WORKLOADS[2] if cache == "bf16" else (WORKLOADS[5] if cache.startswith("fp8") else WORKLOADS[1])
    w = dataclasses.replace(base, num_q_heads=hq, num_kv_heads=hkv, head_dim=head_dim,
                            block_size=block, pool="exact", cache_dtype=base.cache_dtype
                            if not cache.startswith("fp8") else cache)
    return make_batch(w, seed=seed, device=DEV, lens=np.asarray(lens), poison=poison)


EDGE_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 511, 512, 513, 1025]


@pytest.mark.parametrize("cache,head_dim,block", [
    ("bf16", 128, 16), ("bf16", 128, 32), ("bf16", 64, 16), ("bf16", 64, 32),
    ("fp8_e4m3", 128, 32), ("fp8_e4m3", 128, 16), ("fp8_e4m3", 64, 32),
    ("fp8_e5m2", 128, 32), ("fp8_e5m2", 64, 16),
    ("f32", 64, 16), ("f32", 128, 32),
])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_shapes_and_groups(cache, head_dim, block, group):
    hkv = 2
    batch = _custom(cache, head_dim, block, hkv * group, hkv, EDGE_LENS)
    k_ref, v_ref = write_and_reference(batch)
    seqs = list(range(len(EDGE_LENS)))
    ref = oracle_decode_host(batch, k_ref, v_ref, seqs)
    for p in (0, 32, 64, 512, -1):
        out = gpu_decode(batch, p)
        _sync()
        compare(widen(out), ref, cache, f"{cache} d={head_dim} B={block} G={group} P={p}")


@pytest.mark.parametrize("group", [3, 5, 16])
def test_matrix_core_path_odd_groups(group):
    batch = _custom("bf16", 128, 16, group * 2, 2, [1, 40, 300, 777])
    k_ref, v_ref = write_and_reference(batch)
    ref = oracle_decode_host(batch, k_ref, v_ref, range(4))
    for p in (0, 64, -1):
        out = gpu_decode(batch, p)
        _sync()
        compare(widen(out), ref, "bf16", f"G={group} P={p}")


@pytest.mark.parametrize("cache", ["bf16", "fp8_e4m3", "fp8_e5m2"])
@pytest.mark.parametrize("group", [2, 4, 8])
def test_forced_paths_agree_with_oracle(monkeypatch, cache, group):
    batch = _custom(cache, 128, 16 if cache == "bf16" else 32, 2 * group, 2, [5, 333, 1500])
    k_ref, v_ref = write_and_reference(batch)
    ref = oracle_decode_host(batch, k_ref, v_ref, range(3))
    for path in ("valu", "mfma"):
        monkeypatch.setenv("PA_FORCE_PATH", path)
        out = gpu_decode(batch, 512)
        _sync()
        compare(widen(out), ref, cache, f"forced {path} G={group}")


@pytest.mark.parametrize("cache,group", [("bf16", 4), ("bf16", 1), ("f32", 1), ("fp8_e4m3", 4)])
def test_single_token_returns_that_value_row(cache, group):
    """L = 1: the weight is exactly 1, so the output is the V row itself
    (bf16/f32 exactly; FP8 as code * scale rounded once to bf16)."""
    batch = _custom(cache, 128, 16 if cache != "fp8_e4m3" else 32, 2 * group, 2, [1, 1, 1])
    gpu_write(batch)
    out = gpu_decode(batch, 0)
    _sync()
    vrow = batch.v_new.float().cpu().numpy()  # [S, Hkv, D]
    got = widen(out)
    for b in range(3):
        for hq in range(2 * group):
            if cache == "fp8_e4m3":
                # the oracle's code of the new row; code * scale rounded to float32,
                # then to bf16: the kernel's two roundings
                vs = np.float32(batch.v_scale[hq // group].item())
                code = paged.codecs.e4m3_encode(vrow[b, hq // group].astype(np.float32) / vs)
                prod = (paged.codecs.e4m3_to_f64(code).astype(np.float32)
                        * np.float32(batch.v_scale[hq // group].item()))
                want = torch.from_numpy(prod).to(torch.bfloat16).double().numpy()
            else:
                want = vrow[b, hq // group]
            assert np.array_equal(got[b, hq], want), (b, hq)


@pytest.mark.parametrize("p", [0, 64, -1])
def test_empty_context_gives_zeros(p):
    batch = _custom("bf16", 128, 16, 8, 2, [0, 5, 0], poison=False)
    out = torch.full_like(batch.q, 7.0)
    gpu_decode(batch, p, out=out)
    _sync()
    got = widen(out)
    assert (got[0] == 0).all() and (got[2] == 0).all()
    ref = oracle_decode_seqs(batch, [1])
    compare(got[1:2], ref, "bf16", "L=0 neighbours")


# ---------------------------------------------------------------------------
# the split contract: partitions and their merge
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cache", ["bf16", "fp8_e4m3"])
def test_partition_states_match_oracle(cache):
    p = 128
    batch = _custom(cache, 128, 16 if cache == "bf16" else 32, 8, 2, [1, 130, 700, 1024])
    k_ref, v_ref = write_and_reference(batch)
    bt, cl = device_tables(batch)
    ws = pk.decode_partitions(batch.q, batch.k_pool, batch.v_pool, bt, cl, batch.max_context_len,
                              p, batch.scale, batch.k_scale, batch.v_scale)
    _sync()
    po, pm, ps = (widen(x) for x in pk.workspace_views(ws, 4, 8, 128, batch.max_context_len, p))
    w = batch.workload
    m, l, o = paged.decode_partials(host_view(batch.q), k_ref, v_ref, batch.block_tables,
                                    batch.context_lens, w.block_size, batch.scale, w.q_dtype,
                                    w.cache_dtype, p,
                                    None if batch.k_scale is None else batch.k_scale.cpu().numpy(),
                                    None if batch.v_scale is None else batch.v_scale.cpu().numpy())
    have = ~np.isnan(m)
    np.testing.assert_allclose(pm[have], m[have], rtol=1e-4, atol=1e-4)
    np.testing.assert_allclose(ps[have], l[have], rtol=1e-3, atol=1e-4)
    compare(po[have], o[have], cache, "partition outputs")


def test_reduce_of_oracle_partitions():
    """pa_decode_reduce alone, fed partition states the oracle computed."""
    p = 64
    batch = _custom("bf16", 128, 16, 8, 2, [1, 64, 65, 300, 1000], poison=False)
    w = batch.workload
    m, l, o = paged.decode_partials(host_view(batch.q), host_view(batch.k_pool),
                                      host_view(batch.v_pool), batch.block_tables,
                                      batch.context_lens, w.block_size, batch.scale, "bf16",
                                      "bf16", p)
    n = pk.workspace_size(5, 8, 2, 128, batch.max_context_len, p)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    po, pm, ps = pk.workspace_views(ws, 5, 8, 128, batch.max_context_len, p)
    po.copy_(torch.from_numpy(np.nan_to_num(o)).float())
    pm.copy_(torch.from_numpy(np.nan_to_num(m)).float())
    ps.copy_(torch.from_numpy(np.nan_to_num(l)).float())
    _, cl = device_tables(batch)
    out = torch.empty_like(batch.q)
    pk.decode_reduce(out, ws, cl, batch.max_context_len, p)
    _sync()
    ref = np.zeros_like(o[:, :, 0])
    for b in range(5):
        k = -(-int(batch.context_lens[b]) // p)
        for hq in range(8):
            ref[b, hq] = paged.merge(m[b, hq, :k], l[b, hq, :k], o[b, hq, :k])
    compare(widen(out), ref, "bf16", "reduce of oracle partitions")


# ---------------------------------------------------------------------------
# the append
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cache,src", [("fp8_e4m3", "bf16"), ("fp8_e5m2", "bf16"), ("bf16", "bf16"),
                                       ("f32", "f32")])
def test_append_bit_exact_with_padding_and_out_of_range_slots(cache, src):
    batch = _custom(cache, 128, 32 if cache.startswith("fp8") else 16, 8, 2, [40, 90, 3, 200])
    slots = batch.slot_mapping.copy()
    slots[1] = -1                                  # padding token
    slots[2] = batch.num_blocks * batch.workload.block_size + 5  # beyond the pool: skipped
    batch = batch.replace(slot_mapping=slots)
    k_host, v_host = host_view(batch.k_pool), host_view(batch.v_pool)
    gpu_write(batch)
    _sync()
    ok = slots.copy()
    ok[2] = -1
    k_ref, v_ref = oracle_write(batch.replace(slot_mapping=ok), k_host, v_host)
    assert same_bits(host_view(batch.k_pool), k_ref)
    assert same_bits(host_view(batch.v_pool), v_ref)


@pytest.mark.parametrize("fmt", ["fp8_e4m3", "fp8_e5m2"])
def test_fp8_append_rounding_matches_oracle_on_many_values(fmt):
    """The FP8 encoders on the GPU against the oracle's, over a wide spread
    of magnitudes (subnormals, ties, saturation, NaN)."""
    hkv, d, bsz, n = 4, 128, 32, 256
    nb = n
    rng = np.random.default_rng(5)
    big = 100 if fmt == "fp8_e4m3" else 20000
    tiny = 1e-3 if fmt == "fp8_e4m3" else 1e-5
    vals = np.concatenate([rng.standard_normal(n * hkv * d // 2) * big,
                           rng.standard_normal(n * hkv * d // 2) * tiny]).astype(np.float32)
    vals[:10] = [0.0, -0.0, 448.0, 500.0, -1e9, np.nan, 2.0 ** -10, 57344.0, 61440.0, 2.0 ** -17]
    kn = torch.from_numpy(vals.reshape(n, hkv, d)).to(torch.bfloat16)
    vn = torch.from_numpy(vals[::-1].copy().reshape(n, hkv, d)).to(torch.bfloat16)
    ks = torch.tensor([0.5, 1.0, 2.0, 0.01], dtype=torch.float32)
    vs = torch.tensor([1.0, 0.25, 3.0, 0.7], dtype=torch.float32)
    k_pool = torch.zeros(nb, hkv, d // 16, bsz, 16, dtype=torch.uint8)
    v_pool = torch.zeros(nb, hkv, d, bsz, dtype=torch.uint8)
    slots = np.arange(n, dtype=np.int64) * bsz + 7
    k_ref, v_ref = paged.write_tokens(k_pool.numpy(), v_pool.numpy(), host_view(kn), host_view(vn),
                                      slots, bsz, "bf16", fmt, ks.numpy(), vs.numpy())
    kd, vd = k_pool.to(DEV), v_pool.to(DEV)
    pk.kv_cache_write(kn.to(DEV), vn.to(DEV), kd, vd, torch.from_numpy(slots).to(DEV),
                      ks.to(DEV), vs.to(DEV), cache_dtype=fmt)
    _sync()
    assert np.array_equal(kd.cpu().numpy(), k_ref)
    assert np.array_equal(vd.cpu().numpy(), v_ref)


def test_balanced_workspace_size_follows_documented_layout():
    """PA_PARTITION_AUTO (and _MERGED, same layout): a header of 256 bytes,
    a 16-byte merge record and a 4-byte merge counter per possible slice,
    then R = 8 * CUs * 2 * G rows of partial state (the documented bound on
    the decode's wavefronts)."""
    def align(x):
        return (x + 255) // 256 * 256
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for s, hq, hkv, d in [(64, 32, 8, 128), (3, 16, 16, 64), (8, 64, 4, 128)]:
        rows = 8 * cus * 2 * (hq // hkv)
        want = (256 + align(16 * 8 * cus) + align(4 * 8 * cus) + align(rows * d * 4)
                + 2 * align(rows * 4))
        assert pk.workspace_size(s, hq, hkv, d, 4096, -1) == want
        assert pk.workspace_size(s, hq, hkv, d, 4096, -2) == want
