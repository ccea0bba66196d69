"""The oracle against what the pages and the mathematics fix (CPU only).

Every pin is a function of the implementation it checks, so the last
section can run the same pins against deliberately broken copies of the
oracle and show that each plausible mistake is caught.
"""

from __future__ import annotations

import dataclasses
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs, paged
from workloads import (WORKLOADS, contiguous_layout, host_view, make_batch,
                       permute_blocks, unshare)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _impl(**over):
    """The oracle's functions as a namespace, optionally with replacements."""
    ns = dict(slot_of=paged.slot_of, gather=paged.gather, copy_blocks=paged.copy_blocks,
              prefill_chunk=paged.prefill_chunk, swap_blocks=paged.swap_blocks,
              write_tokens=paged.write_tokens, attention=paged.attention,
              decode=paged.decode, partial=paged.partial, merge=paged.merge,
              e4m3_to_f64=codecs.e4m3_to_f64, e4m3_encode=codecs.e4m3_encode,
              e5m2_to_f64=codecs.e5m2_to_f64, e5m2_encode=codecs.e5m2_encode,
              int4_encode=codecs.int4_encode, unpack_octets=paged.unpack_octets,
              pack_octets=paged.pack_octets, int4_k_row=paged.int4_k_row,
              int4_v_row=paged.int4_v_row, int4_block_values=paged.int4_block_values)
    ns.update(over)
    return types.SimpleNamespace(**ns)


ORACLE = _impl()


def _host(batch):
    return dict(q=host_view(batch.q), k=host_view(batch.k_pool),
                v=host_view(batch.v_pool), kn=host_view(batch.k_new),
                vn=host_view(batch.v_new),
                ks=None if batch.k_scale is None else batch.k_scale.numpy(),
                vs=None if batch.v_scale is None else batch.v_scale.numpy())


def _decode_batch(impl, batch, k=None, v=None):
    h = _host(batch)
    w = batch.workload
    return impl.decode(h["q"], h["k"] if k is None else k, h["v"] if v is None else v,
                       batch.block_tables, batch.context_lens, w.block_size,
                       batch.scale, w.q_dtype, w.cache_dtype, h["ks"], h["vs"])


def _k_pool(nb, hkv, bsz, d, x, fill, dtype):
    """Empty chunked K pool [nb, Hkv, d/x, B, x]."""
    return np.full((nb, hkv, d // x, bsz, x), fill, dtype)


def _scatter_contiguous(k_c, v_c, block_size, table, k_pool, v_pool):
    """Place contiguous [L, Hkv, d] rows into pool tiles with explicit index
    arrays (the inverse of a gather, built without the oracle).  Element i
    of a K row sits in chunk i // x at lane i % x of its token."""
    length, _, d = k_c.shape
    x = k_pool.shape[4]
    t = np.arange(length)
    blk = np.asarray(table)[t // block_size]
    off = t % block_size
    for i in range(d):
        k_pool[blk, :, i // x, off, i % x] = k_c[:, :, i]
    for tt in range(length):  # V tiles are dimension-major
        v_pool[blk[tt], :, :, off[tt]] = v_c[tt]


# ==========================================================================
# pins (each takes an implementation namespace)
# ==========================================================================

def pin_golden_index(impl):
    table, bsz, rows = None, None, []
    with open(os.path.join(GOLDEN, "block_table_index.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            if line.startswith("block_size:"):
                bsz = int(line.split(":")[1])
            elif line.startswith("table:"):
                table = [int(x) for x in line.split(":")[1].split()]
            else:
                rows.append([int(x) for x in line.split()])
    assert table == [5, 0, 3] and bsz == 16 and len(rows) == 8
    for t, i, j, phys in rows:
        assert impl.slot_of(np.array(table), t, bsz) == (phys, j)
        assert table[i] == phys


def pin_gather_roundtrip(impl):
    rng = np.random.default_rng(1)
    bsz, hkv, d, nb = 4, 2, 6, 9
    length = 11
    table = rng.permutation(nb)[:3]
    k_c = rng.standard_normal((length, hkv, d)).astype(np.float32)
    v_c = rng.standard_normal((length, hkv, d)).astype(np.float32)
    k_pool = _k_pool(nb, hkv, bsz, d, 2, np.nan, np.float32)
    v_pool = np.full((nb, hkv, d, bsz), np.nan, np.float32)
    _scatter_contiguous(k_c, v_c, bsz, table, k_pool, v_pool)
    kg, vg = impl.gather(k_pool, v_pool, table, length, bsz)
    assert np.array_equal(kg, k_c) and np.array_equal(vg, v_c)


def pin_write_whole_pool(impl):
    """Whole-pool check of an append: every targeted slot holds the new row,
    every other slot is unchanged, padding tokens write nothing."""
    rng = np.random.default_rng(2)
    bsz, hkv, d, nb = 16, 3, 16, 7
    k_pool = rng.integers(0, 2**16, (nb, hkv, d // 8, bsz, 8)).astype(np.uint16)
    v_pool = rng.integers(0, 2**16, (nb, hkv, d, bsz)).astype(np.uint16)
    kn = rng.integers(0, 2**16, (5, hkv, d)).astype(np.uint16)
    vn = rng.integers(0, 2**16, (5, hkv, d)).astype(np.uint16)
    slots = np.array([3 * 16 + 5, -1, 0, 6 * 16 + 15, 2 * 16 + 9], np.int64)
    k2, v2 = impl.write_tokens(k_pool, v_pool, kn, vn, slots, bsz, "bf16", "bf16")
    kexp, vexp = k_pool.copy(), v_pool.copy()
    for n, where in enumerate([(3, 5), None, (0, 0), (6, 15), (2, 9)]):
        if where is None:
            continue
        blk, off = where
        kexp[blk, :, :, off, :] = kn[n].reshape(hkv, d // 8, 8)
        vexp[blk, :, :, off] = vn[n]
    assert np.array_equal(k2, kexp) and np.array_equal(v2, vexp)
    assert np.array_equal(k_pool[1], k2[1])  # input untouched


def pin_write_then_gather(impl):
    """Appending token L through its slot extends the gathered sequence by
    exactly that row (the engine's append, then the block-table read)."""
    w = WORKLOADS[1]
    batch = make_batch(w)
    h = _host(batch)
    for b in range(w.num_seqs):
        length = int(batch.context_lens[b])
        k_old, v_old = impl.gather(h["k"], h["v"], batch.block_tables[b],
                                   length - 1, w.block_size)
        k2, v2 = impl.write_tokens(h["k"], h["v"], h["kn"][b:b + 1], h["vn"][b:b + 1],
                                   batch.slot_mapping[b:b + 1], w.block_size,
                                   "f32", "f32")
        k_new, v_new = impl.gather(k2, v2, batch.block_tables[b], length, w.block_size)
        assert np.array_equal(k_new[:-1], k_old) and np.array_equal(v_new[:-1], v_old)
        assert np.array_equal(k_new[-1], h["kn"][b]) and np.array_equal(v_new[-1], h["vn"][b])


def pin_single_token(impl):
    """L = 1: softmax of one score is 1, the output is that V row exactly."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 16))
    k = rng.standard_normal((1, 2, 16))
    v = rng.standard_normal((1, 2, 16))
    out = impl.attention(q, k, v, 0.25)
    assert np.array_equal(out, v[0, np.arange(4) // 2])


def pin_two_tokens(impl):
    """L = 2: out = v0 + sigmoid(z1 - z0) (v1 - v0), z_t = scale * q.k_t."""
    rng = np.random.default_rng(4)
    d = 8
    q = rng.standard_normal((2, d))
    k = rng.standard_normal((2, 1, d))
    v = rng.standard_normal((2, 1, d))
    scale = 0.37
    out = impl.attention(q, k, v, scale)
    for hq in range(2):
        z = [scale * math.fsum(q[hq, i] * k[t, 0, i] for i in range(d)) for t in range(2)]
        sig = 1.0 / (1.0 + math.exp(-(z[1] - z[0])))
        want = v[0, 0] + sig * (v[1, 0] - v[0, 0])
        np.testing.assert_allclose(out[hq], want, rtol=1e-13, atol=1e-14)


def pin_identical_keys_mean(impl):
    """Identical keys (or q = 0) make every weight 1/L: out = mean of V."""
    rng = np.random.default_rng(5)
    length, d = 37, 16
    q = rng.standard_normal((3, d))
    krow = rng.standard_normal(d)
    k = np.tile(krow, (length, 1, 1))
    v = rng.standard_normal((length, 1, d))
    out = impl.attention(q, k, v, 1.3)
    mean = np.array([math.fsum(v[:, 0, i]) / length for i in range(d)])
    np.testing.assert_allclose(out, np.tile(mean, (3, 1)), rtol=1e-13, atol=1e-14)
    out0 = impl.attention(np.zeros((3, d)), rng.standard_normal((length, 1, d)), v, 1.0)
    np.testing.assert_allclose(out0, np.tile(mean, (3, 1)), rtol=1e-13, atol=1e-14)


def pin_saturation(impl):
    """One key aligned with q and scaled up dominates: out -> that V row."""
    rng = np.random.default_rng(6)
    d, length = 16, 20
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((length, 1, d)) * 0.01
    k[7, 0] = 200.0 * q[0] / np.linalg.norm(q[0])
    v = rng.standard_normal((length, 1, d))
    out = impl.attention(q, k, v, 1.0)
    np.testing.assert_allclose(out[0], v[7, 0], rtol=0, atol=1e-12)


def pin_gqa_equals_repeated_mha(impl):
    """Query head hq reads KV head hq // G: GQA equals MHA whose KV heads
    are each repeated G times (consecutive grouping)."""
    rng = np.random.default_rng(7)
    length, d, hkv, g = 9, 8, 3, 4
    q = rng.standard_normal((hkv * g, d))
    k = rng.standard_normal((length, hkv, d))
    v = rng.standard_normal((length, hkv, d))
    gqa = impl.attention(q, k, v, 0.5)
    mha = impl.attention(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), 0.5)
    assert np.array_equal(gqa, mha)
    # and each head against a single-head call on its own KV head
    for hq in range(hkv * g):
        one = impl.attention(q[hq:hq + 1], k[:, hq // g:hq // g + 1], v[:, hq // g:hq // g + 1], 0.5)
        assert np.array_equal(one[0], gqa[hq])


def pin_library_sdpa(impl):
    """Special case reducing to a library routine: torch's scaled dot-product
    attention in float64 on the CPU, KV heads repeated per group."""
    rng = np.random.default_rng(8)
    for length, hq, hkv, d in [(1, 4, 4, 8), (50, 8, 2, 16), (300, 6, 3, 32)]:
        q = rng.standard_normal((hq, d))
        k = rng.standard_normal((length, hkv, d))
        v = rng.standard_normal((length, hkv, d))
        scale = 1.0 / math.sqrt(d)
        out = impl.attention(q, k, v, scale)
        g = hq // hkv
        kt = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2)[None].contiguous()
        vt = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2)[None].contiguous()
        qt = torch.from_numpy(q)[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        np.testing.assert_allclose(out, ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)


def _brute_decode(q, k_pool, v_pool, tables, lens, bsz, scale, group):
    """Pure-Python loops: gather by the index map, then softmax and sum."""
    x = len(k_pool[0][0][0][0])
    out = []
    for b in range(len(lens)):
        rows = []
        for hq in range(len(q[b])):
            h = hq // group
            ks, vs = [], []
            for t in range(lens[b]):
                blk = tables[b][t // bsz]
                off = t % bsz
                ks.append([float(k_pool[blk][h][i // x][off][i % x]) for i in range(len(q[b][hq]))])
                vs.append([float(v_pool[blk][h][i][off]) for i in range(len(q[b][hq]))])
            z = [scale * sum(float(q[b][hq][i]) * kk[i] for i in range(len(kk))) for kk in ks]
            zmax = max(z)
            e = [math.exp(x - zmax) for x in z]
            tot = sum(e)
            rows.append([sum(e[t] * vs[t][i] for t in range(len(e))) / tot
                         for i in range(len(q[b][hq]))])
        out.append(rows)
    return np.array(out)


def pin_brute_force(impl):
    rng = np.random.default_rng(9)
    bsz, hkv, g, d, nb = 2, 2, 2, 4, 12
    lens = [1, 2, 3, 5]
    tables = [list(rng.permutation(nb)[:3]) for _ in lens]
    q = rng.standard_normal((4, hkv * g, d)).astype(np.float32)
    k_pool = rng.standard_normal((nb, hkv, d // 2, bsz, 2)).astype(np.float32)
    v_pool = rng.standard_normal((nb, hkv, d, bsz)).astype(np.float32)
    got = impl.decode(q, k_pool, v_pool, np.array(tables), np.array(lens), bsz,
                      0.5, "f32", "f32")
    want = _brute_decode(q, k_pool, v_pool, tables, lens, bsz, 0.5, g)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def pin_brute_force_tiny_workload(impl):
    """Brute force on the tiny fp32 workload at a reduced size."""
    w = WORKLOADS[1]
    batch = make_batch(w, lens=np.array([1, 3, 17, 33]))
    h = _host(batch)
    k2, v2 = impl.write_tokens(h["k"], h["v"], h["kn"], h["vn"], batch.slot_mapping,
                               w.block_size, "f32", "f32")
    got = impl.decode(h["q"], k2, v2, batch.block_tables, batch.context_lens,
                      w.block_size, batch.scale, "f32", "f32")
    want = _brute_decode(h["q"], k2, v2, batch.block_tables, batch.context_lens,
                         w.block_size, float(np.float32(batch.scale)), w.group)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def pin_paged_equals_unpaged(impl):
    """Paged attention equals attention on the contiguous per-sequence
    layout, bit for bit ("AI Inference Serving at Scale", FAQ)."""
    rng = np.random.default_rng(10)
    bsz, hkv, g, d, nb, length = 16, 2, 4, 32, 10, 70
    k_c = rng.standard_normal((length, hkv, d)).astype(np.float32)
    v_c = rng.standard_normal((length, hkv, d)).astype(np.float32)
    q = rng.standard_normal((1, hkv * g, d)).astype(np.float32)
    table = rng.permutation(nb)[:5]
    k_pool = _k_pool(nb, hkv, bsz, d, 4, np.nan, np.float32)
    v_pool = np.full((nb, hkv, d, bsz), np.nan, np.float32)
    _scatter_contiguous(k_c, v_c, bsz, table, k_pool, v_pool)
    paged_out = impl.decode(q, k_pool, v_pool, table[None], np.array([length]), bsz,
                            0.125, "f32", "f32")
    flat = impl.attention(q[0].astype(np.float64), k_c.astype(np.float64),
                          v_c.astype(np.float64), 0.125)
    assert np.array_equal(paged_out[0], flat)


def pin_block_permutation(impl):
    """Relabelling physical blocks (moving the data along) changes no bit."""
    for idx in (1, 2):
        w = WORKLOADS[idx]
        batch = make_batch(w, num_seqs=3, lens=None if idx == 1 else np.array([40, 77, 130]))
        base = _decode_batch(impl, batch)
        perm = np.random.default_rng(11).permutation(batch.num_blocks)
        moved = _decode_batch(impl, permute_blocks(batch, perm))
        assert np.array_equal(base, moved)
        cont = _decode_batch(impl, contiguous_layout(batch))
        assert np.array_equal(base, cont)


def pin_shared_prefix(impl):
    """Sequences pointing at shared prefix blocks equal private copies."""
    w = WORKLOADS[4]
    rng = np.random.default_rng(12)
    lens = 2048 + rng.integers(1, 40, size=3)
    batch = make_batch(w, num_seqs=3, lens=lens)
    small = batch.replace(q=batch.q[:, :4].contiguous(),
                          k_pool=batch.k_pool[:, :1].contiguous(),
                          v_pool=batch.v_pool[:, :1].contiguous())
    small = small.replace(workload=dataclasses.replace(w, num_q_heads=4, num_kv_heads=1))
    assert np.all(small.ref_counts[small.block_tables[0, :128]] == 3)
    shared = _decode_batch(impl, small)
    copied = unshare(small)
    assert copied.num_blocks == small.num_blocks + 3 * 128
    assert np.all(copied.ref_counts[copied.ref_counts > 0] == 1)
    assert np.array_equal(shared, _decode_batch(impl, copied))


def pin_split_merge(impl):
    """Merging softmax states of any split equals the unsplit result."""
    rng = np.random.default_rng(13)
    length, hq, hkv, d = 300, 4, 2, 16
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((length, hkv, d)) * 2.0
    v = rng.standard_normal((length, hkv, d))
    full = impl.attention(q, k, v, 0.7)
    for part in (16, 32, 112, 256, 512):
        bounds = list(range(0, length, part)) + [length]
        states = [impl.partial(q, k, v, 0.7, a, b) for a, b in zip(bounds[:-1], bounds[1:])]
        for hh in range(hq):
            ms = np.array([s[0][hh] for s in states])
            ls = np.array([s[1][hh] for s in states])
            os_ = np.array([s[2][hh] for s in states])
            np.testing.assert_allclose(impl.merge(ms, ls, os_), full[hh], rtol=1e-12, atol=1e-13)
    m, l, o = impl.partial(q, k, v, 0.7, 0, length)
    np.testing.assert_allclose(o, full, rtol=1e-13, atol=1e-14)
    for hh in range(hq):
        assert np.array_equal(impl.merge(m[hh:hh + 1], l[hh:hh + 1], o[hh:hh + 1]), o[hh])


def pin_e4m3_decode_table(impl):
    """All 256 E4M3FN codes against torch's float8_e4m3fn dtype."""
    codes = np.arange(256, dtype=np.uint8)
    mine = impl.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def pin_e4m3_encode(impl):
    """Round-to-nearest-even against torch's cast, inside the finite range;
    exact for every representable value and for midpoints (ties to even)."""
    rng = np.random.default_rng(14)
    x = np.concatenate([rng.standard_normal(20000) * 50.0,
                        rng.uniform(-448, 448, 20000),
                        rng.standard_normal(20000) * 1e-2]).astype(np.float32)
    mine = impl.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)
    vals = impl.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    assert np.array_equal(impl.e4m3_encode(vals), np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    ref_mid = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(impl.e4m3_encode(mids), ref_mid)
    assert np.all(impl.e4m3_encode(np.array([449.0, 1e6, -1e9])) == [0x7E, 0x7E, 0xFE])
    assert impl.e4m3_encode(np.array([np.nan]))[0] & 0x7F == 0x7F


def pin_e5m2_decode_table(impl):
    """All 256 E5M2 codes against torch's float8_e5m2 dtype (infinities and
    NaNs included)."""
    codes = np.arange(256, dtype=np.uint8)
    mine = impl.e5m2_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))
    assert mine[0x7B] == 57344.0 and mine[0x01] == 2.0 ** -16 and mine[0x04] == 2.0 ** -14
    assert mine[0x7C] == np.inf and mine[0xFC] == -np.inf


def pin_e5m2_encode(impl):
    """Round-to-nearest-even against torch's float8_e5m2 cast inside the
    finite range, every value and every midpoint exactly; saturation at
    57344 where torch would give infinity."""
    rng = np.random.default_rng(22)
    x = np.concatenate([rng.standard_normal(20000) * 3000.0,
                        rng.uniform(-57344, 57344, 20000),
                        rng.standard_normal(20000) * 1e-4]).astype(np.float32)
    mine = impl.e5m2_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)
    vals = impl.e5m2_to_f64(np.arange(0x7C, dtype=np.uint8))
    assert np.array_equal(impl.e5m2_encode(vals), np.arange(0x7C, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    ref_mid = torch.from_numpy(mids).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(impl.e5m2_encode(mids), ref_mid)
    assert np.all(impl.e5m2_encode(np.array([61440.0, 1e9, -np.inf, np.inf])) == [0x7B, 0x7B, 0xFB, 0x7B])
    assert impl.e5m2_encode(np.array([np.nan]))[0] & 0x7F == 0x7F


def pin_bf16_widen():
    rng = np.random.default_rng(15)
    bits = rng.integers(0, 2**16, 50000).astype(np.uint16)
    mine = codecs.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])


def pin_fp8_write_then_decode(impl):
    """An FP8 append stores the codes of x / scale; the decode multiplies the
    scale back, so a one-token sequence returns the dequantised new row
    (both FP8 formats; codes checked against torch's casts)."""
    for fmt, tdt, widen in (("fp8_e4m3", torch.float8_e4m3fn, impl.e4m3_to_f64),
                            ("fp8_e5m2", torch.float8_e5m2, impl.e5m2_to_f64)):
        rng = np.random.default_rng(16)
        hkv, d, bsz, nb = 2, 16, 32, 3
        k_pool = np.zeros((nb, hkv, d // 16, bsz, 16), np.uint8)
        v_pool = np.zeros((nb, hkv, d, bsz), np.uint8)
        kn = rng.standard_normal((1, hkv, d)).astype(np.float32)
        vn = rng.standard_normal((1, hkv, d)).astype(np.float32)
        ks = np.array([0.01, 0.02], np.float32)
        vs = np.array([0.015, 0.005], np.float32)
        k2, v2 = impl.write_tokens(k_pool, v_pool, kn, vn, np.array([2 * bsz]), bsz,
                                   "f32", fmt, ks, vs)
        ref = torch.from_numpy(vn[0] / vs[:, None]).to(tdt).view(torch.uint8).numpy()
        assert np.array_equal(v2[2, :, :, 0], ref)
        # K codes: chunk c of the token's row sits at [blk, h, c, off, :]
        kref = torch.from_numpy(kn[0] / ks[:, None]).to(tdt).view(torch.uint8).numpy()
        assert np.array_equal(k2[2, :, :, 0, :].reshape(hkv, d), kref)
        q = rng.standard_normal((1, 4, d)).astype(np.float32)
        out = impl.decode(q, k2, v2, np.array([[2]]), np.array([1]), bsz, 0.25,
                          "f32", fmt, ks, vs)
        deq = widen(ref) * vs[:, None].astype(np.float64)
        assert np.array_equal(out[0], deq[np.arange(4) // 2])


def pin_fp8_multi_token_decode(impl):
    """FP8 caches over several tokens, where the K scale no longer cancels
    out of the softmax: sequences of 1, 21 and 40 tokens appended into
    E4M3 / E5M2 pools (K and V codes each checked against torch's cast of
    x / scale) decode to the pinned f32 decode of the dequantised values,
    code * scale per KV head ("AI Inference Serving at Scale", section 6,
    FP8 KV cache), placed in an f32 cache."""
    for fmt, tdt in (("fp8_e4m3", torch.float8_e4m3fn), ("fp8_e5m2", torch.float8_e5m2)):
        rng = np.random.default_rng(41)
        hkv, g, d, bsz, nb = 2, 3, 32, 16, 6
        lens = np.array([1, 21, 40])
        tables = np.array([[4, -1, -1], [0, 5, -1], [1, 2, 3]])
        slots = [int(tables[b, t // bsz]) * bsz + t % bsz
                 for b in range(3) for t in range(lens[b])]
        n = len(slots)
        kn = rng.standard_normal((n, hkv, d)).astype(np.float32)
        vn = rng.standard_normal((n, hkv, d)).astype(np.float32)
        # scales far from 1, unequal between K and V and between heads, and
        # large enough that no |x| / scale passes 448 (torch does not saturate)
        ks = np.array([0.011, 0.031], np.float32)
        vs = np.array([0.023, 0.013], np.float32)
        k_pool = _k_pool(nb, hkv, bsz, d, 16, 0, np.uint8)
        v_pool = np.zeros((nb, hkv, d, bsz), np.uint8)
        k2, v2 = impl.write_tokens(k_pool, v_pool, kn, vn, np.array(slots), bsz,
                                   "f32", fmt, ks, vs)
        kcodes = torch.from_numpy(kn / ks[None, :, None]).to(tdt)
        vcodes = torch.from_numpy(vn / vs[None, :, None]).to(tdt)
        kf = _k_pool(nb, hkv, bsz, d, 4, 0, np.float32)
        vf = np.zeros((nb, hkv, d, bsz), np.float32)
        for idx, sl in enumerate(slots):
            blk, off = divmod(sl, bsz)
            assert np.array_equal(k2[blk, :, :, off, :].reshape(hkv, d),
                                  kcodes[idx].view(torch.uint8).numpy())
            assert np.array_equal(v2[blk, :, :, off], vcodes[idx].view(torch.uint8).numpy())
            kval = kcodes[idx].to(torch.float64).numpy() * ks[:, None].astype(np.float64)
            vval = vcodes[idx].to(torch.float64).numpy() * vs[:, None].astype(np.float64)
            kf[blk, :, :, off, :] = kval.astype(np.float32).reshape(hkv, d // 4, 4)
            vf[blk, :, :, off] = vval.astype(np.float32)
        q = rng.standard_normal((3, hkv * g, d)).astype(np.float32)
        out = impl.decode(q, k2, v2, tables, lens, bsz, 0.5, "f32", fmt, ks, vs)
        ref = impl.decode(q, kf, vf, tables, lens, bsz, 0.5, "f32", "f32")
        # code * scale has up to 28 significant bits: the f32 cache rounds it
        np.testing.assert_allclose(out, ref, rtol=2e-6, atol=2e-7)


def pin_copy_on_write(impl):
    """Copy-on-write: a sequence that shares a partly filled block forks it
    before appending.  After the copy and the append, the forked sequence
    reads the shared tokens plus its new one, every other sequence reads
    what it read before, and every block outside the copy targets keeps its
    bits; dependent pairs are refused."""
    rng = np.random.default_rng(17)
    bsz, hkv, d, nb = 4, 2, 8, 10
    k_pool = rng.standard_normal((nb, hkv, d // 4, bsz, 4)).astype(np.float32)
    v_pool = rng.standard_normal((nb, hkv, d, bsz)).astype(np.float32)
    shared = [3, 7]                 # prefix of 6 tokens: block 7 holds tokens 4, 5
    table_a, table_b = list(shared), list(shared)
    before_b = impl.gather(k_pool, v_pool, np.array(table_b), 6, bsz)
    table_a[1] = 9                  # a forks block 7 into free block 9
    k2, v2 = impl.copy_blocks(k_pool, v_pool, np.array([[7, 9]]))
    kn = rng.standard_normal((1, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((1, hkv, d)).astype(np.float32)
    k3, v3 = impl.write_tokens(k2, v2, kn, vn, np.array([9 * bsz + 2]), bsz, "f32", "f32")
    ka, va = impl.gather(k3, v3, np.array(table_a), 7, bsz)
    kb, vb = impl.gather(k3, v3, np.array(table_b), 6, bsz)
    assert np.array_equal(ka[:6], before_b[0]) and np.array_equal(va[:6], before_b[1])
    assert np.array_equal(ka[6], kn[0]) and np.array_equal(va[6], vn[0])
    assert np.array_equal(kb, before_b[0]) and np.array_equal(vb, before_b[1])
    others = [i for i in range(nb) if i != 9]
    assert np.array_equal(k2[others], k_pool[others]) and np.array_equal(v2[others], v_pool[others])
    for bad in ([[1, 2], [3, 2]], [[1, 2], [2, 4]]):
        try:
            impl.copy_blocks(k_pool, v_pool, np.array(bad))
        except ValueError:
            continue
        raise AssertionError(f"dependent copy pairs accepted: {bad}")


def pin_swap_round_trip(impl):
    """Preemption: a sequence's blocks go out to a host pool and come back
    into different device blocks; through the updated table it reads the
    same tokens, and nothing else changes."""
    rng = np.random.default_rng(21)
    bsz, hkv, d, nb, nh = 4, 2, 8, 12, 6
    k_dev = rng.standard_normal((nb, hkv, d // 4, bsz, 4)).astype(np.float32)
    v_dev = rng.standard_normal((nb, hkv, d, bsz)).astype(np.float32)
    k_host = np.zeros((nh, hkv, d // 4, bsz, 4), np.float32)
    v_host = np.zeros((nh, hkv, d, bsz), np.float32)
    table, length = np.array([3, 7, 1]), 10
    before = impl.gather(k_dev, v_dev, table, length, bsz)
    k_host, v_host = impl.swap_blocks(k_dev, v_dev, k_host, v_host, np.array([[3, 4], [7, 0], [1, 2]]))
    k_dev2, v_dev2 = k_dev.copy(), v_dev.copy()
    k_dev2[[3, 7, 1]] = np.nan                       # the device blocks are reused meanwhile
    v_dev2[[3, 7, 1]] = np.nan
    k_dev3, v_dev3 = impl.swap_blocks(k_host, v_host, k_dev2, v_dev2, np.array([[4, 5], [0, 9], [2, 11]]))
    after = impl.gather(k_dev3, v_dev3, np.array([5, 9, 11]), length, bsz)
    assert np.array_equal(after[0], before[0]) and np.array_equal(after[1], before[1])
    keep = [i for i in range(nb) if i not in (5, 9, 11)]
    assert np.array_equal(k_dev3[keep], k_dev2[keep], equal_nan=True)
    assert np.array_equal(v_dev3[keep], v_dev2[keep], equal_nan=True)
    try:
        impl.swap_blocks(k_dev, v_dev, k_host, v_host, np.array([[1, 2], [3, 2]]))
    except ValueError:
        return
    raise AssertionError("swap pairs with a repeated destination accepted")


def pin_int4_encode(impl):
    """Symmetric INT4 with one scale per group: closed forms (absmax 7 gives
    scale 1, so codes are the nearest-even integers), the extremes at +-7,
    the all-zero group, and a brute-force nearest-level search over -7..7
    on random groups, with the error bound |x - c*s| <= s/2."""
    x = np.array([7.0, -3.5, 2.5, 0.5, -0.5, 1.5, -7.0, 6.25, -2.75, 4.5], np.float32)
    codes, scale = impl.int4_encode(x)
    assert scale == np.float32(1.0)
    assert codes.tolist() == [7, -4, 2, 0, 0, 2, -7, 6, -3, 4]
    codes, scale = impl.int4_encode(np.array([0.3, -0.3, 0.1], np.float32))
    assert codes.tolist()[:2] == [7, -7] and scale == np.float32(np.float32(0.3) / np.float32(7))
    codes, scale = impl.int4_encode(np.zeros(16, np.float32))
    assert scale == 0 and not codes.any()
    rng = np.random.default_rng(31)
    levels = np.arange(-7, 8)
    for mag in (1.0, 1e-3, 40.0):
        g = (rng.standard_normal((64, 32)) * mag).astype(np.float32)
        for row in g:
            codes, scale = impl.int4_encode(row)
            want_scale = np.float32(np.float32(np.abs(row).max()) / np.float32(7))
            assert scale == want_scale
            qv = (row / want_scale).astype(np.float64)
            dist = np.abs(qv[:, None] - levels[None, :])
            best = dist.min(axis=1, keepdims=True)
            cand = np.where(dist == best, levels[None, :], 99)
            even = np.where(cand % 2 == 0, cand, 99).min(axis=1)
            want = np.where((cand != 99).sum(axis=1) > 1, even, cand.min(axis=1))
            assert np.array_equal(codes, want)
            err = np.abs(row.astype(np.float64) - codes * np.float64(scale))
            assert np.all(err <= 0.5 * np.float64(scale) * (1 + 1e-6))
            assert np.abs(codes).max() == 7


def pin_int4_octets(impl):
    """Nibble layout, from literal bytes: byte i of an octet holds element i
    (low nibble) and element i + 4 (high nibble), two's complement."""
    b = np.array([0x51, 0x62, 0x73, 0xF4, 0x88, 0x0F, 0xF0, 0x00], np.uint8)
    want = [1, 2, 3, 4, 5, 6, 7, -1, -8, -1, 0, 0, -8, 0, -1, 0]
    assert impl.unpack_octets(b).tolist() == want
    assert impl.pack_octets(np.array(want)).tolist() == b.tolist()


def pin_int4_tile_index(impl):
    """INT4 tiles built byte by byte from the layout's index arithmetic
    (written here, not taken from the oracle) read back token by token and
    block by block: K element i of token j at byte (i // 32 * B + j) * 16 +
    (i % 32) // 8 * 4 + i % 4, high nibble iff i % 8 >= 4; V element of
    dimension i, token j at byte i * B / 2 + j // 8 * 4 + j % 4, high nibble
    iff j % 8 >= 4; token j's scale at byte B * d / 2 + 4 j.  An append of
    rows with absmax 7 (scale 1, codes = the values) writes those bytes."""
    rng = np.random.default_rng(32)
    for d, bsz in ((64, 16), (128, 32)):
        kc = rng.integers(-8, 8, (bsz, d))
        vc = rng.integers(-8, 8, (bsz, d))
        ks = rng.uniform(0.1, 1.0, bsz).astype(np.float32)
        vs = rng.uniform(0.1, 1.0, bsz).astype(np.float32)
        tiles = np.zeros((2, 1, 1, bsz * (d // 2 + 4)), np.uint8)
        for j in range(bsz):
            for i in range(d):
                kb = (i // 32 * bsz + j) * 16 + (i % 32) // 8 * 4 + i % 4
                vb = i * bsz // 2 + j // 8 * 4 + j % 4
                tiles[0, 0, 0, kb] |= (int(kc[j, i]) & 15) << (4 if i % 8 >= 4 else 0)
                tiles[1, 0, 0, vb] |= (int(vc[j, i]) & 15) << (4 if j % 8 >= 4 else 0)
        at = bsz * d // 2
        tiles[0, 0, 0, at:] = ks.view(np.uint8)
        tiles[1, 0, 0, at:] = vs.view(np.uint8)
        kpool, vpool = tiles[0], tiles[1]
        for j in range(bsz):
            c, s_ = impl.int4_k_row(kpool, 0, 0, j, bsz)
            assert np.array_equal(c, kc[j]) and s_ == ks[j]
            c, s_ = impl.int4_v_row(vpool, 0, 0, j, bsz)
            assert np.array_equal(c, vc[j]) and s_ == vs[j]
        assert np.array_equal(impl.int4_block_values(kpool[0], bsz, "k")[:, 0],
                              kc * ks[:, None].astype(np.float64))
        assert np.array_equal(impl.int4_block_values(vpool[0], bsz, "v")[:, 0],
                              vc * vs[:, None].astype(np.float64))
        # append: rows reaching +-7 get scale 1 and store their own values
        rows_k = np.clip(kc, -7, 7).astype(np.float32)
        rows_v = np.clip(vc, -7, 7).astype(np.float32)
        rows_k[:, 0], rows_v[:, 0] = 7.0, -7.0
        empty = np.zeros((1, 1, bsz * (d // 2 + 4)), np.uint8)
        kw, vw = impl.write_tokens(empty, empty.copy(), rows_k[:, None, :], rows_v[:, None, :],
                                   np.arange(bsz), bsz, "f32", "int4")
        want = np.zeros((2, bsz * (d // 2 + 4)), np.uint8)
        for j in range(bsz):
            for i in range(d):
                kb = (i // 32 * bsz + j) * 16 + (i % 32) // 8 * 4 + i % 4
                vb = i * bsz // 2 + j // 8 * 4 + j % 4
                want[0, kb] |= (int(rows_k[j, i]) & 15) << (4 if i % 8 >= 4 else 0)
                want[1, vb] |= (int(rows_v[j, i]) & 15) << (4 if j % 8 >= 4 else 0)
        want[:, bsz * d // 2:] = np.ones(bsz, np.float32).view(np.uint8)
        assert np.array_equal(kw[0, 0], want[0]) and np.array_equal(vw[0, 0], want[1])


def pin_int4_write_then_decode(impl):
    """An INT4 append stores each row's codes and scale; a one-token
    sequence decodes to its dequantised V row exactly, and the decode of an
    INT4 cache equals the (pinned) f32 decode of the same values placed in
    an f32 cache, up to the f32 rounding of code * scale."""
    rng = np.random.default_rng(33)
    hkv, g, d, bsz, nb = 2, 3, 64, 16, 6
    tile = bsz * (d // 2 + 4)
    k_pool = np.zeros((nb, hkv, tile), np.uint8)
    v_pool = np.zeros((nb, hkv, tile), np.uint8)
    lens = np.array([1, 21, 40])
    tables = np.array([[4, -1, -1], [0, 5, -1], [1, 2, 3]])
    slots = [tables[b, t // bsz] * bsz + t % bsz for b in range(3) for t in range(lens[b])]
    n = len(slots)
    kn = rng.standard_normal((n, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((n, hkv, d)).astype(np.float32)
    k2, v2 = impl.write_tokens(k_pool, v_pool, kn, vn, np.array(slots), bsz, "f32", "int4")
    q = rng.standard_normal((3, hkv * g, d)).astype(np.float32)
    out = impl.decode(q, k2, v2, tables, lens, bsz, 0.125, "f32", "int4")
    vc, vsc = impl.int4_encode(vn[0, 1])
    assert np.array_equal(out[0, g:2 * g], np.tile(vc * np.float64(vsc), (g, 1)))
    kf = np.zeros((nb, hkv, d // 4, bsz, 4), np.float32)
    vf = np.zeros((nb, hkv, d, bsz), np.float32)
    for idx, sl in enumerate(slots):
        blk, off = divmod(sl, bsz)
        for h in range(hkv):
            kcode, kscale = impl.int4_encode(kn[idx, h])
            vcode, vscale = impl.int4_encode(vn[idx, h])
            assert np.array_equal(impl.int4_k_row(k2, blk, h, off, bsz)[0], kcode)
            kf[blk, h, :, off, :] = (kcode * kscale).astype(np.float32).reshape(d // 4, 4)
            vf[blk, h, :, off] = (vcode * vscale).astype(np.float32)
    ref = impl.decode(q, kf, vf, tables, lens, bsz, 0.125, "f32", "f32")
    # code * scale needs up to 27 significant bits: the f32 cache rounds it
    np.testing.assert_allclose(out, ref, rtol=2e-6, atol=2e-7)


def _prefill_case(rng, lens, qlens, hkv=2, g=2, d=8, bsz=4):
    """Random paged pools and tables for several sequences (f32)."""
    nb = sum(-(-L // bsz) for L in lens) + 3
    perm = rng.permutation(nb)
    tables, used = [], 0
    for L in lens:
        n = -(-L // bsz)
        tables.append(list(perm[used:used + n]) + [-1] * 0)
        used += n
    width = max(len(t) for t in tables)
    tab = np.full((len(lens), width), -1, np.int64)
    for b, t in enumerate(tables):
        tab[b, :len(t)] = t
    k_pool = rng.standard_normal((nb, hkv, d // 2, bsz, 2)).astype(np.float32)
    v_pool = rng.standard_normal((nb, hkv, d, bsz)).astype(np.float32)
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int64)
    q = rng.standard_normal((int(qs[-1]), hkv * g, d)).astype(np.float32)
    return q, k_pool, v_pool, tab, np.array(lens), qs, bsz, g


def _brute_prefill(q, k_pool, v_pool, tables, lens, qs, bsz, scale, group):
    """Pure-Python loops: each query row over the tokens up to its position."""
    x = len(k_pool[0][0][0][0])
    out = np.zeros(q.shape)
    for b in range(len(lens)):
        nq = int(qs[b + 1] - qs[b])
        for i in range(nq):
            p = int(lens[b]) - nq + i
            for hq in range(q.shape[1]):
                h = hq // group
                z, vs = [], []
                for t in range(p + 1):
                    blk, off = tables[b][t // bsz], t % bsz
                    kk = [float(k_pool[blk][h][e // x][off][e % x]) for e in range(q.shape[2])]
                    z.append(scale * sum(float(q[qs[b] + i][hq][e]) * kk[e] for e in range(q.shape[2])))
                    vs.append([float(v_pool[blk][h][e][off]) for e in range(q.shape[2])])
                zm = max(z)
                w = [math.exp(v_ - zm) for v_ in z]
                tot = sum(w)
                out[qs[b] + i, hq] = [sum(w[t] * vs[t][e] for t in range(len(w))) / tot
                                      for e in range(q.shape[2])]
    return out


def pin_prefill_brute_force(impl):
    rng = np.random.default_rng(18)
    q, kp, vp, tab, lens, qs, bsz, g = _prefill_case(rng, [5, 9, 3], [2, 4, 3])
    got = impl.prefill_chunk(q, kp, vp, tab, lens, qs, bsz, 0.5, "f32", "f32")
    want = _brute_prefill(q, kp, vp, tab, lens, qs, bsz, 0.5, g)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def pin_prefill_causal(impl):
    """Row i never sees a token after its position; the last row of a
    sequence is the single-query decode over the whole context, and a
    one-token chunk is that decode too."""
    rng = np.random.default_rng(19)
    q, kp, vp, tab, lens, qs, bsz, g = _prefill_case(rng, [21, 13], [6, 5], d=16)
    base = impl.prefill_chunk(q, kp, vp, tab, lens, qs, bsz, 0.7, "f32", "f32")
    # perturb the token at position L - 2 of sequence 0: rows 0..3 (positions < L - 2) keep their bits
    L0, Q0 = int(lens[0]), 6
    t = L0 - 2
    kp2, vp2 = kp.copy(), vp.copy()
    blk, off = tab[0][t // bsz], t % bsz
    kp2[blk, :, :, off, :] += 3.0
    vp2[blk, :, :, off] -= 2.0
    pert = impl.prefill_chunk(q, kp2, vp2, tab, lens, qs, bsz, 0.7, "f32", "f32")
    assert np.array_equal(pert[:Q0 - 2], base[:Q0 - 2])
    assert not np.allclose(pert[Q0 - 2], base[Q0 - 2])
    assert np.array_equal(pert[qs[1]:], base[qs[1]:])       # other sequence untouched
    for b in range(2):
        last = int(qs[b + 1]) - 1
        dec = impl.decode(q[last:last + 1], kp, vp, tab[b:b + 1], lens[b:b + 1], bsz, 0.7,
                          "f32", "f32")
        np.testing.assert_allclose(base[last], dec[0], rtol=1e-13, atol=1e-14)


def pin_prefill_library_sdpa(impl):
    """One sequence laid out contiguously: the chunk's rows equal torch's
    float64 scaled-dot-product attention of the last Q positions with an
    explicit causal mask over the whole context."""
    rng = np.random.default_rng(20)
    L, Q, hkv, g, d, bsz = 40, 7, 2, 3, 16, 8
    q, kp, vp, tab, lens, qs, bsz, g = _prefill_case(rng, [L], [Q], hkv=hkv, g=g, d=d, bsz=bsz)
    got = impl.prefill_chunk(q, kp, vp, tab, lens, qs, bsz, 0.25, "f32", "f32")
    kc = np.stack([kp[tab[0][t // bsz], :, :, t % bsz, :].reshape(hkv, d) for t in range(L)])
    vc = np.stack([vp[tab[0][t // bsz], :, :, t % bsz] for t in range(L)])
    kt = torch.from_numpy(np.repeat(kc, g, axis=1).astype(np.float64)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.repeat(vc, g, axis=1).astype(np.float64)).permute(1, 0, 2)[None]
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]      # [1, Hq, Q, d]
    mask = torch.from_numpy(np.arange(L)[None, :] <= (L - Q + np.arange(Q))[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(qt.contiguous(), kt.contiguous(),
                                                           vt.contiguous(), attn_mask=mask,
                                                           scale=0.25)
    np.testing.assert_allclose(got, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


# ==========================================================================
# the pins on the oracle
# ==========================================================================

PINS = [pin_golden_index, pin_gather_roundtrip, pin_write_whole_pool,
        pin_write_then_gather, pin_single_token, pin_two_tokens,
        pin_identical_keys_mean, pin_saturation, pin_gqa_equals_repeated_mha,
        pin_library_sdpa, pin_brute_force, pin_brute_force_tiny_workload,
        pin_paged_equals_unpaged, pin_block_permutation, pin_shared_prefix,
        pin_split_merge, pin_e4m3_decode_table, pin_e4m3_encode,
        pin_fp8_write_then_decode, pin_fp8_multi_token_decode, pin_copy_on_write, pin_prefill_brute_force,
        pin_prefill_causal, pin_prefill_library_sdpa, pin_swap_round_trip,
        pin_e5m2_decode_table, pin_e5m2_encode, pin_int4_encode, pin_int4_octets,
        pin_int4_tile_index, pin_int4_write_then_decode]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(ORACLE)


def test_bf16_widen():
    pin_bf16_widen()


def test_oracle_decode_partials_contract():
    """decode_partials fills exactly the partitions each sequence has."""
    w = WORKLOADS[2]
    batch = make_batch(w, num_seqs=3, lens=np.array([33, 64, 100]))
    h = _host(batch)
    m, l, o = paged.decode_partials(h["q"], h["k"], h["v"], batch.block_tables,
                                    batch.context_lens, 16, batch.scale, "bf16",
                                    "bf16", 32)
    assert m.shape == (3, 32, 4) and o.shape == (3, 32, 4, 128)
    assert np.isnan(m[0, :, 2:]).all() and not np.isnan(m[0, :, :2]).any()
    assert not np.isnan(m[2]).any()
    full = _decode_batch(ORACLE, batch)
    for b in range(3):
        n = -(-int(batch.context_lens[b]) // 32)
        for hq in range(32):
            np.testing.assert_allclose(
                paged.merge(m[b, hq, :n], l[b, hq, :n], o[b, hq, :n]),
                full[b, hq], rtol=1e-12, atol=1e-13)


def test_oracle_rejects_duplicate_slots():
    k = np.zeros((2, 1, 1, 16, 4), np.float32)
    v = np.zeros((2, 1, 4, 16), np.float32)
    rows = np.ones((2, 1, 4), np.float32)
    with pytest.raises(ValueError):
        paged.write_tokens(k, v, rows, rows, np.array([3, 3]), 16, "f32", "f32")


def test_oracle_empty_context_is_zero():
    out = paged.attention(np.ones((2, 4)), np.zeros((0, 1, 4)), np.zeros((0, 1, 4)), 1.0)
    assert np.array_equal(out, np.zeros((2, 4)))


def test_oracle_package_header_says_test_only():
    assert "TEST INFRASTRUCTURE ONLY" in oracle.__doc__


# ==========================================================================
# planted mistakes: each broken copy of the oracle must fail some pin
# ==========================================================================

def _bad_slot_of(table_row, t, block_size):
    i, j = divmod(int(t) + 1, int(block_size))  # off by one
    return int(table_row[i]), j


def _bad_gather_v_layout(k_pool, v_pool, table_row, length, block_size):
    k, _ = paged.gather(k_pool, v_pool, table_row, length, block_size)
    v = np.empty_like(k)
    for t in range(length):  # reads V as if it were token-major like K
        blk, off = paged.slot_of(table_row, t, block_size)
        v[t] = v_pool.reshape(v_pool.shape[0], v_pool.shape[1], block_size, -1)[blk, :, off, :]
    return k, v


def _bad_gather_k_token_major(k_pool, v_pool, table_row, length, block_size):
    _, v = paged.gather(k_pool, v_pool, table_row, length, block_size)
    k = np.empty_like(v)
    nb, hkv = k_pool.shape[:2]
    flat = k_pool.reshape(nb, hkv, block_size, -1)  # ignores the 16-byte chunking
    for t in range(length):
        blk, off = paged.slot_of(table_row, t, block_size)
        k[t] = flat[blk, :, off, :]
    return k, v


def _bad_attention_no_scale(q, k, v, scale):
    return paged.attention(q, k, v, 1.0)


def _bad_attention_gqa_modulo(q, k, v, scale):
    n_q = q.shape[0]
    out = np.zeros_like(q, dtype=np.float64)
    for hq in range(n_q):
        h = hq % k.shape[1]  # interleaved instead of consecutive grouping
        z = scale * (k[:, h, :] @ q[hq])
        e = np.exp(z - z.max())
        out[hq] = (e / e.sum()) @ v[:, h, :]
    return out


def _bad_attention_sign(q, k, v, scale):
    return paged.attention(-q, k, v, scale)


def _bad_attention_drop_last(q, k, v, scale):
    return paged.attention(q, k[:-1], v[:-1], scale) if k.shape[0] > 1 else paged.attention(q, k, v, scale)


def _bad_merge_no_rescale(ms, ls, os_):
    return (ls[:, None] * os_).sum(axis=0) / ls.sum()


def _bad_e4m3_bias(codes):
    return paged.codecs.e4m3_to_f64(codes) * 2.0


def _bad_encode_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    vals = codecs.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mag = np.minimum(np.abs(x), 448.0)
    idx = np.searchsorted(vals, mag, side="right") - 1
    return (idx.astype(np.uint8) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8))


def _bad_write_skip_v(k_pool, v_pool, k_new, v_new, slot_mapping, block_size,
                      src_dtype, cache_dtype, k_scale=None, v_scale=None):
    k2, _ = paged.write_tokens(k_pool, v_pool, k_new, v_new, slot_mapping, block_size,
                               src_dtype, cache_dtype, k_scale, v_scale)
    return k2, v_pool.copy()


def _bad_copy_k_only(k_pool, v_pool, block_mapping):
    k2, _ = paged.copy_blocks(k_pool, v_pool, block_mapping)
    return k2, v_pool.copy()


def _bad_copy_first_head(k_pool, v_pool, block_mapping):
    k2, v2 = k_pool.copy(), v_pool.copy()
    for src, dst in np.asarray(block_mapping).reshape(-1, 2):
        k2[dst, 0] = k_pool[src, 0]
        v2[dst, 0] = v_pool[src, 0]
    return k2, v2


def _bad_copy_reversed(k_pool, v_pool, block_mapping):
    return paged.copy_blocks(k_pool, v_pool, np.asarray(block_mapping)[:, ::-1])


def _bad_prefill_excludes_self(q, k_pool, v_pool, block_tables, context_lens, query_start,
                               block_size, scale, q_dtype, cache_dtype, k_scale=None,
                               v_scale=None, seqs=None):
    out = np.zeros(q.shape)
    for b in range(len(query_start) - 1):
        r0, r1 = int(query_start[b]), int(query_start[b + 1])
        L = int(context_lens[b])
        k, v = paged.sequence_kv_f64(k_pool, v_pool, block_tables[b], L, block_size, cache_dtype)
        for i in range(r1 - r0):
            p = L - (r1 - r0) + i
            out[r0 + i] = paged.attention(paged.to_f64(q[r0 + i], q_dtype), k[:max(p, 1)],
                                          v[:max(p, 1)], float(np.float32(scale)))
    return out


def _bad_prefill_from_start(q, k_pool, v_pool, block_tables, context_lens, query_start,
                            block_size, scale, q_dtype, cache_dtype, k_scale=None,
                            v_scale=None, seqs=None):
    out = np.zeros(q.shape)
    for b in range(len(query_start) - 1):
        r0, r1 = int(query_start[b]), int(query_start[b + 1])
        L = int(context_lens[b])
        k, v = paged.sequence_kv_f64(k_pool, v_pool, block_tables[b], L, block_size, cache_dtype)
        for i in range(r1 - r0):  # positions counted from 0 instead of L - Q
            out[r0 + i] = paged.attention(paged.to_f64(q[r0 + i], q_dtype), k[:i + 1], v[:i + 1],
                                          float(np.float32(scale)))
    return out


def _bad_prefill_no_mask(q, k_pool, v_pool, block_tables, context_lens, query_start,
                         block_size, scale, q_dtype, cache_dtype, k_scale=None,
                         v_scale=None, seqs=None):
    out = np.zeros(q.shape)
    for b in range(len(query_start) - 1):
        r0, r1 = int(query_start[b]), int(query_start[b + 1])
        L = int(context_lens[b])
        k, v = paged.sequence_kv_f64(k_pool, v_pool, block_tables[b], L, block_size, cache_dtype)
        for i in range(r1 - r0):
            out[r0 + i] = paged.attention(paged.to_f64(q[r0 + i], q_dtype), k, v,
                                          float(np.float32(scale)))
    return out


def _bad_swap_first_token_only(src_k, src_v, dst_k, dst_v, block_mapping):
    k2, v2 = dst_k.copy(), dst_v.copy()
    for s_, d in np.asarray(block_mapping).reshape(-1, 2):
        k2[d, :, :, 0] = src_k[s_, :, :, 0]
        v2[d, :, :, 0] = src_v[s_, :, :, 0]
    return k2, v2


def _bad_e5m2_bias(codes):
    return codecs.e5m2_to_f64(codes) * 0.5


def _bad_e5m2_overflow_to_inf(x):
    out = codecs.e5m2_encode(x)
    big = np.abs(np.asarray(x, np.float64)) > 57344.0
    return np.where(big, out | 0x7C, out).astype(np.uint8)


def _bad_int4_truncate(x):
    codes, scale = codecs.int4_encode(x)
    if scale == 0:
        return codes, scale
    q = (np.asarray(x, np.float32) / scale).astype(np.float32)
    return np.clip(np.trunc(q), -7, 7).astype(np.int8), scale


def _bad_int4_scale_8(x):
    x = np.asarray(x, np.float32)
    scale = np.float32(np.float32(np.abs(x).max()) / np.float32(8))
    if scale == 0:
        return np.zeros(x.shape, np.int8), scale
    return np.clip(np.rint(x / scale), -8, 7).astype(np.int8), scale


def _bad_unpack_swapped(b):
    b = np.asarray(b, np.uint8)
    return paged.unpack_octets(((b & 0xF) << 4) | (b >> 4))


def _bad_unpack_ones_complement(b):
    c = paged.unpack_octets(b)
    return np.where(c < 0, c + 1, c)


def _bad_int4_v_token_major(v_pool, blk, h, off, block_size):
    tile = v_pool[blk, h]
    d = paged.int_tile_head_dim(tile.shape[0], block_size)
    rows = paged.unpack_octets(tile[:block_size * d // 2].reshape(block_size, d // 2))
    return rows[off].copy(), paged._int4_scale(tile, d, block_size, off)


def _bad_int4_block_v_token_major(tiles, block_size, which):
    if which == "k":
        return paged.int4_block_values(tiles, block_size, which)
    n_kv, tile = tiles.shape
    d = paged.int_tile_head_dim(tile, block_size)
    c = paged.unpack_octets(tiles[:, :block_size * d // 2].reshape(n_kv, block_size, d // 2))
    s_ = tiles[:, block_size * d // 2:].copy().view(np.float32).astype(np.float64)
    return c.transpose(1, 0, 2) * s_.T[:, :, None]


def _bad_int4_k_dims_interleaved(k_pool, blk, h, off, block_size):
    codes, scale = paged.int4_k_row(k_pool, blk, h, off, block_size)
    return codes.reshape(-1, 2)[:, ::-1].reshape(-1), scale


def _bad_fp8_decode_drops_k_scale(q, k_pool, v_pool, block_tables, context_lens, block_size,
                                  scale, q_dtype, cache_dtype, k_scale=None, v_scale=None,
                                  seqs=None):
    if cache_dtype in ("fp8_e4m3", "fp8_e5m2"):
        k_scale = np.ones_like(np.asarray(k_scale, np.float32))
    return paged.decode(q, k_pool, v_pool, block_tables, context_lens, block_size, scale,
                        q_dtype, cache_dtype, k_scale, v_scale, seqs)


def _bad_fp8_write_k_uses_v_scale(k_pool, v_pool, k_new, v_new, slot_mapping, block_size,
                                  src_dtype, cache_dtype, k_scale=None, v_scale=None):
    return paged.write_tokens(k_pool, v_pool, k_new, v_new, slot_mapping, block_size,
                              src_dtype, cache_dtype, v_scale, v_scale)


def _mk_decode(**over):
    """decode() rebuilt on top of possibly broken parts."""
    impl = _impl(**over)

    def decode(q, k_pool, v_pool, block_tables, context_lens, block_size, scale,
               q_dtype, cache_dtype, k_scale=None, v_scale=None, seqs=None):
        q64 = paged.to_f64(q, q_dtype)
        out = np.zeros(q64.shape)
        scale = float(np.float32(scale))
        for b in range(q64.shape[0]):
            if cache_dtype == "int4":  # tiles of codes and scales: no raw-row gather
                k, v = paged.gather_int4_f64(k_pool, v_pool, block_tables[b],
                                             int(context_lens[b]), block_size)
                out[b] = impl.attention(q64[b], k, v, scale)
                continue
            kr, vr = impl.gather(k_pool, v_pool, block_tables[b], int(context_lens[b]), block_size)
            k = paged.to_f64(kr, cache_dtype)
            v = paged.to_f64(vr, cache_dtype)
            if cache_dtype in ("fp8_e4m3", "fp8_e5m2"):
                k = k * np.asarray(k_scale, np.float64)[None, :, None]
                v = v * np.asarray(v_scale, np.float64)[None, :, None]
            out[b] = impl.attention(q64[b], k, v, scale)
        return out
    return decode


MUTANTS = {
    "index-off-by-one": dict(slot_of=_bad_slot_of),
    "v-layout-transposed": dict(gather=_bad_gather_v_layout),
    "k-layout-token-major": dict(gather=_bad_gather_k_token_major),
    "scale-dropped": dict(attention=_bad_attention_no_scale),
    "gqa-interleaved": dict(attention=_bad_attention_gqa_modulo),
    "score-sign": dict(attention=_bad_attention_sign),
    "last-token-dropped": dict(attention=_bad_attention_drop_last),
    "merge-no-rescale": dict(merge=_bad_merge_no_rescale),
    "e4m3-exponent-bias": dict(e4m3_to_f64=_bad_e4m3_bias),
    "e4m3-truncating": dict(e4m3_encode=_bad_encode_truncate),
    "write-drops-v": dict(write_tokens=_bad_write_skip_v),
    "e5m2-exponent-bias": dict(e5m2_to_f64=_bad_e5m2_bias),
    "e5m2-overflow-to-inf": dict(e5m2_encode=_bad_e5m2_overflow_to_inf),
    "copy-drops-v": dict(copy_blocks=_bad_copy_k_only),
    "copy-first-head-only": dict(copy_blocks=_bad_copy_first_head),
    "copy-reversed": dict(copy_blocks=_bad_copy_reversed),
    "swap-first-token-only": dict(swap_blocks=_bad_swap_first_token_only),
    "prefill-excludes-self": dict(prefill_chunk=_bad_prefill_excludes_self),
    "prefill-positions-from-zero": dict(prefill_chunk=_bad_prefill_from_start),
    "prefill-no-causal-mask": dict(prefill_chunk=_bad_prefill_no_mask),
    "int4-truncating": dict(int4_encode=_bad_int4_truncate),
    "int4-scale-absmax-over-8": dict(int4_encode=_bad_int4_scale_8),
    "int4-nibbles-swapped": dict(unpack_octets=_bad_unpack_swapped),
    "int4-ones-complement": dict(unpack_octets=_bad_unpack_ones_complement),
    "int4-v-token-major": dict(int4_v_row=_bad_int4_v_token_major),
    "int4-k-dims-interleaved": dict(int4_k_row=_bad_int4_k_dims_interleaved),
    "int4-block-v-token-major": dict(int4_block_values=_bad_int4_block_v_token_major),
    "fp8-decode-drops-k-scale": dict(decode=_bad_fp8_decode_drops_k_scale),
    "fp8-append-k-uses-v-scale": dict(write_tokens=_bad_fp8_write_k_uses_v_scale),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    over = MUTANTS[name]
    impl = _impl(**over)
    if "gather" in over or "attention" in over:
        impl.decode = _mk_decode(**over)
    caught = []
    for pin in PINS:
        try:
            pin(impl)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"
