"""Host-side input machinery: byte accounting against the pages' printed
figures, the block allocator's semantics, and the workload generator."""

import math
import os

import numpy as np
import pytest

from workloads import (WORKLOADS, BlockManager, Sequence, decode_bytes,
                       kv_bytes, make_batch, permute_blocks, unshare)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [line.split() for line in f if line.strip() and not line.startswith("#")]


@pytest.mark.parametrize("row", _golden_rows("kv_bytes.txt"), ids=lambda r: r[-1])
def test_kv_bytes_match_printed_figures(row):
    layers, heads, dim, elt, tokens = (int(x) for x in row[:5])
    printed, rel = float(row[5]), float(row[6])
    got = kv_bytes(tokens, layers, heads, dim, elt)
    if rel == 0:
        assert got == printed
    else:
        assert abs(got - printed) <= rel * printed


def test_kv_bytes_gqa_request_and_users():
    # "vLLM & High-Throughput Serving", section 1: 4,096 tokens at the
    # rounded 320 KB per token is ~1.31 GB; 50 such users need 65.5 GB.
    per_token = kv_bytes(1, 80, 8, 128, 2)
    assert round(per_token / 1024) == 320
    assert round(4096 * 320 * 1000 / 1e9, 2) == 1.31
    assert round(50 * 1.31, 1) == 65.5


def test_allocator_lifo_and_exhaustion():
    mgr = BlockManager(3, 16, order=[2, 0, 1])
    s = Sequence("a")
    assert mgr.allocate(s) and mgr.allocate(s) and mgr.allocate(s)
    assert s.blocks == [2, 0, 1]
    assert not mgr.allocate(s)          # exhausted: reports failure
    assert mgr.free_blocks == 0
    mgr.free(s)
    assert mgr.free_blocks == 3 and mgr.ref_count(2) == 0


def test_allocator_refcounts_with_sharing():
    mgr = BlockManager(4, 16)
    a, b = Sequence("a"), Sequence("b")
    assert mgr.allocate_tokens(a, 20)   # 2 blocks
    mgr.share(a, b, 2)
    assert [mgr.ref_count(x) for x in a.blocks] == [2, 2]
    mgr.free(a)
    assert mgr.free_blocks == 2         # still held by b
    mgr.free(b)
    assert mgr.free_blocks == 4


def test_allocator_blocks_needed_counts_the_new_token():
    # the scheduler sketch sizes a running sequence as ceil((cached + 1) / B)
    mgr = BlockManager(10, 16)
    s = Sequence("a")
    assert mgr.allocate_tokens(s, 16 + 1)
    assert len(s.blocks) == 2


@pytest.mark.parametrize("idx", [1, 2, 4])
def test_batch_structure(idx):
    w = WORKLOADS[idx]
    lens = None if idx == 1 else (np.array([600, 513, 4096]) if idx == 2 else 2048 + np.array([1, 16, 17]))
    batch = make_batch(w, num_seqs=None if idx == 1 else 3, lens=lens, poison=True)
    bsz = w.block_size
    for b, length in enumerate(batch.context_lens):
        nblk = -(-int(length) // bsz)
        assert (batch.block_tables[b, :nblk] >= 0).all()
        assert (batch.block_tables[b, nblk:] == -1).all()
        blk, off = divmod(int(batch.slot_mapping[b]), bsz)
        assert blk == batch.block_tables[b, (length - 1) // bsz] and off == (length - 1) % bsz
    used = batch.block_tables[batch.block_tables >= 0]
    if idx != 4:
        assert len(np.unique(used)) == len(used)
    else:
        assert (batch.ref_counts[batch.block_tables[0, :128]] == 3).all()
    # the slot of the new token is poisoned before the write
    blk, off = divmod(int(batch.slot_mapping[0]), bsz)
    assert batch.k_pool.dim() == 5 and batch.k_pool.shape[3] == bsz
    assert batch.k_pool.shape[2] * batch.k_pool.shape[4] == w.head_dim
    assert batch.k_pool.shape[4] * batch.k_pool.element_size() == 16
    assert np.isnan(batch.k_pool[blk, :, :, off, :].float().numpy()).all()


def test_batch_is_seeded():
    w = WORKLOADS[2]
    a = make_batch(w, num_seqs=4)
    b = make_batch(w, num_seqs=4)
    assert np.array_equal(a.context_lens, b.context_lens)
    assert np.array_equal(a.block_tables, b.block_tables)
    assert (a.k_pool.view(dtype=a.k_pool.dtype) == b.k_pool).all()
    c = make_batch(w, seed=w.seed + 1, num_seqs=4)
    assert not np.array_equal(a.context_lens, c.context_lens)


def test_full_size_lengths_and_pool():
    # lengths and pool sizes of the full workloads (no tensors drawn)
    from workloads.batch import draw_lens
    w3 = WORKLOADS[3]
    lens = draw_lens(w3, np.random.default_rng(w3.seed), w3.num_seqs)
    assert lens.min() >= 16 and lens.max() <= 32768
    assert 700 < np.median(lens) < 1400
    w2 = WORKLOADS[2]
    lens2 = draw_lens(w2, np.random.default_rng(w2.seed), w2.num_seqs)
    assert lens2.min() >= 512 and lens2.max() <= 4096
    bytes2 = decode_bytes(lens2, 32, 8, 128, 16, "bf16", "bf16")
    assert bytes2["kv"] == int(lens2.sum()) * 4096


def test_fp8_batch_codes_and_scales():
    w = WORKLOADS[5]
    batch = make_batch(w, num_seqs=2, lens=np.array([100, 64]))
    assert batch.k_pool.dtype.itemsize == 1 and batch.k_scale.shape == (8,)
    import torch
    deq = batch.k_pool.view(torch.float8_e4m3fn).float() * batch.k_scale[None, :, None, None, None]
    assert deq.abs().max() <= 448 * batch.k_scale.max() + 1e-6
    assert math.isclose(float(deq.std()), 1.0, rel_tol=0.05)


def test_relayouts_preserve_tables():
    w = WORKLOADS[4]
    batch = make_batch(w, num_seqs=2, lens=2048 + np.array([3, 40]))
    u = unshare(batch)
    assert (u.ref_counts[u.ref_counts > 0] == 1).all()
    perm = np.random.default_rng(0).permutation(u.num_blocks)
    p = permute_blocks(u, perm)
    assert (p.k_pool[p.block_tables[1, 5]] == u.k_pool[u.block_tables[1, 5]]).all()


def test_chunk_k_pool_keeps_each_token_row():
    import torch
    from workloads import chunk_k_pool
    k = torch.randn(3, 2, 16, 64, dtype=torch.float32)
    for t in (k, k.to(torch.bfloat16), (k * 10).to(torch.float8_e4m3fn).view(torch.uint8)):
        c = chunk_k_pool(t)
        x = 16 // t.element_size()
        assert tuple(c.shape) == (3, 2, 64 // x, 16, x)
        for blk, h, off in ((0, 0, 0), (2, 1, 15), (1, 0, 7)):
            assert torch.equal(c[blk, h, :, off, :].reshape(-1), t[blk, h, off])


def test_fork_for_append_copies_only_shared_blocks():
    mgr = BlockManager(6, 16)
    a, b = Sequence("a"), Sequence("b")
    assert mgr.allocate_tokens(a, 20)              # blocks 0, 1
    mgr.share(a, b, 2)
    assert mgr.ref_count(1) == 2
    pair = mgr.fork_for_append(b, 20)             # token 20 lives in block 1, shared
    assert pair == (1, 2) and b.blocks == [0, 2] and a.blocks == [0, 1]
    assert mgr.ref_count(1) == 1 and mgr.ref_count(2) == 1 and mgr.ref_count(0) == 2
    assert mgr.fork_for_append(b, 20) is None      # now private: no copy
    assert mgr.fork_for_append(a, 21) is None      # a holds block 1 alone again
    c = Sequence("c")
    mgr.share(a, c, 2)
    while mgr.free_blocks:
        assert mgr.allocate(Sequence("filler"))
    assert mgr.fork_for_append(c, 17) is False     # no free block: nothing changes
    assert c.blocks == [0, 1] and mgr.ref_count(1) == 2
