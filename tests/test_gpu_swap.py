"""Block swap between the device pools and pinned host pools
(``pa_swap_blocks``): bit-exact against the oracle in both directions, and
a preemption round trip that leaves the decode unchanged."""

import numpy as np
import pytest
import torch

import paged_kv_cache_253_amd as pk
from oracle import paged
from tests.parity import same_bits
from tests.test_gpu_copy import _independent_pairs, _random_pools
from workloads import WORKLOADS, host_view, make_batch

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pinned_like(t, num_blocks):
    shape = (num_blocks,) + tuple(t.shape[1:])
    return torch.zeros(shape, dtype=t.dtype, pin_memory=True)


@pytest.mark.parametrize("dtype,hkv,d,bsz,npairs", [
    ("bf16", 8, 128, 16, 40),
    ("fp8_e4m3", 8, 128, 32, 17),
    ("f32", 2, 64, 16, 9),
])
def test_swap_out_and_in_bit_exact(dtype, hkv, d, bsz, npairs):
    print(f"[swap] {dtype} hkv={hkv} d={d} B={bsz} pairs={npairs}", flush=True)
    nb, nh = 2 * npairs + 5, npairs + 3
    k, v = _random_pools(nb, hkv, d, bsz, dtype, seed=npairs)
    kd, vd = k.to(DEV), v.to(DEV)
    kh, vh = _pinned_like(k, nh), _pinned_like(v, nh)
    rng = np.random.default_rng(npairs)
    out_pairs = np.stack([rng.permutation(nb)[:npairs], rng.permutation(nh)[:npairs]], axis=1)
    k_ref, v_ref = paged.swap_blocks(host_view(k), host_view(v), host_view(kh), host_view(vh),
                                     out_pairs)
    pk.swap_blocks(kh, vh, kd, vd, torch.from_numpy(out_pairs.astype(np.int64)).to(DEV))
    torch.cuda.synchronize()
    assert same_bits(host_view(kh), k_ref) and same_bits(host_view(vh), v_ref)
    # and back in, to other device blocks
    in_pairs = _independent_pairs(nb, npairs, rng)
    in_pairs[:, 0] = out_pairs[:, 1]
    k2, v2 = paged.swap_blocks(k_ref, v_ref, host_view(kd), host_view(vd), in_pairs)
    pk.swap_blocks(kd, vd, kh, vh, torch.from_numpy(in_pairs.astype(np.int64)).to(DEV))
    torch.cuda.synchronize()
    assert same_bits(host_view(kd), k2) and same_bits(host_view(vd), v2)


def test_swap_refuses_unpinned_host_pools():
    k, v = _random_pools(8, 2, 64, 16, "bf16", seed=1)
    kd, vd = k.to(DEV), v.to(DEV)
    st = pk.load().pa_swap_blocks(k.data_ptr(), v.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                                  torch.zeros((1, 2), dtype=torch.int64, device=DEV).data_ptr(), 1,
                                  8, 8, 2, 64, 16, 1, None)
    assert st == 1  # PA_ERR_INVALID_ARG, nothing launched


def test_preemption_round_trip_keeps_the_decode():
    """Swap a sequence out, let other blocks overwrite its device blocks,
    swap it back into different blocks: the decode is bit-identical."""
    w = WORKLOADS[2]
    batch = make_batch(w, device=DEV, lens=np.array([700, 1500, 150]))  # pool has 10% spare blocks
    bt = batch.block_tables.copy()
    cl = torch.from_numpy(batch.context_lens).to(DEV)

    def dec(tables):
        return pk.decode(batch.q, batch.k_pool, batch.v_pool, torch.from_numpy(tables).to(DEV),
                         cl, batch.max_context_len, batch.scale, partition_size=0)
    before = dec(bt).clone()
    blocks = bt[2][bt[2] >= 0]                 # the short sequence is preempted
    n = len(blocks)
    kh, vh = _pinned_like(batch.k_pool, n), _pinned_like(batch.v_pool, n)
    out_pairs = np.stack([blocks, np.arange(n)], axis=1).astype(np.int64)
    pk.swap_blocks(kh, vh, batch.k_pool, batch.v_pool, torch.from_numpy(out_pairs).to(DEV))
    # the freed device blocks get other data (sequence 0's first blocks copied over them)
    src = np.resize(bt[0][bt[0] >= 0], n)
    pk.copy_blocks(batch.k_pool, batch.v_pool,
                   torch.from_numpy(np.stack([src, blocks], axis=1).astype(np.int64)).to(DEV))
    # back into blocks nobody uses
    used = set(int(x) for x in bt[bt >= 0])
    free = np.array([i for i in range(batch.num_blocks) if i not in used][:n], np.int64)
    assert len(free) == n
    in_pairs = np.stack([np.arange(n), free], axis=1).astype(np.int64)
    pk.swap_blocks(batch.k_pool, batch.v_pool, kh, vh, torch.from_numpy(in_pairs).to(DEV))
    bt2 = bt.copy()
    bt2[2, :n] = free
    after = dec(bt2)
    torch.cuda.synchronize()
    assert torch.equal(after.view(torch.int16), before.view(torch.int16))
