"""Copy-on-write block copy on the GPU (``pa_copy_blocks``) against the
oracle's copy, bit for bit, and the whole copy-on-write flow: host fork,
device copy, device append, device decode."""

import numpy as np
import pytest
import torch

import paged_kv_cache_253_amd as pk
from oracle import paged
from tests.parity import compare, same_bits
from workloads import BlockManager, Sequence, chunk_k_pool, host_view

pytestmark = pytest.mark.gpu
DEV = "cuda"

TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}


def _random_pools(nb, hkv, d, bsz, dtype, seed):
    """Pools of random bit patterns (NaNs included) in the library layout."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    nbytes = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[dtype]
    k = torch.randint(0, 256, (nb, hkv, bsz, d * nbytes), generator=g, dtype=torch.uint8)
    v = torch.randint(0, 256, (nb, hkv, d * nbytes, bsz), generator=g, dtype=torch.uint8)
    if dtype != "fp8_e4m3":
        k = k.view(TORCH[dtype])
        v = v.view(nb, hkv, d, nbytes, bsz).permute(0, 1, 2, 4, 3).contiguous().view(TORCH[dtype])
        v = v.view(nb, hkv, d, bsz)
    return chunk_k_pool(k.contiguous()), v.contiguous()


def _independent_pairs(nb, n, rng):
    ids = rng.permutation(nb)[:2 * n]
    return np.stack([ids[:n], ids[n:]], axis=1).astype(np.int64)


@pytest.mark.parametrize("dtype,hkv,d,bsz,npairs", [
    ("bf16", 8, 128, 16, 37),
    ("fp8_e4m3", 1, 64, 16, 5),      # 1 KiB blocks: less than one 4 KiB chunk
    ("fp8_e4m3", 8, 128, 32, 64),
    ("f32", 4, 64, 32, 9),
    ("f32", 64, 128, 16, 3),         # 512 KiB blocks
    ("bf16", 2, 64, 16, 0),
])
def test_copy_blocks_bit_exact(dtype, hkv, d, bsz, npairs):
    print(f"[copy] {dtype} hkv={hkv} d={d} B={bsz} pairs={npairs}", flush=True)
    nb = max(2 * npairs + 3, 8)
    k, v = _random_pools(nb, hkv, d, bsz, dtype, seed=hkv * 1000 + d + bsz + npairs)
    rng = np.random.default_rng(npairs + 7)
    pairs = _independent_pairs(nb, npairs, rng)
    k_ref, v_ref = paged.copy_blocks(host_view(k), host_view(v), pairs)
    kd, vd = k.to(DEV), v.to(DEV)
    pk.copy_blocks(kd, vd, torch.from_numpy(pairs.reshape(-1, 2)).to(DEV))
    torch.cuda.synchronize()
    assert same_bits(host_view(kd), k_ref)
    assert same_bits(host_view(vd), v_ref)


def test_copy_blocks_skips_out_of_range_pairs():
    nb, hkv, d, bsz = 12, 8, 128, 16
    k, v = _random_pools(nb, hkv, d, bsz, "bf16", seed=3)
    pairs = np.array([[2, 5], [-1, 6], [3, nb], [nb + 4, 7], [8, -2], [9, 10]], np.int64)
    k_ref, v_ref = paged.copy_blocks(host_view(k), host_view(v), pairs[[0, 5]])
    kd, vd = k.to(DEV), v.to(DEV)
    pk.copy_blocks(kd, vd, torch.from_numpy(pairs).to(DEV))
    torch.cuda.synchronize()
    assert same_bits(host_view(kd), k_ref) and same_bits(host_view(vd), v_ref)


@pytest.mark.parametrize("prefix", [37, 48, 5])
def test_copy_on_write_flow(prefix):
    """Sequences share a prompt whose last block is partly filled (or full,
    for prefix 48).  Each appends its own token: the block manager forks the
    shared block where needed, pa_copy_blocks copies it, pa_kv_cache_write
    appends, pa_decode attends -- against the oracle running the same steps."""
    print(f"[cow] prefix={prefix}", flush=True)
    hkv, g, d, bsz, nb, n = 8, 4, 128, 16, 64, 5
    torch.manual_seed(prefix)
    k32 = torch.randn(nb, hkv, bsz, d)
    v32 = torch.randn(nb, hkv, d, bsz)
    k_pool = chunk_k_pool(k32.to(torch.bfloat16))
    v_pool = v32.to(torch.bfloat16).contiguous()
    q = torch.randn(n, hkv * g, d).to(torch.bfloat16)
    kn = torch.randn(n, hkv, d).to(torch.bfloat16)
    vn = torch.randn(n, hkv, d).to(torch.bfloat16)

    mgr = BlockManager(nb, bsz, order=np.random.default_rng(prefix).permutation(nb))
    parent = Sequence("prompt")
    assert mgr.allocate_tokens(parent, prefix)
    kids = [Sequence(f"s{i}") for i in range(n)]
    for s in kids:
        mgr.share(parent, s, len(parent.blocks))
    mgr.free(parent)
    pairs, slots = [], []
    for s in kids:
        if prefix % bsz == 0:
            assert mgr.allocate(s)              # the prompt filled its last block
        else:
            fork = mgr.fork_for_append(s, prefix)
            assert fork is not False
            if fork is not None:
                pairs.append(fork)
        slots.append(s.blocks[prefix // bsz] * bsz + prefix % bsz)
    assert len(pairs) == (n - 1 if prefix % bsz else 0)  # the last holder writes in place
    max_blocks = max(len(s.blocks) for s in kids)
    tables = np.full((n, max_blocks), -1, np.int32)
    for i, s in enumerate(kids):
        tables[i, :len(s.blocks)] = s.blocks
    lens = np.full(n, prefix + 1, np.int32)
    slots = np.array(slots, np.int64)
    pairs = np.array(pairs, np.int64).reshape(-1, 2)

    # oracle: copy, append, decode on host copies
    kh, vh = paged.copy_blocks(host_view(k_pool), host_view(v_pool), pairs)
    kh, vh = paged.write_tokens(kh, vh, host_view(kn), host_view(vn), slots, bsz, "bf16", "bf16")
    scale = 1.0 / np.sqrt(d)
    ref = paged.decode(host_view(q), kh, vh, tables, lens, bsz, scale, "bf16", "bf16")

    kd, vd = k_pool.to(DEV), v_pool.to(DEV)
    if len(pairs):
        pk.copy_blocks(kd, vd, torch.from_numpy(pairs).to(DEV))
    pk.kv_cache_write(kn.to(DEV), vn.to(DEV), kd, vd, torch.from_numpy(slots).to(DEV))
    out = pk.decode(q.to(DEV), kd, vd, torch.from_numpy(tables).to(DEV),
                    torch.from_numpy(lens).to(DEV), int(lens.max()), scale)
    torch.cuda.synchronize()
    assert same_bits(host_view(kd), kh) and same_bits(host_view(vd), vh)
    compare(out.float().cpu().numpy().astype(np.float64), ref, "bf16", f"cow prefix {prefix}")
