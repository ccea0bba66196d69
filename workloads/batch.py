"""Seeded synthetic decode batches shaped like the pages' examples.

This module draws inputs and lays out blocks; it computes nothing of the
method itself.  Both sides of every parity check read the tensors it
returns: the HIP library through device pointers, the oracle through host
copies.

Recipe (one batch = one layer's decode step):

* ``context_lens[b]`` = tokens the decode attends to.  The first
  ``L_b - 1`` are already cached; token ``L_b - 1`` is the new token, whose
  K/V rows (``k_new``, ``v_new``) the step appends with a cache write to
  ``slot_mapping[b]`` before attending.  Capacity is therefore
  ``ceil(L_b / B)`` blocks per sequence, the running-sequence block count of
  the scheduler sketch in "How LLM Inference Engines Work" (cached tokens
  plus one).
* Block ids come from ``BlockManager`` whose free list is a seeded
  permutation of the pool, so each sequence's blocks are scattered.
* q, K, V and the new rows are N(0, 1) drawn in float32 from a seeded
  torch generator on the target device, then rounded to the storage type
  (round-to-nearest-even).  An FP8 cache holds E4M3FN (or E5M2) codes of
  ``x / scale_h`` with ``scale_h = absmax_h / fmax`` per KV head (absmax
  over that head's pool data and new rows; fmax = 448 for E4M3FN, 57344
  for E5M2), made with torch's float8 cast.
* An INT4 cache is drawn directly in its storage: every code byte uniform
  over 0..255 (so every 4-bit pattern, -8..7, occurs) and one float32 scale
  per (block, KV head, token) for K and for V, uniform in [0.25, 0.5); no
  quantisation happens here.  New rows are N(0, 1) bf16 like the others.
* ``poison=True`` fills every slot that holds no valid token -- unused
  blocks, the tail of each last block, and the new token's slot before
  the write -- with NaN (code 0x7F in both FP8 formats; a NaN scale for
  INT4), so a kernel that reads past a context length produces NaN.
* The unused table entries are -1.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np
import torch

from .allocator import BlockManager, Sequence

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16,
               "fp8_e4m3": torch.uint8, "fp8_e5m2": torch.uint8, "int4": torch.uint8}
# the largest finite value of each FP8 format (the per-head scale maps absmax there)
FP8_FORMATS = {"fp8_e4m3": (torch.float8_e4m3fn, 448.0), "fp8_e5m2": (torch.float8_e5m2, 57344.0)}


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    cache_dtype: str
    q_dtype: str
    lens: tuple            # ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi)
                           # | ("fixed", n) | ("prefix", prefix, lo, hi)
    pool: str              # "fixed:N" | "plus10" | "exact"
    partition_size: int    # context split the workload is quoted with (0 = library choice)
    description: str

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def src_dtype(self) -> str:
        return "f32" if self.cache_dtype == "f32" else "bf16"

    @property
    def seed(self) -> int:
        return 253 * 10 + self.index


WORKLOADS = {
    1: Workload(1, "tiny-mha-f32", 4, 8, 8, 64, 16, "f32", "f32",
                ("uniform", 1, 200), "fixed:64", 0,
                "Tiny MHA paged decode, fp32: 4 sequences, 8 query heads = 8 KV "
                "heads, head_dim 64, block_size 16, lengths U[1,200], pool of 64 "
                "blocks in seeded random order"),
    2: Workload(2, "llama3-8b-decode-bf16", 64, 32, 8, 128, 16, "bf16", "bf16",
                ("uniform", 512, 4096), "plus10", 0,
                "Llama-3-8B-shaped single-layer decode, bf16 KV: batch 64, 32 "
                "query heads, 8 KV heads (group 4), head_dim 128, block_size 16, "
                "lengths U[512,4096], pool = blocks needed + 10%, shuffled"),
    3: Workload(3, "llama3-70b-decode-bf16", 256, 64, 8, 128, 16, "bf16", "bf16",
                ("lognormal", 1024, 1.0, 16, 32768), "exact", 0,
                "Llama-3-70B-shaped single-layer decode, bf16 KV: batch 256, 64 "
                "query heads, 8 KV heads (group 8), head_dim 128, block_size 16, "
                "lengths lognormal(median 1024, sigma 1) clipped to [16,32768]"),
    4: Workload(4, "shared-prefix-mha-bf16", 32, 64, 64, 128, 16, "bf16", "bf16",
                ("prefix", 2048, 1, 2048), "exact", 0,
                "Shared-prefix MHA decode, bf16: 32 sequences whose first 2048 "
                "tokens map to the same 128 physical blocks, each followed by a "
                "private suffix of U[1,2048] tokens; 64 heads, head_dim 128"),
    5: Workload(5, "long-context-fp8", 8, 32, 8, 128, 32, "fp8_e4m3", "bf16",
                ("fixed", 131072), "exact", 512,
                "Long-context decode with an fp8 e4m3 KV cache: batch 8, 32 query "
                "heads, 8 KV heads, head_dim 128, block_size 32, 131072 tokens "
                "each, per-KV-head fp32 scales, 512-token context partitions"),
}


# Several query tokens per sequence (chunked prefill, speculative verify):
# the batch shape and the query tokens per sequence.  Speculative
# verification checks the pages' 5 drafted tokens on the 8B-shaped batch;
# chunked prefill feeds 512-token chunks (the pages' example size) at 8K
# context for 8 sequences.
PREFILL_WORKLOADS = {
    "spec-verify-8b": (WORKLOADS[2], 5),
    "chunked-prefill-8b": (Workload(6, "chunked-prefill-bf16", 8, 32, 8, 128, 16, "bf16", "bf16",
                                    ("fixed", 8192), "exact", 0,
                                    "Chunked prefill: 8 sequences at 8192 cached tokens whose "
                                    "last 512 are the new chunk; Llama-3-8B heads (32/8, d 128), "
                                    "bf16 KV, block 16"), 512),
    "chunked-prefill-8b-fp8": (Workload(7, "chunked-prefill-fp8", 8, 32, 8, 128, 16, "fp8_e4m3",
                                        "bf16", ("fixed", 8192), "exact", 0,
                                        "Chunked prefill as chunked-prefill-8b with an fp8 e4m3 "
                                        "KV cache (per-KV-head fp32 scales)"), 512),
}


@dataclass
class Batch:
    workload: Workload
    seed: int
    context_lens: np.ndarray          # int32 [S]
    block_tables: np.ndarray          # int32 [S, max_blocks], -1 padded
    slot_mapping: np.ndarray          # int64 [S], slot of each new token
    ref_counts: np.ndarray            # int32 [num_blocks]
    q: torch.Tensor                   # [S, Hq, d] q dtype
    k_pool: torch.Tensor              # [nb, Hkv, d/x, B, x] cache storage, x = 16 B / elt
    v_pool: torch.Tensor              # [nb, Hkv, d, B] cache storage
                                      # (INT4: both uint8 [nb, Hkv, B * (d/2 + 4)] tiles)
    k_new: torch.Tensor               # [S, Hkv, d] source dtype
    v_new: torch.Tensor
    k_scale: torch.Tensor | None      # float32 [Hkv] (FP8 cache only)
    v_scale: torch.Tensor | None
    extra: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.workload.head_dim)

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if len(self.context_lens) else 0

    def replace(self, **kw) -> "Batch":
        return dataclasses.replace(self, **kw)


# --------------------------------------------------------------------------
# drawing
# --------------------------------------------------------------------------

def draw_lens(w: Workload, rng: np.random.Generator, num_seqs: int) -> np.ndarray:
    kind = w.lens[0]
    if kind == "uniform":
        lens = rng.integers(w.lens[1], w.lens[2] + 1, size=num_seqs)
    elif kind == "lognormal":
        med, sigma, lo, hi = w.lens[1:]
        x = np.exp(np.log(med) + sigma * rng.standard_normal(num_seqs))
        lens = np.clip(np.rint(x), lo, hi)
    elif kind == "fixed":
        lens = np.full(num_seqs, w.lens[1])
    elif kind == "prefix":
        prefix, lo, hi = w.lens[1:]
        lens = prefix + rng.integers(lo, hi + 1, size=num_seqs)
    else:
        raise ValueError(kind)
    return lens.astype(np.int32)


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _store(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x.to(TORCH_DTYPE[dtype]) if dtype not in FP8_FORMATS else x


def chunk_k_pool(k: torch.Tensor) -> torch.Tensor:
    """Token-major ``[nb, Hkv, B, d]`` K storage -> the pool's chunked layout
    ``[nb, Hkv, d/x, B, x]`` (x elements = 16 bytes).  Moves elements only."""
    nb, hkv, bsz, d = k.shape
    x = 16 // k.element_size()
    return k.view(nb, hkv, bsz, d // x, x).permute(0, 1, 3, 2, 4).contiguous()


def make_batch(w: Workload, seed: int | None = None, device="cpu",
               num_seqs: int | None = None, lens: np.ndarray | None = None,
               poison: bool = False) -> Batch:
    """Draw one batch of workload ``w`` (optionally fewer sequences or given
    lengths, for small CPU-side cases of the same shape)."""
    seed = w.seed if seed is None else int(seed)
    rng = np.random.default_rng(seed)
    s_count = w.num_seqs if num_seqs is None else int(num_seqs)
    if lens is None:
        lens = draw_lens(w, rng, s_count)
    lens = np.asarray(lens, dtype=np.int32)
    s_count = len(lens)
    bsz = w.block_size
    need = -(-lens.astype(np.int64) // bsz)

    shared_blocks = 0
    if w.lens[0] == "prefix":
        shared_blocks = w.lens[1] // bsz
        if np.any(lens <= w.lens[1]):
            raise ValueError("prefix workload needs a private suffix")
        total = shared_blocks + int((need - shared_blocks).sum())
    else:
        total = int(need.sum())
    if w.pool.startswith("fixed:"):
        num_blocks = int(w.pool.split(":")[1])
        if num_blocks < total:
            raise ValueError("fixed pool too small for the drawn lengths")
    elif w.pool == "plus10":
        num_blocks = int(math.ceil(1.1 * total))
    else:
        num_blocks = total

    mgr = BlockManager(num_blocks, bsz, order=rng.permutation(num_blocks))
    seqs = [Sequence(f"seq{b}") for b in range(s_count)]
    if shared_blocks:
        owner = Sequence("prefix")
        for _ in range(shared_blocks):
            assert mgr.allocate(owner)
        for s in seqs:
            mgr.share(owner, s, shared_blocks)
        mgr.free(owner)  # the prompt owner leaves; its sequences keep the blocks
    for s, n in zip(seqs, lens):
        if not mgr.allocate_tokens(s, int(n)):
            raise RuntimeError("pool exhausted while building the batch")
    max_blocks = max(1, int(need.max()) if s_count else 1)
    tables = np.full((s_count, max_blocks), -1, dtype=np.int32)
    for b, s in enumerate(seqs):
        tables[b, :len(s.blocks)] = s.blocks
    refs = np.array([mgr.ref_count(i) for i in range(num_blocks)], dtype=np.int32)
    new_pos = lens.astype(np.int64) - 1
    slot_mapping = np.array(
        [tables[b, p // bsz] * bsz + p % bsz if p >= 0 else -1 for b, p in enumerate(new_pos)],
        dtype=np.int64)  # an empty context has no new token

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    hkv, hq, d = w.num_kv_heads, w.num_q_heads, w.head_dim
    q = _randn((s_count, hq, d), gen, device)
    if w.cache_dtype == "int4":
        return _int4_batch(w, seed, lens, tables, slot_mapping, refs, q, gen, device,
                           num_blocks, poison)
    k32 = _randn((num_blocks, hkv, bsz, d), gen, device)
    v32 = _randn((num_blocks, hkv, d, bsz), gen, device)
    kn = _randn((s_count, hkv, d), gen, device)
    vn = _randn((s_count, hkv, d), gen, device)
    q = q.to(TORCH_DTYPE[w.q_dtype])
    kn = kn.to(TORCH_DTYPE[w.src_dtype])
    vn = vn.to(TORCH_DTYPE[w.src_dtype])
    k_scale = v_scale = None
    if w.cache_dtype in FP8_FORMATS:
        fmt, fmax = FP8_FORMATS[w.cache_dtype]
        kabs = torch.maximum(k32.abs().amax(dim=(0, 2, 3)),
                             kn.float().abs().amax(dim=(0, 2)))
        vabs = torch.maximum(v32.abs().amax(dim=(0, 2, 3)),
                             vn.float().abs().amax(dim=(0, 2)))
        k_scale = (kabs / fmax).to(torch.float32)
        v_scale = (vabs / fmax).to(torch.float32)
        k_pool = (k32 / k_scale[None, :, None, None]).to(fmt).view(torch.uint8)
        v_pool = (v32 / v_scale[None, :, None, None]).to(fmt).view(torch.uint8)
        del k32, v32
    else:
        k_pool = k32.to(TORCH_DTYPE[w.cache_dtype])
        v_pool = v32.to(TORCH_DTYPE[w.cache_dtype])
        del k32, v32

    if poison:
        bad = _invalid_slots(lens, tables, num_blocks, bsz, device)
        if w.cache_dtype in FP8_FORMATS:  # 0x7F is NaN in both formats
            k_pool.masked_fill_(bad[:, None, :, None], 0x7F)
            v_pool.masked_fill_(bad[:, None, None, :], 0x7F)
        else:
            k_pool.masked_fill_(bad[:, None, :, None], float("nan"))
            v_pool.masked_fill_(bad[:, None, None, :], float("nan"))

    return Batch(w, seed, lens, tables, slot_mapping, refs, q.contiguous(),
                 chunk_k_pool(k_pool), v_pool.contiguous(), kn.contiguous(),
                 vn.contiguous(), k_scale, v_scale,
                 {"shared_blocks": shared_blocks, "poison": poison})


def _invalid_slots(lens, tables, num_blocks, bsz, device) -> torch.Tensor:
    """[num_blocks, B] bool: slots that hold no cached token of any sequence
    (the new token's slot counts as empty before the write)."""
    valid = np.zeros((num_blocks, bsz), dtype=bool)
    for b in range(len(lens)):
        pos = np.arange(int(lens[b]) - 1)  # cached tokens, new token excluded
        valid[tables[b, pos // bsz], pos % bsz] = True
    return torch.from_numpy(~valid).to(device)


def _int4_batch(w, seed, lens, tables, slot_mapping, refs, q, gen, device, num_blocks,
                poison) -> Batch:
    """INT4 pools drawn in storage form: random code bytes, then per-token
    float32 scales at the end of each (block, head) tile."""
    hkv, d, bsz = w.num_kv_heads, w.head_dim, w.block_size
    pools = []
    for _ in range(2):  # K, then V
        codes = torch.randint(0, 256, (num_blocks, hkv, bsz * d // 2), generator=gen,
                              device=device, dtype=torch.uint8)
        scales = 0.25 + 0.25 * torch.rand((num_blocks, hkv, bsz), generator=gen,
                                          device=device, dtype=torch.float32)
        if poison:
            bad = _invalid_slots(lens, tables, num_blocks, bsz, device)
            scales.masked_fill_(bad[:, None, :], float("nan"))
        pools.append(torch.cat([codes, scales.view(torch.uint8)], dim=2).contiguous())
    kn = _randn((len(lens), hkv, d), gen, device).to(TORCH_DTYPE[w.src_dtype])
    vn = _randn((len(lens), hkv, d), gen, device).to(TORCH_DTYPE[w.src_dtype])
    return Batch(w, seed, lens, tables, slot_mapping, refs,
                 q.to(TORCH_DTYPE[w.q_dtype]).contiguous(), pools[0], pools[1],
                 kn.contiguous(), vn.contiguous(), None, None,
                 {"shared_blocks": 0, "poison": poison})


# --------------------------------------------------------------------------
# block-level relayouts (whole blocks move; nothing inside a block changes)
# --------------------------------------------------------------------------

def _map_tables(tables: np.ndarray, new_id: np.ndarray) -> np.ndarray:
    out = tables.copy()
    live = out >= 0
    out[live] = new_id[out[live]]
    return out


def permute_blocks(batch: Batch, perm: np.ndarray) -> Batch:
    """Relabel physical block i as ``perm[i]``, moving its contents along."""
    perm = np.asarray(perm, dtype=np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    idx = torch.from_numpy(inv).to(batch.k_pool.device)
    bsz = batch.workload.block_size
    new_tables = _map_tables(batch.block_tables, perm)
    slot = batch.slot_mapping
    new_slot = perm[slot // bsz] * bsz + slot % bsz
    refs = batch.ref_counts[inv]
    return batch.replace(block_tables=new_tables.astype(np.int32),
                         slot_mapping=new_slot.astype(np.int64),
                         ref_counts=refs,
                         k_pool=batch.k_pool.index_select(0, idx).contiguous(),
                         v_pool=batch.v_pool.index_select(0, idx).contiguous())


def unshare(batch: Batch) -> Batch:
    """Give every sequence private copies of blocks it shares with others."""
    refs = batch.ref_counts
    tables = batch.block_tables.copy()
    src = list(range(batch.num_blocks))
    for b in range(tables.shape[0]):
        for i in range(tables.shape[1]):
            blk = int(tables[b, i])
            if blk >= 0 and refs[blk] > 1:
                tables[b, i] = len(src)
                src.append(blk)
    idx = torch.tensor(src, dtype=torch.int64, device=batch.k_pool.device)
    new_refs = np.zeros(len(src), dtype=np.int32)
    for blk in tables[tables >= 0]:
        new_refs[blk] += 1
    return batch.replace(block_tables=tables, ref_counts=new_refs,
                         k_pool=batch.k_pool.index_select(0, idx).contiguous(),
                         v_pool=batch.v_pool.index_select(0, idx).contiguous())


def contiguous_layout(batch: Batch) -> Batch:
    """Renumber blocks so each sequence's blocks are consecutive ids in
    sequence order (the unpaged layout, up to block padding).  Requires an
    unshared batch."""
    if np.any(batch.ref_counts > 1):
        raise ValueError("unshare the batch first")
    order = [int(x) for x in batch.block_tables.reshape(-1) if x >= 0]
    used = set(order)
    rest = [i for i in range(batch.num_blocks) if i not in used]
    old_order = np.array(order + rest, dtype=np.int64)
    perm = np.empty(batch.num_blocks, dtype=np.int64)
    perm[old_order] = np.arange(batch.num_blocks)
    return permute_blocks(batch, perm)


def host_view(t: torch.Tensor) -> np.ndarray:
    """Raw host copy of a storage tensor (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def extract_sequences(batch: Batch, seqs) -> dict:
    """Host copy of just the blocks ``seqs`` use, with remapped tables.

    For checking a few sequences of a full-size batch on the CPU without
    copying the whole pool.
    """
    seqs = list(seqs)
    used = sorted({int(x) for b in seqs for x in batch.block_tables[b] if x >= 0})
    new_id = np.full(batch.num_blocks, -1, dtype=np.int64)
    new_id[used] = np.arange(len(used))
    idx = torch.tensor(used, dtype=torch.int64, device=batch.k_pool.device)
    tables = _map_tables(batch.block_tables[seqs], new_id).astype(np.int32)
    out = {
        "seqs": seqs,
        "k_pool": host_view(batch.k_pool.index_select(0, idx)),
        "v_pool": host_view(batch.v_pool.index_select(0, idx)),
        "block_tables": tables,
        "context_lens": batch.context_lens[seqs].copy(),
        "q": host_view(batch.q[seqs]),
        "k_scale": None if batch.k_scale is None else batch.k_scale.cpu().numpy(),
        "v_scale": None if batch.v_scale is None else batch.v_scale.cpu().numpy(),
    }
    return out
