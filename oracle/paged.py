"""Paged KV cache and decode attention, written as plain definitions.

TEST INFRASTRUCTURE ONLY (oracle): see the package docstring for who may
import this.  No blocking, fusion or reordering beyond the definitions.

Pool layout (the library's documented layout, restated here from its
definition, not shared with it):

* K pool: ``[num_blocks, num_kv_heads, head_dim // x, block_size, x]`` with
  ``x = 16 / element bytes`` (4 f32, 8 bf16, 16 E4M3) -- inside a (block,
  head) tile the head dimension is cut into 16-byte chunks, and each chunk
  row holds that chunk of every token of the block, token-major.  Token
  ``j``'s K row is ``pool[blk, h, :, j, :]`` read chunk by chunk.
* V pool: ``[num_blocks, num_kv_heads, head_dim, block_size]`` -- inside a
  (block, head) tile, dimension-major rows of ``block_size`` tokens.

Storage is raw: ``"f32"`` arrays are float32, ``"bf16"`` arrays hold
bfloat16 bit patterns as uint16, ``"fp8_e4m3"`` / ``"fp8_e5m2"`` arrays hold FP8 codes as
uint8 with one float32 scale per KV head.

An ``"int4"`` pool is uint8 ``[num_blocks, num_kv_heads, B * (d/2 + 4)]``:
each (block, head) tile is its 4-bit codes (``B * d / 2`` bytes) followed
by ``B`` float32 scales, token j's at byte ``B*d/2 + 4j``.  Codes are
grouped in octets of 8 consecutive elements in 4 bytes; byte i of an octet
holds element i in its low nibble and element i + 4 in its high nibble
(two's complement).  K codes keep the chunked layout with x = 32 elements
(16 bytes): ``[d/32, B, 16 bytes]``, a token's 32-element chunk being 4
octets of consecutive dimensions.  V codes are ``[d, B/2 bytes]``: row
``dim`` holds the block's tokens, in octets of consecutive tokens.

Token t of a sequence lives in physical block ``table[t // B]`` at offset
``t % B`` ("vLLM & High-Throughput Serving", section 2, block-table
equation; "AI Inference Serving at Scale", section 3, logical-to-physical
block table).
"""

from __future__ import annotations

import numpy as np

from . import codecs

DTYPES = ("f32", "bf16", "fp8_e4m3", "fp8_e5m2", "int4")
FP8 = ("fp8_e4m3", "fp8_e5m2")
INT4 = "int4"


# --------------------------------------------------------------------------
# element storage
# --------------------------------------------------------------------------

def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Widen raw storage of ``dtype`` to float64 (exact for all three)."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return codecs.bf16_bits_to_f64(raw)
    if dtype == "fp8_e4m3":
        return codecs.e4m3_to_f64(raw)
    if dtype == "fp8_e5m2":
        return codecs.e5m2_to_f64(raw)
    raise ValueError(f"unknown dtype {dtype!r}")


def source_to_f32(raw: np.ndarray, dtype: str) -> np.ndarray:
    """New K/V rows arrive as f32 or bf16; both are exact in float32."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32)
    if dtype == "bf16":
        return codecs.bf16_bits_to_f64(raw).astype(np.float32)
    raise ValueError(f"new K/V rows must be f32 or bf16, not {dtype!r}")


# --------------------------------------------------------------------------
# K rows in the chunked K pool
# --------------------------------------------------------------------------

def k_row(k_pool: np.ndarray, blk: int, h: int, off: int) -> np.ndarray:
    """K row (``head_dim`` elements, raw storage) of the token at offset
    ``off`` of block ``blk``, KV head ``h``: its chunks in order."""
    return k_pool[blk, h, :, off, :].reshape(-1)


def set_k_row(k_pool: np.ndarray, blk: int, h: int, off: int, row: np.ndarray) -> None:
    """Store one K row (``head_dim`` elements) at (``blk``, ``h``, ``off``)."""
    n_chunks, x = k_pool.shape[2], k_pool.shape[4]
    k_pool[blk, h, :, off, :] = np.asarray(row).reshape(n_chunks, x)


def k_head_dim(k_pool: np.ndarray, block_size: int | None = None) -> int:
    if k_pool.ndim == 3:  # INT4 tiles: B * (d/2 + 4) bytes
        return int_tile_head_dim(k_pool.shape[2], block_size)
    return int(k_pool.shape[2] * k_pool.shape[4])


# --------------------------------------------------------------------------
# INT4 tiles (codes in octets, then one float32 scale per token)
# --------------------------------------------------------------------------

def int_tile_head_dim(tile_bytes: int, block_size: int) -> int:
    """head_dim of an INT4 tile of ``tile_bytes`` = B * (d/2 + 4)."""
    if block_size is None or tile_bytes % block_size:
        raise ValueError("INT4 tiles need the block size")
    return 2 * (tile_bytes // block_size - 4)


def int4_tile_bytes(head_dim: int, block_size: int) -> int:
    return block_size * (head_dim // 2 + 4)


def unpack_octets(b: np.ndarray) -> np.ndarray:
    """Bytes ``[..., 4k]`` -> INT4 codes ``[..., 8k]``: byte i of each group
    of 4 holds element i (low nibble) and element i + 4 (high nibble)."""
    b = np.asarray(b, dtype=np.uint8)
    g = b.reshape(b.shape[:-1] + (-1, 4))
    lo = codecs.nibble_to_int4(g & 0xF)
    hi = codecs.nibble_to_int4(g >> 4)
    return np.concatenate([lo, hi], axis=-1).reshape(b.shape[:-1] + (-1,))


def pack_octets(c: np.ndarray) -> np.ndarray:
    """Inverse of ``unpack_octets``: codes ``[..., 8k]`` -> bytes ``[..., 4k]``."""
    c = np.asarray(c)
    g = codecs.int4_to_nibble(c).reshape(c.shape[:-1] + (-1, 8))
    b = g[..., :4] | (g[..., 4:] << 4)
    return b.astype(np.uint8).reshape(c.shape[:-1] + (-1,))


def _int4_scale(tile: np.ndarray, head_dim: int, block_size: int, off: int) -> np.float32:
    at = block_size * head_dim // 2 + 4 * off
    return tile[at:at + 4].copy().view(np.float32)[0]


def _set_int4_scale(tile: np.ndarray, head_dim: int, block_size: int, off: int, s) -> None:
    at = block_size * head_dim // 2 + 4 * off
    tile[at:at + 4] = np.array([s], dtype=np.float32).view(np.uint8)


def int4_k_row(k_pool, blk, h, off, block_size):
    """K codes (``head_dim`` integers) and scale of one token of an INT4 pool."""
    tile = k_pool[blk, h]
    d = int_tile_head_dim(tile.shape[0], block_size)
    chunks = tile[:block_size * d // 2].reshape(d // 32, block_size, 16)
    return unpack_octets(chunks[:, off, :]).reshape(-1), _int4_scale(tile, d, block_size, off)


def int4_v_row(v_pool, blk, h, off, block_size):
    """V codes (``head_dim`` integers) and scale of one token of an INT4 pool."""
    tile = v_pool[blk, h]
    d = int_tile_head_dim(tile.shape[0], block_size)
    rows = unpack_octets(tile[:block_size * d // 2].reshape(d, block_size // 2))  # [d, B]
    return rows[:, off].copy(), _int4_scale(tile, d, block_size, off)


def set_int4_k_row(k_pool, blk, h, off, block_size, codes, scale) -> None:
    tile = k_pool[blk, h]
    d = int_tile_head_dim(tile.shape[0], block_size)
    chunks = tile[:block_size * d // 2].reshape(d // 32, block_size, 16)
    chunks[:, off, :] = pack_octets(np.asarray(codes).reshape(d // 32, 32))
    _set_int4_scale(tile, d, block_size, off, scale)


def set_int4_v_row(v_pool, blk, h, off, block_size, codes, scale) -> None:
    tile = v_pool[blk, h]
    d = int_tile_head_dim(tile.shape[0], block_size)
    region = tile[:block_size * d // 2].reshape(d, block_size // 2)
    rows = unpack_octets(region)
    rows[:, off] = codes
    region[:] = pack_octets(rows)
    _set_int4_scale(tile, d, block_size, off, scale)


# --------------------------------------------------------------------------
# block table: index map and gather
# --------------------------------------------------------------------------

def slot_of(table_row: np.ndarray, t: int, block_size: int) -> tuple[int, int]:
    """Physical (block, offset) of logical token ``t``.

    Logical block ``i = floor(t / B)`` and offset ``j = t mod B``
    ("vLLM & High-Throughput Serving", section 2, block-table equation);
    the block table maps ``i`` to a physical block id ("AI Inference
    Serving at Scale", section 3).
    """
    i, j = divmod(int(t), int(block_size))
    return int(table_row[i]), j


def gather(k_pool: np.ndarray, v_pool: np.ndarray, table_row: np.ndarray,
           length: int, block_size: int) -> tuple[np.ndarray, np.ndarray]:
    """Copy one sequence's K and V out of the pool into contiguous arrays.

    Returns raw-storage arrays ``[length, num_kv_heads, head_dim]`` in
    token order, the contiguous per-sequence layout of "vLLM &
    High-Throughput Serving", section 1.  The paged kernel gathers K and V
    from non-adjacent blocks ("How LLM Inference Engines Work", section on
    PagedAttention); here the gather is one token at a time.
    """
    n_kv, head_dim = k_pool.shape[1], k_head_dim(k_pool, block_size)
    k = np.empty((length, n_kv, head_dim), dtype=k_pool.dtype)
    v = np.empty((length, n_kv, head_dim), dtype=v_pool.dtype)
    for t in range(length):
        blk, off = slot_of(table_row, t, block_size)
        for h in range(n_kv):
            k[t, h] = k_row(k_pool, blk, h, off)
        v[t] = v_pool[blk, :, :, off]
    return k, v


# --------------------------------------------------------------------------
# append (cache write)
# --------------------------------------------------------------------------

def write_tokens(k_pool: np.ndarray, v_pool: np.ndarray,
                 k_new: np.ndarray, v_new: np.ndarray,
                 slot_mapping: np.ndarray, block_size: int,
                 src_dtype: str, cache_dtype: str,
                 k_scale: np.ndarray | None = None,
                 v_scale: np.ndarray | None = None
                 ) -> tuple[np.ndarray, np.ndarray]:
    """Store new tokens' K and V rows at their slots; return new pools.

    Token n goes to slot ``s = slot_mapping[n]``: block ``s // B``, offset
    ``s % B`` (the block-table equation of "vLLM & High-Throughput
    Serving", section 2, applied to a flat slot number).  The engine
    appends each generated token's K/V into the sequence's current block
    ("AI Inference Serving at Scale", section 3, on-demand allocation).
    A negative slot marks a padding token and is skipped.  Two tokens with
    the same slot are a caller error and raise.

    Same-type caches store the bits unchanged.  An E4M3 cache stores
    ``e4m3_encode(float32(x) / float32(scale[h]))`` per KV head h (E5M2:
    ``e5m2_encode``): the quotient rounded once in binary32, then rounded
    to nearest-even with saturation at the format's largest finite value
    (the pages give FP8 KV caches without a rounding rule; this is the
    plain reading).  An INT4 cache stores each row's ``int4_encode``: its
    codes and its own float32 scale, per token and KV head, for K and V
    separately (the scales arguments are not used).
    """
    slot_mapping = np.asarray(slot_mapping, dtype=np.int64)
    live = slot_mapping[slot_mapping >= 0]
    if len(np.unique(live)) != len(live):
        raise ValueError("duplicate slot in slot_mapping")
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    n_kv = k_pool.shape[1]
    for n, s in enumerate(slot_mapping):
        if s < 0:
            continue
        blk, off = divmod(int(s), int(block_size))
        for h in range(n_kv):
            if cache_dtype == INT4:
                kc, ks = codecs.int4_encode(source_to_f32(k_new[n, h], src_dtype))
                vc, vs = codecs.int4_encode(source_to_f32(v_new[n, h], src_dtype))
                set_int4_k_row(k_out, blk, h, off, block_size, kc, ks)
                set_int4_v_row(v_out, blk, h, off, block_size, vc, vs)
            elif cache_dtype in FP8:
                encode = codecs.e4m3_encode if cache_dtype == "fp8_e4m3" else codecs.e5m2_encode
                kx = source_to_f32(k_new[n, h], src_dtype)
                vx = source_to_f32(v_new[n, h], src_dtype)
                kq = kx / np.float32(k_scale[h])
                vq = vx / np.float32(v_scale[h])
                set_k_row(k_out, blk, h, off, encode(kq))
                v_out[blk, h, :, off] = encode(vq)
            else:
                if src_dtype != cache_dtype:
                    raise ValueError("non-fp8 caches store the source bits")
                set_k_row(k_out, blk, h, off, k_new[n, h])
                v_out[blk, h, :, off] = v_new[n, h]
    return k_out, v_out


# --------------------------------------------------------------------------
# copy-on-write block copy
# --------------------------------------------------------------------------

def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray,
                block_mapping: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Copy whole blocks, every KV head, for each (src, dst) pair; return
    new pools.

    When a sequence is about to write into a block other sequences share,
    it gets a private copy of that one block ("AI Inference Serving at
    Scale", section 3, copy-on-write sharing; "vLLM & High-Throughput
    Serving", copy-on-write prefix caching).  The pairs must be
    independent: distinct destinations, none of them also a source (else
    the result would depend on the order); a violation raises.
    """
    pairs = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    dst = pairs[:, 1]
    if len(np.unique(dst)) != len(dst) or np.isin(dst, pairs[:, 0]).any():
        raise ValueError("copy pairs must have distinct destinations that are not sources")
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for src, d in pairs:
        k_out[d] = k_pool[src]
        v_out[d] = v_pool[src]
    return k_out, v_out


def swap_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray,
                dst_v: np.ndarray, block_mapping: np.ndarray
                ) -> tuple[np.ndarray, np.ndarray]:
    """Copy whole blocks from one pair of pools to another; return the new
    destination pools.

    The scheduler preempts a sequence by swapping its blocks out to CPU
    memory and later back ("How LLM Inference Engines Work", the
    scheduler).  For each (src, dst) pair, block src of the source pools
    (every KV head) becomes block dst of the destination pools.
    Destinations must be distinct (else the result would depend on the
    order); a violation raises.
    """
    pairs = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    if len(np.unique(pairs[:, 1])) != len(pairs):
        raise ValueError("swap pairs must have distinct destinations")
    k_out = dst_k.copy()
    v_out = dst_v.copy()
    for s_, d in pairs:
        k_out[d] = src_k[s_]
        v_out[d] = src_v[s_]
    return k_out, v_out


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
              scale: float) -> np.ndarray:
    """Textbook single-query attention of one sequence, in float64.

    ``q``: ``[Hq, d]``; ``k``, ``v``: ``[L, Hkv, d]`` (contiguous).
    Query head ``hq`` uses KV head ``hq // (Hq / Hkv)``: consecutive query
    heads share one KV head (grouped-query attention, "AI Inference
    Serving at Scale", section 6).  For each query head the weights are
    ``softmax(scale * K q)`` over all L cached tokens and the output is the
    weighted sum of the V rows (dot-product attention against all preceding
    tokens, same page, section 2).  The maximum is subtracted before exp,
    which leaves the softmax unchanged.  An empty context gives zeros.
    """
    n_q, d = q.shape
    length, n_kv, _ = k.shape
    group = n_q // n_kv
    out = np.zeros((n_q, d), dtype=np.float64)
    if length == 0:
        return out
    for hq in range(n_q):
        h = hq // group
        z = scale * (k[:, h, :] @ q[hq])
        e = np.exp(z - z.max())
        p = e / e.sum()
        out[hq] = p @ v[:, h, :]
    return out


def int4_block_values(tiles: np.ndarray, block_size: int, which: str) -> np.ndarray:
    """Values of every token of one block of an INT4 pool, all KV heads:
    ``tiles`` is ``pool[blk]`` (``[Hkv, T]`` bytes); returns float64
    ``[B, Hkv, head_dim]``, code times its token's scale.  ``which`` is
    "k" (chunked K codes) or "v" (dimension-major V codes)."""
    n_kv, tile = tiles.shape
    d = int_tile_head_dim(tile, block_size)
    code_bytes = block_size * d // 2
    scales = tiles[:, code_bytes:].copy().view(np.float32).astype(np.float64)  # [Hkv, B]
    region = tiles[:, :code_bytes]
    if which == "k":
        c = unpack_octets(region.reshape(n_kv, d // 32, block_size, 16))  # [Hkv, d/32, B, 32]
        c = c.transpose(2, 0, 1, 3).reshape(block_size, n_kv, d)
    else:
        c = unpack_octets(region.reshape(n_kv, d, block_size // 2))         # [Hkv, d, B]
        c = c.transpose(2, 0, 1)
    return c.astype(np.float64) * scales.T[:, :, None]


def gather_int4_f64(k_pool, v_pool, table_row, length, block_size):
    """One sequence of an INT4 pool, gathered through its block table and
    decoded (code times its token's scale) to float64 ``[length,
    num_kv_heads, head_dim]``: logical block i is physical block
    ``table_row[i]``, token t its offset ``t mod B``."""
    n_blocks = -(-int(length) // int(block_size))
    ks, vs = [], []
    for i in range(n_blocks):
        blk = int(table_row[i])
        ks.append(int4_block_values(k_pool[blk], block_size, "k"))
        vs.append(int4_block_values(v_pool[blk], block_size, "v"))
    if not ks:
        n_kv = k_pool.shape[1]
        d = int_tile_head_dim(k_pool.shape[2], block_size)
        return np.zeros((0, n_kv, d)), np.zeros((0, n_kv, d))
    return np.concatenate(ks)[:length], np.concatenate(vs)[:length]


def sequence_kv_f64(k_pool, v_pool, table_row, length, block_size,
                    cache_dtype, k_scale=None, v_scale=None):
    """Gather one sequence and widen it to float64 (times the FP8 scales;
    INT4 codes times their per-token scales)."""
    if cache_dtype == INT4:
        return gather_int4_f64(k_pool, v_pool, table_row, length, block_size)
    kr, vr = gather(k_pool, v_pool, table_row, length, block_size)
    k = to_f64(kr, cache_dtype)
    v = to_f64(vr, cache_dtype)
    if cache_dtype in FP8:
        k = k * np.asarray(k_scale, dtype=np.float32).astype(np.float64)[None, :, None]
        v = v * np.asarray(v_scale, dtype=np.float32).astype(np.float64)[None, :, None]
    return k, v


def decode(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
           block_tables: np.ndarray, context_lens: np.ndarray,
           block_size: int, scale: float, q_dtype: str, cache_dtype: str,
           k_scale=None, v_scale=None, seqs=None) -> np.ndarray:
    """Decode-phase attention for a batch: gather, then textbook attention.

    One query token per sequence attends to its ``context_lens[b]`` cached
    tokens, reached through ``block_tables[b]``.  Returns float64
    ``[S, Hq, d]`` (rows of sequences not in ``seqs`` are left zero when a
    subset is asked for).  ``scale`` is taken at its float32 value.
    """
    q64 = to_f64(q, q_dtype)
    s_count = q64.shape[0]
    out = np.zeros(q64.shape, dtype=np.float64)
    scale = float(np.float32(scale))
    for b in (range(s_count) if seqs is None else seqs):
        k, v = sequence_kv_f64(k_pool, v_pool, block_tables[b],
                               int(context_lens[b]), block_size,
                               cache_dtype, k_scale, v_scale)
        out[b] = attention(q64[b], k, v, scale)
    return out


# --------------------------------------------------------------------------
# several query tokens per sequence (chunked prefill, speculative verify)
# --------------------------------------------------------------------------

def query_positions(context_len: int, num_query: int) -> np.ndarray:
    """Positions of a sequence's query tokens: they are its last
    ``num_query`` cached tokens (their K/V were appended before attending),
    i.e. ``L - Q .. L - 1``."""
    if num_query > context_len:
        raise ValueError("a sequence has more query tokens than cached tokens")
    return np.arange(context_len - num_query, context_len)


def prefill_chunk(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                  block_tables: np.ndarray, context_lens: np.ndarray,
                  query_start: np.ndarray, block_size: int, scale: float,
                  q_dtype: str, cache_dtype: str, k_scale=None, v_scale=None,
                  seqs=None) -> np.ndarray:
    """Attention of several new tokens per sequence over the paged cache.

    Chunked prefill feeds a prompt in chunks of tokens next to the decodes
    ("vLLM & High-Throughput Serving", section 4); speculative decoding
    checks K drafted tokens in one pass over the context plus the
    candidates ("AI Inference Serving at Scale", section 7; "How LLM
    Inference Engines Work", speculative decoding).  Sequence b owns query
    rows ``query_start[b] .. query_start[b+1] - 1`` of ``q [T, Hq, d]``;
    they are its last Q_b cached tokens, and the token at position p
    attends to cached tokens 0..p -- each token sees the tokens before it
    and itself ("vLLM & High-Throughput Serving", section 1), never a later
    one.  Returns float64 ``[T, Hq, d]``.
    """
    q64 = to_f64(q, q_dtype)
    out = np.zeros(q64.shape, dtype=np.float64)
    scale = float(np.float32(scale))
    qs = np.asarray(query_start, dtype=np.int64)
    for b in (range(len(qs) - 1) if seqs is None else seqs):
        length = int(context_lens[b])
        r0, r1 = int(qs[b]), int(qs[b + 1])
        pos = query_positions(length, r1 - r0)
        if r1 == r0:
            continue
        k, v = sequence_kv_f64(k_pool, v_pool, block_tables[b], length,
                               block_size, cache_dtype, k_scale, v_scale)
        for i, p in enumerate(pos):
            out[r0 + i] = attention(q64[r0 + i], k[:p + 1], v[:p + 1], scale)
    return out


# --------------------------------------------------------------------------
# split context: partial softmax states and their merge
# --------------------------------------------------------------------------

def partial(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
            t0: int, t1: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Softmax state of one query over the token range ``[t0, t1)``.

    Returns, per query head: ``m`` = max of ``scale * K q`` over the range,
    ``l`` = sum of ``exp(scale * K q - m)``, ``o`` = the range's own
    normalised attention output (sum of ``exp(.. - m) * v`` divided by l).
    This is the state a context split keeps for later merging.
    """
    n_q, d = q.shape
    group = n_q // k.shape[1]
    m = np.empty(n_q)
    l = np.empty(n_q)
    o = np.empty((n_q, d))
    for hq in range(n_q):
        h = hq // group
        z = scale * (k[t0:t1, h, :] @ q[hq])
        m[hq] = z.max()
        e = np.exp(z - m[hq])
        l[hq] = e.sum()
        o[hq] = (e @ v[t0:t1, h, :]) / l[hq]
    return m, l, o


def merge(ms: np.ndarray, ls: np.ndarray, os_: np.ndarray) -> np.ndarray:
    """Combine softmax states of disjoint token ranges into the output.

    With ``M = max_p m_p`` and ``w_p = l_p * exp(m_p - M)``:
    ``out = sum_p w_p o_p / sum_p w_p``.  Each range's exp terms are
    rescaled to the common maximum, so this equals softmax over the union.
    ``ms``, ``ls``: ``[P]``; ``os_``: ``[P, d]``.
    """
    big_m = ms.max()
    w = ls * np.exp(ms - big_m)
    return (w[:, None] * os_).sum(axis=0) / w.sum()


def decode_partials(q, k_pool, v_pool, block_tables, context_lens,
                    block_size, scale, q_dtype, cache_dtype, partition_size,
                    k_scale=None, v_scale=None, seqs=None):
    """Per-partition softmax states of a split decode.

    Partition p of sequence b covers tokens ``[p*P, min((p+1)*P, L_b))``.
    Returns ``(m, l, o)`` shaped ``[S, Hq, maxP]``, ``[S, Hq, maxP]``,
    ``[S, Hq, maxP, d]`` with ``maxP = ceil(max L / P)``; entries of
    partitions a sequence does not have are NaN.
    """
    q64 = to_f64(q, q_dtype)
    s_count, n_q, d = q64.shape
    scale = float(np.float32(scale))
    lens = np.asarray(context_lens, dtype=np.int64)
    max_p = max(1, int(-(-int(lens.max()) // partition_size))) if len(lens) else 1
    m = np.full((s_count, n_q, max_p), np.nan)
    l = np.full((s_count, n_q, max_p), np.nan)
    o = np.full((s_count, n_q, max_p, d), np.nan)
    for b in (range(s_count) if seqs is None else seqs):
        length = int(lens[b])
        k, v = sequence_kv_f64(k_pool, v_pool, block_tables[b], length,
                               block_size, cache_dtype, k_scale, v_scale)
        for p in range(-(-length // partition_size)):
            t0 = p * partition_size
            t1 = min(t0 + partition_size, length)
            m[b, :, p], l[b, :, p], o[b, :, p] = partial(q64[b], k, v, scale, t0, t1)
    return m, l, o
