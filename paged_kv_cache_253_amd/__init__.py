"""Python binding of ``libpagedattn`` -- paged decode attention on MI355X.

Argument marshalling only: torch tensors become device pointers and torch's
current HIP stream becomes the ``hipStream_t``; every step of the
computation runs in the library's HIP kernels (C ABI in
``include/pagedattn.h``).  There is no CPU fallback: when the shared library
is missing or a call fails, these functions raise.

Pool layout (the library's): K ``[num_blocks, Hkv, D / X, B, X]`` with X
elements = 16 bytes (head-dim chunks, token-major per chunk row), V
``[num_blocks, Hkv, D, B]``; bf16 / f32 pools hold ``torch.bfloat16`` /
``torch.float32``, an FP8 pool holds its codes as ``torch.uint8`` (E4M3FN
unless ``cache_dtype="fp8_e5m2"`` says E5M2; ``torch.float8_e4m3fn`` /
``torch.float8_e5m2`` tensors say it themselves) with float32 scales per KV
head.  An INT4 pool (``cache_dtype="int4"``) is ``torch.uint8 [num_blocks,
Hkv, B * (D/2 + 4)]``: per (block, head) tile the 4-bit codes, then one
float32 scale per token.
"""

from __future__ import annotations

import ctypes
import functools
import math
import os

import torch

__all__ = ["PagedAttnError", "load", "kv_cache_write", "copy_blocks", "swap_blocks", "decode",
           "decode_append", "decode_partitions", "decode_noalloc",
           "prefill_chunk", "stream_read",
           "decode_reduce", "workspace_size", "new_workspace", "workspace_views", "default_partition_size",
           "PARTITION_AUTO", "PARTITION_AUTO_MERGED", "LIB_PATH", "prefill_partition"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_F32, PA_BF16, PA_FP8_E4M3, PA_FP8_E5M2, PA_INT4 = 0, 1, 2, 3, 4
_CACHE_CODES = {"f32": PA_F32, "bf16": PA_BF16, "fp8_e4m3": PA_FP8_E4M3, "fp8_e5m2": PA_FP8_E5M2,
                "int4": PA_INT4}
PARTITION_AUTO = -1  # balanced context split (PA_PARTITION_AUTO)
PARTITION_AUTO_MERGED = -2  # the same, merged inside the decode launch (PA_PARTITION_AUTO_MERGED)
_STATUS = {0: "PA_OK", 1: "PA_ERR_INVALID_ARG", 2: "PA_ERR_UNSUPPORTED",
           3: "PA_ERR_WORKSPACE", 4: "PA_ERR_HIP"}


class PagedAttnError(RuntimeError):
    def __init__(self, call: str, status: int):
        super().__init__(f"{call} failed: {_STATUS.get(status, status)}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load the shared library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m paged_kv_cache_253_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, szt = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                              ctypes.c_float, ctypes.c_size_t)
    lib.pa_kv_cache_write.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i32, i32,
                                      vp, vp, vp]
    lib.pa_kv_cache_write.restype = i32
    lib.pa_decode.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, i64,
                              f32, i32, i32, vp, vp, i32, vp, szt, vp]
    lib.pa_decode.restype = i32
    lib.pa_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32,
                                     i32, i64, f32, i32, i32, i32, vp, vp, i32, vp, szt, vp]
    lib.pa_decode_append.restype = i32
    lib.pa_decode_reduce.argtypes = [vp, vp, szt, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.pa_decode_reduce.restype = i32
    lib.pa_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.pa_decode_workspace_size.restype = szt
    lib.pa_copy_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i32, i64, i32, vp]
    lib.pa_copy_blocks.restype = i32
    lib.pa_prefill_chunk.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32,
                                     i32, i32, i64, f32, i32, i32, vp, vp, i32, vp, szt, vp]
    lib.pa_prefill_chunk.restype = i32
    lib.pa_prefill_reduce.argtypes = [vp, vp, szt, vp, i32, vp, i32, i32, i32, i32, i32, i32, i32,
                                      i32, vp]
    lib.pa_prefill_reduce.restype = i32
    lib.pa_swap_blocks.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, i32, vp]
    lib.pa_swap_blocks.restype = i32
    lib.pa_status_string.argtypes = [i32]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32,
                                      i32, i32, i64, f32, i32, i32, i32, vp, vp, vp]
    lib.pa_decode_noalloc.restype = i32
    lib.pa_stream_read.argtypes = [vp, szt, vp, vp]
    lib.pa_stream_read.restype = i32
    _lib = lib
    return lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PA_FP8_E4M3
    if t.dtype == torch.float8_e5m2:
        return PA_FP8_E5M2
    raise TypeError(f"unsupported element type {t.dtype}")


def _cache_code(k_cache: torch.Tensor, cache_dtype: str | None) -> int:
    """Element code of a pool: ``cache_dtype`` when given ("f32", "bf16",
    "fp8_e4m3", "fp8_e5m2"), else from the tensor (uint8 codes are E4M3,
    a ``torch.float8_e5m2`` tensor is E5M2)."""
    if cache_dtype is not None:
        code = _CACHE_CODES[cache_dtype]
        if code == PA_INT4:
            if k_cache.dtype != torch.uint8:
                raise ValueError("an int4 pool holds uint8 bytes")
            return code
        if (code in (PA_FP8_E4M3, PA_FP8_E5M2)) != (k_cache.element_size() == 1):
            raise ValueError(f"a {cache_dtype} pool cannot have {k_cache.dtype} elements")
        return code
    if k_cache.dtype == torch.float8_e5m2:
        return PA_FP8_E5M2
    return _dtype_code(k_cache)


def _ptr(t: torch.Tensor | None, pinned_ok: bool = False):
    if t is None:
        return None
    if not (t.is_cuda or (pinned_ok and t.is_pinned())):
        raise ValueError("tensors must live in GPU memory"
                         + (" or pinned host memory" if pinned_ok else ""))
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(call: str, status: int) -> None:
    if status != 0:
        raise PagedAttnError(call, status)


def workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                   max_context_len: int, partition_size: int) -> int:
    n = load().pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                        max_context_len, partition_size)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid workspace arguments")
    return int(n)


def new_workspace(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                  max_context_len: int, partition_size: int, device) -> torch.Tensor:
    """A zeroed workspace for a split decode (fixed partitions or the
    balanced split), sized by ``workspace_size``."""
    n = workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                       partition_size)
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=device)


def workspace_views(workspace: torch.Tensor, num_seqs: int, num_q_heads: int, head_dim: int,
                    max_context_len: int, partition_size: int):
    """(part_out, part_max, part_sum) float32 views of a fixed-partition
    workspace, in the layout documented at ``pa_decode_workspace_size``."""
    parts = max(1, -(-max_context_len // partition_size))
    rows = num_seqs * num_q_heads * parts

    def align(x):
        return (x + 255) // 256 * 256

    out_b = align(rows * head_dim * 4)
    max_b = align(rows * 4)
    flat = workspace.view(torch.uint8)
    part_out = flat[:rows * head_dim * 4].view(torch.float32).view(num_seqs, num_q_heads, parts, head_dim)
    part_max = flat[out_b:out_b + rows * 4].view(torch.float32).view(num_seqs, num_q_heads, parts)
    part_sum = flat[out_b + max_b:out_b + max_b + rows * 4].view(torch.float32).view(
        num_seqs, num_q_heads, parts)
    return part_out, part_max, part_sum


def default_partition_size(max_context_len: int) -> int:
    """Context split used when the caller gives none: the balanced split
    with a separate merge launch (the merge inside the decode launch,
    ``PARTITION_AUTO_MERGED``, measured no faster on MI355X: its last
    wavefront's store, count and reload take about as long as that launch)."""
    return PARTITION_AUTO


def _pool_dims(k_cache: torch.Tensor, v_cache: torch.Tensor | None, cache_dtype: str | None,
               head_dim: int | None = None,
               block_size: int | None = None) -> tuple[int, int, int, int]:
    """(num_blocks, num_kv_heads, block_size, head_dim) of a K/V pool pair,
    checking the V pool against the K pool.  An INT4 pool's tiles give
    block_size * (head_dim/2 + 4), so one of the two must be known."""
    if cache_dtype == "int4":
        if k_cache.dim() != 3 or k_cache.dtype != torch.uint8:
            raise ValueError("an int4 pool is uint8 [num_blocks, num_kv_heads, B * (D/2 + 4)]")
        nb, hkv, tile = (int(x) for x in k_cache.shape)
        if head_dim is not None:
            bsz, rem = divmod(tile, head_dim // 2 + 4)
        elif block_size is not None:
            bsz = int(block_size)
            per_token, rem = divmod(tile, bsz)
            head_dim = 2 * (per_token - 4)
        else:
            raise ValueError("an int4 pool needs head_dim or block_size")
        if rem or bsz < 1 or head_dim < 1:
            raise ValueError("int4 tile size does not match the head_dim / block_size")
        if v_cache is not None and (tuple(v_cache.shape) != tuple(k_cache.shape)
                                    or v_cache.dtype != k_cache.dtype):
            raise ValueError("V pool does not match the K pool")
        return nb, hkv, bsz, int(head_dim)
    nb, hkv, bsz, d = _k_pool_shape(k_cache)
    if v_cache is not None and (tuple(v_cache.shape) != (nb, hkv, d, bsz)
                                or v_cache.dtype != k_cache.dtype):
        raise ValueError("V pool does not match the K pool")
    return nb, hkv, bsz, d


def _k_pool_shape(k_cache: torch.Tensor) -> tuple[int, int, int, int]:
    """(num_blocks, num_kv_heads, block_size, head_dim) of a K pool laid out
    ``[nb, Hkv, head_dim / X, block_size, X]`` with X elements = 16 bytes."""
    if k_cache.dim() != 5 or k_cache.shape[4] * k_cache.element_size() != 16:
        raise ValueError("K pool must be [num_blocks, num_kv_heads, head_dim/X, block_size, X] "
                         "with X elements = 16 bytes")
    nb, hkv, nc, bsz, x = k_cache.shape
    return int(nb), int(hkv), int(bsz), int(nc * x)


def kv_cache_write(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                   v_cache: torch.Tensor, slot_mapping: torch.Tensor,
                   k_scale: torch.Tensor | None = None,
                   v_scale: torch.Tensor | None = None, cache_dtype: str | None = None) -> None:
    """``pa_kv_cache_write``: store row n of k_new/v_new at slot_mapping[n].
    ``cache_dtype`` names the pool's element format when its tensor type
    does not ("fp8_e5m2" for a uint8 pool of E5M2 codes)."""
    n, hkv, d = k_new.shape
    nb, hkv2, bsz, d2 = _pool_dims(k_cache, v_cache, cache_dtype, head_dim=d)
    if (hkv2, d2) != (hkv, d):
        raise ValueError("cache shapes do not match the new rows")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != n:
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    st = load().pa_kv_cache_write(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(slot_mapping), n, hkv, d, bsz, nb,
                                  _dtype_code(k_new), _cache_code(k_cache, cache_dtype),
                                  _ptr(k_scale), _ptr(v_scale), _stream(k_cache))
    _check("pa_kv_cache_write", st)


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor,
                block_mapping: torch.Tensor, cache_dtype: str | None = None,
                block_size: int | None = None) -> None:
    """``pa_copy_blocks``: copy block src to dst in both pools for each row
    (src, dst) of the int64 device tensor ``block_mapping [n, 2]``.  INT4
    pools need ``cache_dtype="int4"`` and their ``block_size``."""
    nb, hkv, bsz, d = _pool_dims(k_cache, v_cache, cache_dtype, block_size=block_size)
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be int64 [n, 2]")
    if not block_mapping.is_contiguous():
        raise ValueError("block_mapping must be contiguous")
    st = load().pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(block_mapping),
                               int(block_mapping.shape[0]), hkv, d, bsz, nb,
                               _cache_code(k_cache, cache_dtype), _stream(k_cache))
    _check("pa_copy_blocks", st)


def swap_blocks(dst_k: torch.Tensor, dst_v: torch.Tensor, src_k: torch.Tensor,
                src_v: torch.Tensor, block_mapping: torch.Tensor, cache_dtype: str | None = None,
                block_size: int | None = None) -> None:
    """``pa_swap_blocks``: copy block src -> dst from the (src_k, src_v) pools
    to the (dst_k, dst_v) pools for each row of ``block_mapping [n, 2]``
    (int64, on the GPU).  Either side may be a pinned host pool
    (``pin_memory=True``); the call runs on the current stream.  INT4 pools
    need ``cache_dtype="int4"`` and their ``block_size``."""
    snb, hkv, bsz, d = _pool_dims(src_k, src_v, cache_dtype, block_size=block_size)
    dnb, hkv2, bsz2, d2 = _pool_dims(dst_k, dst_v, cache_dtype, block_size=block_size)
    if (hkv2, bsz2, d2) != (hkv, bsz, d) or src_k.dtype != dst_k.dtype:
        raise ValueError("source and destination pools differ in shape or type")
    for t in (src_k, src_v, dst_k, dst_v):
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError("host pools must be pinned (pin_memory=True)")
        if not t.is_contiguous():
            raise ValueError("pools must be contiguous")
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be int64 [n, 2]")
    if not block_mapping.is_cuda or not block_mapping.is_contiguous():
        raise ValueError("block_mapping must be a contiguous GPU tensor")
    st = load().pa_swap_blocks(_ptr(dst_k, True), _ptr(dst_v, True), _ptr(src_k, True),
                               _ptr(src_v, True),
                               _ptr(block_mapping), int(block_mapping.shape[0]), snb, dnb, hkv,
                               d, bsz, _cache_code(src_k, cache_dtype), _stream(block_mapping))
    _check("pa_swap_blocks", st)


@functools.lru_cache(maxsize=None)
def _compute_units(device_index: int) -> int:
    return torch.cuda.get_device_properties(device_index).multi_processor_count


def prefill_partition(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                      max_query_len: int, max_context_len: int, two_tiles: bool,
                      device: torch.device | None = None, compute_units: int | None = None) -> int:
    """The split ``prefill_chunk`` takes when given none: the longest
    partitions (unsplit, then 4096, 2048, 1024 tokens, else 512) whose work
    units -- (sequence, KV head, query tile) triples times partitions at the
    longest context -- give the device two wavefronts per compute unit;
    unsplit for contexts of at most 1024 tokens.  ``two_tiles``: the kernel
    takes two 16-column tiles per wavefront (head_dim 128 with a bf16 or
    INT4 cache), else four.  ``compute_units``: the device's, unless given."""
    if max_context_len <= 1024:
        return 0
    rows = max(1, 16 * (2 if two_tiles else 4) // (num_q_heads // num_kv_heads))
    units = num_seqs * num_kv_heads * (-(-max_query_len // rows) if max_query_len else 0)
    if compute_units is None:
        compute_units = _compute_units(device.index if device is not None and device.index is not None
                                       else torch.cuda.current_device())
    want = 2 * compute_units
    for p in (0, 4096, 2048, 1024):
        parts = 1 if p == 0 else -(-max_context_len // p)
        if units * parts >= want:
            return p
    return 512


def prefill_chunk(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                  query_start: torch.Tensor, max_query_len: int, scale: float | None = None,
                  k_scale: torch.Tensor | None = None, v_scale: torch.Tensor | None = None,
                  partition_size: int | None = None, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None,
                  cache_dtype: str | None = None) -> torch.Tensor:
    """``pa_prefill_chunk`` (+ ``pa_prefill_reduce`` when split): attention
    of each sequence's last Q_b cached tokens (rows ``query_start[b] ..
    query_start[b+1]-1`` of ``q [T, Hq, D]``) over its prefix; returns out.

    ``partition_size`` None: ``prefill_partition``'s choice.  (Measured on
    MI355X, 8B-shaped batches with 5 query tokens per sequence: 16 sequences
    run best split at 1024 tokens, 48 at 2048, 64 and more unsplit; a fixed
    512 ran up to 1.4x slower.)"""
    t, hq, d = q.shape
    nb, hkv, bsz, _ = _pool_dims(k_cache, v_cache, cache_dtype, head_dim=d)
    s = int(query_start.numel()) - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 or \
            query_start.dtype != torch.int32:
        raise ValueError("block_tables, context_lens and query_start must be int32")
    if out is None:
        out = torch.empty_like(q)
    if partition_size is None:
        two_tiles = d == 128 and (q.dtype == k_cache.dtype or cache_dtype == "int4")
        partition_size = prefill_partition(s, hq, hkv, d, max_query_len, max_context_len,
                                           two_tiles, q.device)
    if partition_size and workspace is None:
        workspace = new_workspace(t, hq, hkv, d, max_context_len, partition_size, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().pa_prefill_chunk(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                 int(max_context_len), _ptr(query_start), t, int(max_query_len),
                                 s, hq, hkv, d, bsz, nb, float(scale), _dtype_code(q),
                                 _cache_code(k_cache, cache_dtype), _ptr(k_scale), _ptr(v_scale),
                                 int(partition_size), _ptr(workspace), ws_bytes, _stream(q))
    _check("pa_prefill_chunk", st)
    if partition_size:
        st = load().pa_prefill_reduce(_ptr(out), _ptr(workspace), ws_bytes, _ptr(context_lens),
                                      int(max_context_len), _ptr(query_start), t,
                                      int(max_query_len), s, hq, hkv, d, int(partition_size),
                                      _dtype_code(out), _stream(out))
        _check("pa_prefill_reduce", st)
    return out


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                   scale: float | None = None, k_scale: torch.Tensor | None = None,
                   v_scale: torch.Tensor | None = None, out: torch.Tensor | None = None,
                   cache_dtype: str | None = None, k_new: torch.Tensor | None = None,
                   v_new: torch.Tensor | None = None) -> torch.Tensor:
    """``pa_decode_noalloc``: the balanced-split decode step (appending
    ``k_new``/``v_new`` first when given) and its merge, with the split's
    states in the library's static scratch array -- no workspace and no
    allocation by the library (give ``out`` to allocate nothing here
    either).  Calls that overlap on one GPU share that array and race."""
    s, hq, d = q.shape
    nb, hkv, bsz, _ = _pool_dims(k_cache, v_cache, cache_dtype, head_dim=d)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if out is None:
        out = torch.empty_like(q)
    src = _dtype_code(k_new) if k_new is not None else PA_BF16
    st = load().pa_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(block_tables), block_tables.shape[1],
                                  _ptr(context_lens), int(max_context_len), s, hq, hkv, d, bsz,
                                  nb, float(scale), _dtype_code(q), src,
                                  _cache_code(k_cache, cache_dtype), _ptr(k_scale), _ptr(v_scale),
                                  _stream(q))
    _check("pa_decode_noalloc", st)
    return out


def stream_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """``pa_stream_read`` (measurement aid, ``include/pa_measure.h``): read
    every byte of ``buf`` once with the decode's 16-byte non-temporal loads;
    ``sink`` is a one-element int32 device tensor the kernel may write."""
    if sink.numel() < 1 or sink.element_size() != 4:
        raise ValueError("sink must hold one 4-byte element")
    nbytes = buf.numel() * buf.element_size()
    _check("pa_stream_read", load().pa_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(buf)))


def _decode_call(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                 scale, k_scale, v_scale, partition_size, workspace, cache_dtype=None,
                 k_new=None, v_new=None):
    s, hq, d = q.shape
    nb, hkv, bsz, _ = _pool_dims(k_cache, v_cache, cache_dtype, head_dim=d)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if k_new is not None:
        if (k_new.shape != (s, hkv, d) or v_new is None or v_new.shape != k_new.shape
                or v_new.dtype != k_new.dtype or not k_new.is_contiguous()
                or not v_new.is_contiguous()):
            raise ValueError("k_new and v_new must be contiguous [num_seqs, num_kv_heads, "
                             "head_dim] tensors of one dtype")
        st = load().pa_decode_append(
            _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
            _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), int(max_context_len),
            s, hq, hkv, d, bsz, nb, float(scale), _dtype_code(q), _dtype_code(k_new),
            _cache_code(k_cache, cache_dtype), _ptr(k_scale), _ptr(v_scale), int(partition_size),
            _ptr(workspace), ws_bytes, _stream(q))
        _check("pa_decode_append", st)
        return
    st = load().pa_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                          block_tables.shape[1], _ptr(context_lens), int(max_context_len), s, hq,
                          hkv, d, bsz, nb, float(scale), _dtype_code(q),
                          _cache_code(k_cache, cache_dtype),
                          _ptr(k_scale), _ptr(v_scale), int(partition_size), _ptr(workspace),
                          ws_bytes, _stream(q))
    _check("pa_decode", st)


def decode_partitions(q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                      partition_size, scale=None, k_scale=None, v_scale=None,
                      workspace=None, out=None, cache_dtype=None, k_new=None,
                      v_new=None) -> torch.Tensor:
    """Split ``pa_decode`` only (fixed partitions, or the balanced split,
    which also writes the rows of ``out`` it finishes), or
    ``pa_decode_append`` when ``k_new``/``v_new`` are given; returns the
    workspace."""
    s, hq, d = q.shape
    hkv = k_cache.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = new_workspace(s, hq, hkv, d, max_context_len, partition_size, q.device)
    _decode_call(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                 k_scale, v_scale, partition_size, workspace, cache_dtype, k_new, v_new)
    return workspace


def decode_reduce(out: torch.Tensor, workspace: torch.Tensor, context_lens: torch.Tensor,
                  max_context_len: int, partition_size: int,
                  num_kv_heads: int | None = None) -> torch.Tensor:
    """``pa_decode_reduce``: merge the workspace's states into ``out``.
    ``num_kv_heads`` defaults to the query heads (it only matters for the
    balanced split)."""
    s, hq, d = out.shape
    hkv = hq if num_kv_heads is None else int(num_kv_heads)
    st = load().pa_decode_reduce(_ptr(out), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(),
                                 _ptr(context_lens), int(max_context_len), s, hq, hkv, d,
                                 int(partition_size), _dtype_code(out), _stream(out))
    _check("pa_decode_reduce", st)
    return out


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
           scale: float | None = None, k_scale: torch.Tensor | None = None,
           v_scale: torch.Tensor | None = None, partition_size: int | None = None,
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
           cache_dtype: str | None = None, k_new: torch.Tensor | None = None,
           v_new: torch.Tensor | None = None) -> torch.Tensor:
    """Decode attention over the paged cache; returns ``out [S, Hq, D]``.

    ``partition_size`` 0 runs unsplit; > 0 (fixed partitions) or
    ``PARTITION_AUTO`` (balanced split) runs the split decode followed by
    the merge; ``PARTITION_AUTO_MERGED`` is the balanced split merged in the
    decode launch (a given ``workspace`` must then hold zero merge counters,
    as a new one and every merged call leave it; ``pa_decode_append``
    clears them itself).  None picks ``default_partition_size(max_context_len)``.
    With ``k_new``/``v_new`` ([S, Hkv, D]) each sequence's newest token
    (position ``context_lens[b] - 1``, slot from its block table) is
    appended first (``pa_decode_append``).
    """
    s, hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if partition_size is None:
        partition_size = default_partition_size(max_context_len)
    if out is None:
        out = torch.empty_like(q)
    if partition_size == 0:
        _decode_call(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                     scale, k_scale, v_scale, 0, None, cache_dtype, k_new, v_new)
        return out
    workspace = decode_partitions(q, k_cache, v_cache, block_tables, context_lens,
                                  max_context_len, partition_size, scale, k_scale, v_scale,
                                  workspace, out=out, cache_dtype=cache_dtype, k_new=k_new,
                                  v_new=v_new)
    if partition_size == PARTITION_AUTO_MERGED:
        return out
    return decode_reduce(out, workspace, context_lens, max_context_len, partition_size,
                         k_cache.shape[1])


def decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                  k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                  context_lens: torch.Tensor, max_context_len: int, **kw) -> torch.Tensor:
    """One decode step: append every sequence's newest K/V row (its slot
    taken from the block table) and attend (``pa_decode_append``, then the
    merge of a split unless it is ``PARTITION_AUTO_MERGED``).  Keyword
    arguments as ``decode``."""
    return decode(q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                  k_new=k_new, v_new=v_new, **kw)
