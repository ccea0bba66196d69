/*
 * pagedattn.h -- C ABI of the paged decode-attention library (AMD MI355X, gfx950).
 *
 * What it computes (restated from the pages it follows):
 *
 *   - A KV cache lives in a pre-allocated pool of fixed-size physical blocks
 *     of B tokens; each sequence reaches its blocks through a block table
 *     ("AI Inference Serving at Scale", section 3: physical block pool,
 *     logical-to-physical block table, on-demand allocation; "How LLM
 *     Inference Engines Work", PagedAttention section: pages of 16 or 32
 *     tokens).  Token t of a sequence is at offset t mod B of the physical
 *     block named by table entry floor(t / B) ("vLLM & High-Throughput
 *     Serving", section 2, block-table equation).  Several tables may name
 *     the same physical block (prefix sharing, same sections).
 *   - Decode-phase attention: one new query token per sequence attends to
 *     every cached token of that sequence ("AI Inference Serving at Scale",
 *     sections 1 and 2); the kernel gathers K and V from the non-adjacent
 *     blocks ("How LLM Inference Engines Work", PagedAttention section).
 *     Query head hq reads KV head hq / (Hq / Hkv) (grouped-query attention,
 *     "AI Inference Serving at Scale", section 6).  The result equals plain,
 *     un-paged attention (same page, FAQ).
 *   - An FP8 KV cache ("AI Inference Serving at Scale", section 6) stores
 *     OCP E4M3FN codes with one float32 scale per KV head: value = code *
 *     scale.
 *   - An INT4 KV cache (same section: 4-bit keys and values) stores, for
 *     every token and KV head, its K row (and its V row) as signed 4-bit
 *     codes plus one float32 scale of its own: value = code * scale, with
 *     scale = absmax(row) / 7 and codes in -7..7 written by the append.
 *
 * Conventions for every entry point:
 *
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The
 *     library allocates no memory and keeps no state between calls
 *     (pa_decode_noalloc's static scratch array aside).
 *   - Work is enqueued on `stream` (0 = the null stream) and is
 *     asynchronous; no call synchronizes the device or copies to the host.
 *   - Arguments are checked on the host before anything is launched; on
 *     failure the call returns a non-zero pa_status, launches nothing and
 *     leaves every buffer untouched.  A launch failure reported by the HIP
 *     runtime returns PA_ERR_HIP.  No C++ exception crosses this interface.
 *   - Contents of device arrays cannot be checked without a device sync;
 *     they are the caller's contract.  The kernels keep every memory access
 *     inside the buffers described here even when that contract is broken
 *     (see each call), but the results are then meaningless.
 *   - Calls that share no output buffers may run concurrently on different
 *     streams.
 *
 * Pool layout (one pool for K, one for V, `num_blocks` blocks each):
 *
 *   K cache: [num_blocks][num_kv_heads][head_dim / X][block_size][X]
 *            X = 16 bytes / element size (4 f32, 8 bf16, 16 fp8): inside a
 *            (block, head) tile the head dimension is cut into 16-byte
 *            chunks, and chunk row c holds chunk c of every token of the
 *            block in token order.  Element d of token j's K row sits at
 *            ((d / X) * block_size + j) * X + d % X within the tile.
 *   V cache: [num_blocks][num_kv_heads][head_dim][block_size]
 *            (inside a (block, head) tile: one row of block_size tokens per
 *            dimension)
 *
 * PA_INT4 pools are bytes [num_blocks][num_kv_heads][T] with tile size
 * T = block_size * (head_dim / 2 + 4): the tile's codes (block_size *
 * head_dim / 2 bytes) in the layout above with 4-bit elements -- K chunk
 * rows of X = 32 elements (16 bytes per token), V rows of block_size / 2
 * bytes -- followed by block_size float32 scales, token j's at byte
 * block_size * head_dim / 2 + 4 * j.  Codes are two's complement nibbles
 * grouped in octets of 8 consecutive elements of a row (8 dimensions of a K
 * row, 8 tokens of a V row) in 4 bytes: byte i of an octet holds element i
 * in its low nibble and element i + 4 in its high nibble.
 *
 * Supported shapes: head_dim 64 or 128; block_size 16 or 32; element types
 * as listed per call.
 *
 * Environment switches (read by the host side; none changes a result's
 * definition, only which kernel computes it):
 *
 *   PA_FORCE_PATH=valu|mfma   decode kernel family (vector units or matrix
 *                             cores) where both support the arguments
 *   PA_AUTO_WAVES_PER_CU=n    persistent wavefronts per compute unit for the
 *                             balanced split (1..8; default per kernel)
 *   PA_FIXED_GRID=1           fixed partitions one wavefront per partition
 *                             instead of on the persistent streaming grid
 *                             (same bits)
 *   PA_SEPARATE_APPEND=1      pa_decode_append launches its append on its
 *                             own even where the decode kernel can append
 *                             (same bits)
 *   PA_LOG=1                  one line per decode call on stderr (kernel
 *                             path, shape, split) and HIP error strings
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1, /* null pointer, negative count, inconsistent sizes */
  PA_ERR_UNSUPPORTED = 2, /* well-formed but not implemented (shape / type / group) */
  PA_ERR_WORKSPACE = 3,   /* split decode given too small a workspace */
  PA_ERR_HIP = 4          /* the HIP runtime reported an error */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,      /* IEEE binary32 */
  PA_BF16 = 1,     /* bfloat16 (upper half of a binary32) */
  PA_FP8_E4M3 = 2, /* OCP FP8 E4M3FN code, one byte, with a per-KV-head scale */
  PA_FP8_E5M2 = 3, /* OCP FP8 E5M2 code, one byte, with a per-KV-head scale */
  PA_INT4 = 4      /* signed 4-bit code, with a float32 scale per (token, KV head) */
} pa_dtype;

/* partition_size values selecting the balanced context split (see pa_decode):
 * merged by pa_decode_reduce, or merged inside the decode launch itself. */
#define PA_PARTITION_AUTO (-1)
#define PA_PARTITION_AUTO_MERGED (-2)

/*
 * pa_kv_cache_write -- append new tokens' K and V rows into the pool.
 *
 * Follows "AI Inference Serving at Scale", section 3 (each generated
 * token's K/V goes into its sequence's current block) and the block-table
 * equation of "vLLM & High-Throughput Serving", section 2 applied to a flat
 * slot number: token n is stored at block slot_mapping[n] / block_size,
 * offset slot_mapping[n] % block_size, for every KV head.
 *
 *   k_new, v_new   [num_tokens][num_kv_heads][head_dim], element src_dtype
 *   k_cache        K pool, element cache_dtype (layout above)
 *   v_cache        V pool, element cache_dtype (layout above)
 *   slot_mapping   [num_tokens] int64; a negative slot marks a padding token
 *                  and writes nothing
 *   num_blocks     pool size in blocks
 *   src_dtype      PA_F32 or PA_BF16
 *   cache_dtype    equal to src_dtype (the bits are copied unchanged), or
 *                  PA_FP8_E4M3: each element x of KV head h is stored as
 *                  round_to_nearest_even_e4m3(fp32(x) / k_scale[h]) (V with
 *                  v_scale), saturated to +-448; NaN stays NaN;
 *                  PA_FP8_E5M2: the same with E5M2 codes, saturated to
 *                  +-57344 (the largest finite E5M2 value; no infinities
 *                  are written);
 *                  PA_INT4: each token's K row of KV head h gets its own
 *                  scale s = fp32(absmax of the row) / 7 and codes
 *                  round_to_nearest_even(fp32(x) / s) within -7..7 (all
 *                  zero when s == 0); V rows likewise.  Rows must be finite
 *                  (a row with NaN or infinity stores unspecified codes)
 *   k_scale, v_scale  [num_kv_heads] float32, device; required for an FP8
 *                  cache, ignored otherwise (may be NULL)
 *
 * Caller contract: two tokens must not share a slot (the stored row is then
 * one of them, unspecified which).  A slot at or beyond
 * num_blocks * block_size is skipped.  num_tokens == 0 is a no-op.
 */
pa_status pa_kv_cache_write(const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache,
                            const int64_t* slot_mapping, int num_tokens,
                            int num_kv_heads, int head_dim, int block_size,
                            int64_t num_blocks,
                            pa_dtype src_dtype, pa_dtype cache_dtype,
                            const float* k_scale, const float* v_scale,
                            hipStream_t stream);

/*
 * pa_decode -- single-query attention of every sequence over its paged
 * context (the decode phase of "AI Inference Serving at Scale", section 1;
 * the gather of "How LLM Inference Engines Work", PagedAttention section).
 *
 * For sequence b and query head hq, with G = num_q_heads / num_kv_heads,
 * h = hq / G, L = context_lens[b] and k_t, v_t the K/V rows of token t
 * (read through block_tables[b] by the block-table equation):
 *
 *   z_t = scale * dot(q[b][hq], k_t)              (FP8: k_t = code * k_scale[h])
 *   out[b][hq] = sum_t softmax(z)_t * v_t          (FP8: v_t = code * v_scale[h])
 *
 * (INT4: k_t and v_t are codes times token t's own K and V scales.)
 *
 * accumulated in float32.  L == 0 gives zeros.
 *
 *   out            [num_seqs][num_q_heads][head_dim], element q_dtype; see
 *                  partition_size for which rows this call writes (may be
 *                  NULL for fixed partitions)
 *   q              [num_seqs][num_q_heads][head_dim], element q_dtype
 *   k_cache, v_cache   the pools (layout above), element cache_dtype
 *   block_tables   [num_seqs][max_blocks_per_seq] int32 physical block ids;
 *                  only entries below ceil(L / block_size) are read
 *   context_lens   [num_seqs] int32, device
 *   max_context_len    host-side upper bound of context_lens (sizes the
 *                  launch and the workspace without a device sync)
 *   num_blocks     pool size in blocks
 *   scale          softmax scale (typically 1 / sqrt(head_dim))
 *   q_dtype / cache_dtype  (PA_F32, PA_F32), (PA_BF16, PA_BF16),
 *                  (PA_BF16, PA_FP8_E4M3), (PA_BF16, PA_FP8_E5M2) or
 *                  (PA_BF16, PA_INT4); FP8 codes are widened exactly,
 *                  times the per-head scales; INT4 scales are applied in
 *                  float32 to the scores and to the softmax weights
 *   k_scale, v_scale   [num_kv_heads] float32, device; FP8 cache only;
 *                  finite and >= 0 (a scale is an absolute maximum over a
 *                  code range; the device reads them, the host cannot check)
 *   partition_size selects how contexts are cut into ranges, one range per
 *                  wavefront (split-context decoding; a wavefront's softmax
 *                  state over its range is merged with the others afterwards):
 *                  0: unsplit -- each (sequence, KV head) is one range and
 *                     `out` is written; no workspace.
 *                  P > 0 (a multiple of 32): fixed partitions -- partition p
 *                     of sequence b covers tokens [p*P, min((p+1)*P, L)); the
 *                     softmax state of every partition goes to `workspace`
 *                     and `out` is NOT written; pa_decode_reduce merges.
 *                  PA_PARTITION_AUTO: balanced -- every (sequence, KV head)
 *                     is a run of ceil(L / 32) 32-token steps (one step for
 *                     L == 0); the runs of the batch, KV head major, are cut
 *                     into W equal slices, one per persistent wavefront
 *                     (W = 2 to 8 per compute unit of the current device, by
 *                     kernel variant).  Runs one slice covers whole are
 *                     written to `out` here; the state of each run cut by a
 *                     slice boundary goes to `workspace`, and pa_decode_reduce
 *                     (same arguments) writes those runs' output.
 *                  PA_PARTITION_AUTO_MERGED: the same split, with every cut
 *                     run merged inside this launch by the wavefront that
 *                     finishes its last piece (an arrival counter per cut
 *                     run in the workspace header), so `out` is complete when
 *                     the call's work ends and pa_decode_reduce has nothing
 *                     to do.  Same output bits as PA_PARTITION_AUTO followed
 *                     by pa_decode_reduce.  The workspace's counters must be
 *                     zero on entry -- as in a zero-filled new workspace --
 *                     and every call leaves them zero (pa_decode_append
 *                     clears them itself before its decode).
 *   workspace, workspace_bytes  device scratch for the split modes; at least
 *                  pa_decode_workspace_size(...) bytes, 256-byte aligned;
 *                  ignored when partition_size == 0.  Concurrent calls must
 *                  not share a workspace.
 *
 * Group sizes: any G <= 16 for a bf16, FP8 or INT4 cache; G in {1, 2, 4, 8}
 * for an f32 cache.
 *
 * Caller contract: context_lens[b] <= max_context_len and <=
 * max_blocks_per_seq * block_size, and the table entries read are in
 * [0, num_blocks).  If not, L is clamped to max_context_len, no token at or
 * past max_blocks_per_seq * block_size is read (the context ends there; a
 * range lying wholly past it leaves the empty state: maximum -inf, exp-sum
 * 0, zero row), and block 0 is read in place of an out-of-range id, so no
 * access leaves the buffers and the split modes give the unsplit result.
 */
pa_status pa_decode(void* out, const void* q,
                    const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, int max_blocks_per_seq,
                    const int32_t* context_lens, int max_context_len,
                    int num_seqs, int num_q_heads, int num_kv_heads,
                    int head_dim, int block_size, int64_t num_blocks,
                    float scale, pa_dtype q_dtype, pa_dtype cache_dtype,
                    const float* k_scale, const float* v_scale,
                    int partition_size, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * pa_decode_append -- one decode step's append and attention in one call:
 * the effect of pa_kv_cache_write of every sequence's newest token followed
 * by pa_decode ("AI Inference Serving at Scale", section 3: the token just
 * generated joins its sequence's current block, and the next query attends
 * over the context including it).
 *
 * Sequence b's newest token is position L - 1, L = context_lens[b] clamped
 * to [0, max_context_len]; its slot is block_tables[b][(L - 1) / block_size]
 * * block_size + (L - 1) % block_size.  Rows k_new[b], v_new[b] are written
 * there exactly as pa_kv_cache_write writes a token with that slot; nothing
 * is written for b when L == 0, when (L - 1) / block_size >=
 * max_blocks_per_seq, or when that table entry is outside [0, num_blocks).
 * Then the attention is pa_decode with the same arguments: out, workspace
 * and pa_decode_reduce behave as there, and the results (pool contents and
 * out, bit for bit) are those of the two calls in sequence.
 *
 *   k_new, v_new   [num_seqs][num_kv_heads][head_dim], element src_dtype
 *                  (PA_F32 or PA_BF16; cache_dtype equal to it, FP8 or INT4)
 *   other arguments as pa_decode
 *
 * The caller needs no slot mapping for a decode step.  With a bf16 cache
 * and bf16 rows, PA_PARTITION_AUTO and G >= 2, the decode launch appends
 * the rows itself: the wavefront that reads a newest token's step takes
 * its rows from k_new / v_new and writes them to the pool after its last
 * read, so that block must not be read by any other sequence of the call
 * (copy-on-write first, as for any append into a shared block).  Otherwise
 * the append is a launch of its own on `stream`, before the decode's; with
 * PA_PARTITION_AUTO_MERGED it also clears the workspace's merge counters,
 * so a step is two launches and needs no pa_decode_reduce.
 *
 * Caller contract: that of pa_decode and of pa_kv_cache_write (two
 * sequences' newest tokens must not share a slot).
 */
pa_status pa_decode_append(void* out, const void* q,
                           const void* k_new, const void* v_new,
                           void* k_cache, void* v_cache,
                           const int32_t* block_tables, int max_blocks_per_seq,
                           const int32_t* context_lens, int max_context_len,
                           int num_seqs, int num_q_heads, int num_kv_heads,
                           int head_dim, int block_size, int64_t num_blocks,
                           float scale, pa_dtype q_dtype, pa_dtype src_dtype,
                           pa_dtype cache_dtype,
                           const float* k_scale, const float* v_scale,
                           int partition_size, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * pa_decode_workspace_size -- bytes of workspace a split pa_decode needs
 * (0 when partition_size == 0; SIZE_MAX for invalid arguments, or for
 * PA_PARTITION_AUTO when the current HIP device cannot be queried).
 *
 * Layout: a header of H bytes, then R rows of partial softmax state,
 * align(x) = x rounded up to a multiple of 256,
 *
 *   float part_out[R][head_dim]   at H
 *   float part_max[R]             at H + align(R * head_dim * 4)
 *   float part_sum[R]             at that + align(R * 4)
 *
 * Fixed partitions: H = 0, R = num_seqs * num_q_heads * maxP with
 * maxP = max(1, ceil(max_context_len / partition_size)); the state of
 * partition p of sequence b, query head hq is row (b * num_q_heads + hq) *
 * maxP + p; rows of partitions a sequence does not have are unused.
 * PA_PARTITION_AUTO and PA_PARTITION_AUTO_MERGED: H = 256 + align(16 * 8 *
 * CUs) + align(4 * 8 * CUs), R = 8 * CUs * 2 * G (CUs = compute units of
 * the current device, G = num_q_heads / num_kv_heads; a decode uses at most
 * W = 8 * CUs slices).  pa_decode stores W as an int32 at offset 0 and, at
 * offset 256 + 16 s, four int32 naming the cut run whose first piece slice
 * s holds (sequence, KV head, number of slices holding a piece, state slot
 * of the first piece; a piece count of 0 = none), for pa_decode_reduce.
 * Then, at offset 256 + align(16 * 8 * CUs), 8 * CUs int32 arrival
 * counters for PA_PARTITION_AUTO_MERGED (counter s counts the finished
 * pieces of the cut run whose first piece slice s holds).  Slice s keeps
 * the state of its first run in rows (2s) * G + g and of its last run in
 * rows (2s + 1) * G + g, for the group's query heads g, when those runs are
 * cut.
 *
 * A state over tokens T of a query head, with z_t as in pa_decode:
 * part_max = max_{t in T} z_t, part_sum = sum_t exp(z_t - part_max),
 * part_out = sum_t exp(z_t - part_max) v_t / part_sum.
 */
size_t pa_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                int max_context_len, int partition_size);

/*
 * pa_decode_reduce -- merge the partial states of a split decode into `out`.
 *
 * The ranges of one (sequence, query head) are disjoint; rescaling each
 * range's exp-sum to the common maximum and weighting the range outputs by
 * it gives softmax over the whole context (the split-context merge of flash
 * decoding; the pages' un-paged attention is the result it must reproduce):
 *
 *   M = max_p part_max[p];  w_p = part_sum[p] * exp(part_max[p] - M)
 *   out = sum_p w_p * part_out[p] / sum_p w_p
 *
 * in float32, ranges added in a fixed order (identical bits on every call).
 * Fixed partitions: every row of `out` is written (L == 0 gives zeros).
 * PA_PARTITION_AUTO: only the rows of runs that pa_decode left cut are
 * written; pa_decode wrote the others.  PA_PARTITION_AUTO_MERGED: nothing
 * to merge (the decode launch did); returns PA_OK after the argument checks.
 *
 *   out            [num_seqs][num_q_heads][head_dim], element out_dtype
 *                  (PA_F32 or PA_BF16, rounded to nearest even)
 *   workspace      as filled by pa_decode called with the same num_seqs,
 *                  num_q_heads, num_kv_heads, head_dim, max_context_len,
 *                  partition_size (and, for PA_PARTITION_AUTO, on the same
 *                  device and stream order)
 *   context_lens   [num_seqs] int32, device (clamped to max_context_len)
 */
pa_status pa_decode_reduce(void* out, const void* workspace, size_t workspace_bytes,
                           const int32_t* context_lens, int max_context_len,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int partition_size, pa_dtype out_dtype,
                           hipStream_t stream);

/*
 * pa_copy_blocks -- copy whole blocks inside the pools (copy-on-write).
 *
 * When a sequence is about to write a token into a block that other
 * sequences also reference, the engine gives it a private copy of that one
 * block first ("AI Inference Serving at Scale", section 3, copy-on-write
 * sharing; "vLLM & High-Throughput Serving", copy-on-write prefix caching).
 * The caller's block manager picks the pairs and updates reference counts
 * and block tables; this call copies the bytes: for each pair i, the K and
 * V data of every KV head of block src_i is copied to block dst_i.
 *
 *   k_cache, v_cache  the pools (layout above), element cache_dtype; a
 *                  block is num_kv_heads * block_size * head_dim elements
 *                  of each pool, contiguous (PA_INT4: num_kv_heads tiles of
 *                  block_size * (head_dim / 2 + 4) bytes, scales included)
 *   block_mapping  [num_pairs][2] int64, device: (src_i, dst_i)
 *   num_blocks     blocks in each pool
 *
 * Contract: the dst ids are distinct and none is also a src, so the pairs
 * are independent and their order does not matter.  Pairs with an id
 * outside [0, num_blocks) are skipped (no access leaves the pools).
 * Errors: PA_ERR_INVALID_ARG for null pools, a null mapping with
 * num_pairs > 0, or negative counts; PA_ERR_UNSUPPORTED for shapes outside
 * head_dim {64, 128} and block_size {16, 32}; PA_ERR_HIP for a failed
 * launch.  num_pairs == 0 does nothing.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                         int num_pairs, int num_kv_heads, int head_dim, int block_size,
                         int64_t num_blocks, pa_dtype cache_dtype, hipStream_t stream);

/*
 * pa_swap_blocks -- move whole blocks between two pools, e.g. the device
 * pools and pools in pinned host memory, for preemption ("How LLM Inference
 * Engines Work", the scheduler swaps a sequence's blocks to CPU memory when
 * the GPU is full and back when it resumes).
 *
 * For each pair i, the K and V data of every KV head of block src_i of the
 * source pools is copied to block dst_i of the destination pools, in one
 * launch on `stream`; the GPU reads or writes the host side directly.
 *
 *   dst_k, dst_v / src_k, src_v  pools in the layout above, element
 *                  cache_dtype, device memory or host memory from
 *                  hipHostMalloc (device-accessible); src_num_blocks /
 *                  dst_num_blocks blocks each
 *   block_mapping  [num_pairs][2] int64 (src_i, dst_i), device-accessible
 *
 * Contract: distinct dst ids (and, when the pools are the same, no dst is a
 * src).  Pairs with an id outside its pool are skipped.  Each pool pointer
 * is checked with hipPointerGetAttributes: memory the GPU cannot address at
 * that pointer (unpinned host memory, host memory mapped elsewhere) gives
 * PA_ERR_INVALID_ARG.  Other errors as pa_copy_blocks.  Host memory holds
 * the GPU's writes once the stream has been synchronised.
 */
pa_status pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                         const int64_t* block_mapping, int num_pairs, int64_t src_num_blocks,
                         int64_t dst_num_blocks, int num_kv_heads, int head_dim, int block_size,
                         pa_dtype cache_dtype, hipStream_t stream);

/*
 * pa_prefill_chunk -- attention of several new tokens per sequence over the
 * paged cache: a prompt fed in chunks next to the decodes ("vLLM &
 * High-Throughput Serving", section 4, chunked prefill) or K drafted tokens
 * checked in one pass ("AI Inference Serving at Scale", section 7,
 * speculative decoding).
 *
 * Sequence b owns query rows query_start[b] .. query_start[b+1]-1 of q and
 * out.  They are its last Q_b cached tokens -- their K/V rows were appended
 * (pa_kv_cache_write) before this call -- and row i, at position
 * p = L_b - Q_b + i, attends to cached tokens 0 .. p (each token sees the
 * tokens before it and itself):
 *
 *   out[r][hq] = sum_{t <= p} softmax_t(z_t) v_t,  z_t = scale * q[r][hq] . k_t
 *
 * with the GQA mapping, FP8 / INT4 scales and block-table walk of pa_decode.
 *
 *   out            [num_query_tokens][num_q_heads][head_dim] bf16; written
 *                  when partition_size == 0
 *   q              [num_query_tokens][num_q_heads][head_dim] bf16, device
 *   query_start    [num_seqs + 1] int32, device: nondecreasing,
 *                  query_start[0] = 0, query_start[num_seqs] = num_query_tokens
 *   max_query_len  host upper bound of Q_b (sizes the grid)
 *   other arguments as pa_decode (cache PA_BF16, PA_FP8_E4M3, PA_FP8_E5M2
 *                  or PA_INT4)
 *   partition_size 0: each query tile over its whole prefix, `out`
 *                     written: one wavefront per (query tile, KV head,
 *                     sequence), or for bf16 caches with G * max_query_len
 *                     >= 256, one workgroup of eight wavefronts per eight
 *                     consecutive query tiles, sharing K and V through LDS;
 *                  P > 0 (a multiple of 32): fixed partitions of the prefix;
 *                     states to `workspace`, pa_prefill_reduce merges.
 *   workspace      P > 0: at least pa_decode_workspace_size(num_query_tokens,
 *                  num_q_heads, num_kv_heads, head_dim, max_context_len, P)
 *                  bytes, 256-byte aligned; the state of query row r, query
 *                  head hq, partition p is row (r * num_q_heads + hq) * maxP + p
 *                  of that layout (maxP = ceil(max_context_len / P)).
 *
 * Group sizes: G in {1, 2, 4, 8, 16}.  PA_PARTITION_AUTO is not supported
 * here (PA_ERR_UNSUPPORTED).  Caller contract: Q_b <= L_b; a row whose
 * position would be negative attends to nothing and gets zeros.
 */
pa_status pa_prefill_chunk(void* out, const void* q,
                           const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, int max_blocks_per_seq,
                           const int32_t* context_lens, int max_context_len,
                           const int32_t* query_start, int num_query_tokens,
                           int max_query_len, int num_seqs, int num_q_heads,
                           int num_kv_heads, int head_dim, int block_size,
                           int64_t num_blocks, float scale, pa_dtype q_dtype,
                           pa_dtype cache_dtype, const float* k_scale,
                           const float* v_scale, int partition_size,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * pa_prefill_reduce -- merge the partition states of a split
 * pa_prefill_chunk into `out` (the merge of pa_decode_reduce, per query row:
 * row i of sequence b merges partitions p < ceil((L_b - Q_b + i + 1) / P)).
 * Arguments as given to pa_prefill_chunk; out_dtype PA_BF16 or PA_F32.
 */
pa_status pa_prefill_reduce(void* out, const void* workspace, size_t workspace_bytes,
                            const int32_t* context_lens, int max_context_len,
                            const int32_t* query_start, int num_query_tokens,
                            int max_query_len, int num_seqs, int num_q_heads,
                            int num_kv_heads, int head_dim, int partition_size,
                            pa_dtype out_dtype, hipStream_t stream);

/*
 * pa_decode_noalloc -- for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The decode step of pa_decode_append (k_new and v_new given)
 * or pa_decode (both NULL) with the balanced split (PA_PARTITION_AUTO),
 * followed by its merge (pa_decode_reduce), so `out` is complete when the
 * call's work ends -- the same launches, kernels and result bits as those
 * calls with a caller's workspace, but the split's partial states live in a
 * scratch array inside the library.
 *
 * Scratch: one static device array of PA_NOALLOC_SCRATCH_BYTES per GPU the
 * library runs on, held until the process ends; its device address is
 * looked up once per device, on the first call made with that device
 * current (make that call before capturing a graph).  A batch whose
 * balanced-split workspace (pa_decode_workspace_size with PA_PARTITION_AUTO)
 * is larger returns PA_ERR_WORKSPACE and launches nothing; on a 256-CU
 * MI355X every supported shape fits (the largest, G = 16 at head_dim 128,
 * needs 34.1 MB).  Nothing in the array needs to start at zero, and it
 * keeps the last call's states.  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (on different streams, or
 * from host threads without ordering) race and give wrong results; calls
 * ordered on one stream are safe.
 *
 * This call allocates nothing: no hipMalloc, hipFree or allocating library
 * routine.  Arguments as pa_decode_append (or pa_decode), without
 * partition_size and the workspace; src_dtype is ignored when k_new is NULL.
 * Errors as those calls, plus PA_ERR_INVALID_ARG when only one of k_new and
 * v_new is given, PA_ERR_WORKSPACE as above, PA_ERR_HIP when the device or
 * the array's address cannot be queried.
 */
#define PA_NOALLOC_SCRATCH_BYTES (40u << 20)

pa_status pa_decode_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache,
                            const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* context_lens, int max_context_len,
                            int num_seqs, int num_q_heads, int num_kv_heads,
                            int head_dim, int block_size, int64_t num_blocks,
                            float scale, pa_dtype q_dtype, pa_dtype src_dtype,
                            pa_dtype cache_dtype, const float* k_scale, const float* v_scale,
                            hipStream_t stream);

/* pa_status_string -- static, human-readable name of a status code. */
const char* pa_status_string(pa_status status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
