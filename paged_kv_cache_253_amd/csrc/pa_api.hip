// C ABI: argument checks, kernel choice, launch on the caller's stream.
// Declared and documented in include/pagedattn.h.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "pa_internal.hpp"
#include "pagedattn.h"

using pa::Elem;

static_assert(pa::kAuto == PA_PARTITION_AUTO && pa::kAutoMerged == PA_PARTITION_AUTO_MERGED,
              "split-mode values of the ABI");

namespace {

constexpr int kStepTokens = 32;  // kernels walk the context in 32-token steps

bool supported_dim(int head_dim) { return head_dim == 64 || head_dim == 128; }
bool supported_block(int block_size) { return block_size == 16 || block_size == 32; }

bool to_elem(pa_dtype t, Elem* e) {
  switch (t) {
    case PA_F32: *e = Elem::F32; return true;
    case PA_BF16: *e = Elem::BF16; return true;
    case PA_FP8_E4M3: *e = Elem::FP8; return true;
    case PA_FP8_E5M2: *e = Elem::E5M2; return true;
    case PA_INT4: *e = Elem::I4; return true;
  }
  return false;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t head_bytes, out_bytes, max_bytes, total;
  size_t counters_off;  // balanced split: offset of the merge counters in the header
  int max_parts;   // fixed partitions: partitions per (sequence, query head)
  int slices_max;  // balanced split: most persistent wavefronts
  int cus;         // balanced split: compute units
};

// Wavefronts per compute unit for the balanced split: 0 = each decode
// kernel's own choice, or PA_AUTO_WAVES_PER_CU (1..kAutoMaxWavesPerCU) for
// tuning.
int auto_waves_override() {
  static const int n = [] {
    const char* e = std::getenv("PA_AUTO_WAVES_PER_CU");
    const int v = e ? std::atoi(e) : 0;
    return (v >= 1 && v <= pa::kAutoMaxWavesPerCU) ? v : 0;
  }();
  return n;
}

// Compute units of the current device, 0 if it cannot be queried.
int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 0;
  if (dev < 64) cached[dev] = cus;
  return cus;
}

bool workspace_layout(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int max_context_len, int partition_size, Layout* l) {
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads ||
      head_dim < 1 || max_context_len < 0)
    return false;
  size_t rows;
  l->max_parts = 1;
  l->slices_max = 0;
  l->cus = 0;
  l->head_bytes = 0;
  l->counters_off = 0;
  if (partition_size == pa::kAuto || partition_size == pa::kAutoMerged) {
    l->cus = device_cus();
    if (l->cus <= 0) return false;
    l->slices_max = l->cus * pa::kAutoMaxWavesPerCU;
    l->counters_off = pa::kHdrRecordsBytes + align256((size_t)l->slices_max * pa::kMergeRecordBytes);
    l->head_bytes = l->counters_off + align256((size_t)l->slices_max * sizeof(int));
    rows = (size_t)l->slices_max * 2 * (size_t)(num_q_heads / num_kv_heads);
  } else if (partition_size > 0) {
    const long long parts = std::max(1LL, ((long long)max_context_len + partition_size - 1) / partition_size);
    l->max_parts = (int)parts;
    rows = (size_t)num_seqs * num_q_heads * (size_t)parts;
  } else {
    return false;
  }
  l->out_bytes = align256(rows * head_dim * sizeof(float));
  l->max_bytes = align256(rows * sizeof(float));
  l->total = l->head_bytes + l->out_bytes + 2 * l->max_bytes;
  return true;
}

// PA_SEPARATE_APPEND=1 makes pa_decode_append launch its append separately
// even where the decode kernel can append (cross-checks and timing).
bool separate_append_forced() {
  const char* e = std::getenv("PA_SEPARATE_APPEND");
  return e && e[0] == '1';
}

// PA_FIXED_GRID=1 runs fixed partitions one wavefront per partition
// instead of on the persistent streaming grid (cross-checks and timing).
bool fixed_grid_forced() {
  const char* e = std::getenv("PA_FIXED_GRID");
  return e && e[0] == '1';
}

// "valu" / "mfma" forces a decode kernel family (tuning and cross-checks).
int forced_path() {
  const char* e = std::getenv("PA_FORCE_PATH");
  if (!e) return 0;
  if (std::strcmp(e, "valu") == 0) return 1;
  if (std::strcmp(e, "mfma") == 0) return 2;
  return 0;
}

bool log_enabled() {
  const char* e = std::getenv("PA_LOG");
  return e && e[0] == '1';
}

pa_status from_hip(hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  if (log_enabled()) std::fprintf(stderr, "[pagedattn] HIP error: %s\n", hipGetErrorString(e));
  return PA_ERR_HIP;
}

}  // namespace

namespace {

pa_status copy_or_swap(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                       const int64_t* block_mapping, int num_pairs, int64_t src_blocks,
                       int64_t dst_blocks, int num_kv_heads, int head_dim, int block_size,
                       pa_dtype cache_dtype, hipStream_t stream) {
  if (num_pairs < 0 || num_kv_heads < 1 || src_blocks < 1 || dst_blocks < 1)
    return PA_ERR_INVALID_ARG;
  Elem cache;
  if (!to_elem(cache_dtype, &cache)) return PA_ERR_INVALID_ARG;
  if (!supported_dim(head_dim) || !supported_block(block_size)) return PA_ERR_UNSUPPORTED;
  if (!src_k || !src_v || !dst_k || !dst_v) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;  // an empty mapping may come with a null pointer
  if (!block_mapping) return PA_ERR_INVALID_ARG;
  pa::CopyArgs a;
  a.src_k = src_k; a.src_v = src_v; a.dst_k = dst_k; a.dst_v = dst_v;
  a.mapping = block_mapping;
  a.src_blocks = src_blocks; a.dst_blocks = dst_blocks;
  a.block_bytes = (int64_t)num_kv_heads * pa::tile_bytes(cache, head_dim, block_size);
  a.num_pairs = num_pairs;
  if (a.block_bytes > (int64_t)65535 * 4096) return PA_ERR_UNSUPPORTED;  // grid z limit
  return from_hip(pa::launch_copy_blocks(a, stream));
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
  }
  return "PA_ERR_UNKNOWN";
}

size_t pa_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                int max_context_len, int partition_size) {
  if (partition_size == 0 && num_seqs >= 0 && num_q_heads >= 1 && num_kv_heads >= 1 &&
      num_q_heads % num_kv_heads == 0 && head_dim >= 1 && max_context_len >= 0)
    return 0;
  Layout l;
  if (!workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                        partition_size, &l))
    return SIZE_MAX;
  return l.total;
}

pa_status pa_kv_cache_write(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                            int head_dim, int block_size, int64_t num_blocks, pa_dtype src_dtype,
                            pa_dtype cache_dtype, const float* k_scale, const float* v_scale,
                            hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads < 1 || num_blocks < 1) return PA_ERR_INVALID_ARG;
  Elem src, cache;
  if (!to_elem(src_dtype, &src) || !to_elem(cache_dtype, &cache)) return PA_ERR_INVALID_ARG;
  if (!supported_dim(head_dim) || !supported_block(block_size)) return PA_ERR_UNSUPPORTED;
  if (src != Elem::F32 && src != Elem::BF16) return PA_ERR_UNSUPPORTED;
  if (cache != src && !is_fp8(cache) && cache != Elem::I4) return PA_ERR_UNSUPPORTED;
  if (num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (is_fp8(cache) && (!k_scale || !v_scale)) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  pa::WriteArgs a;
  std::memset(&a, 0, sizeof a);
  a.k_new = k_new; a.v_new = v_new; a.k_cache = k_cache; a.v_cache = v_cache;
  a.slots = slot_mapping; a.k_scale = k_scale; a.v_scale = v_scale;
  a.num_slots = num_blocks * block_size;
  a.num_tokens = num_tokens; a.num_kv_heads = num_kv_heads;
  return from_hip(pa::launch_cache_write(a, src, cache, head_dim, block_size, stream));
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                         int num_pairs, int num_kv_heads, int head_dim, int block_size,
                         int64_t num_blocks, pa_dtype cache_dtype, hipStream_t stream) {
  return copy_or_swap(k_cache, v_cache, k_cache, v_cache, block_mapping, num_pairs, num_blocks,
                      num_blocks, num_kv_heads, head_dim, block_size, cache_dtype, stream);
}

pa_status pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                         const int64_t* block_mapping, int num_pairs, int64_t src_num_blocks,
                         int64_t dst_num_blocks, int num_kv_heads, int head_dim, int block_size,
                         pa_dtype cache_dtype, hipStream_t stream) {
  // The kernel dereferences all four pools: each must be memory the GPU
  // addresses at the same pointer (device memory, or pinned host memory
  // mapped into the device's address space) -- anything else is refused
  // here instead of faulting there.
  for (const void* p : {static_cast<const void*>(dst_k), static_cast<const void*>(dst_v), src_k, src_v}) {
    if (!p) return PA_ERR_INVALID_ARG;
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
      (void)hipGetLastError();  // leave no sticky error behind
      return PA_ERR_INVALID_ARG;
    }
    if (attr.type == hipMemoryTypeUnregistered) return PA_ERR_INVALID_ARG;
    if (attr.type == hipMemoryTypeHost && attr.devicePointer != p) return PA_ERR_INVALID_ARG;
  }
  return copy_or_swap(src_k, src_v, dst_k, dst_v, block_mapping, num_pairs, src_num_blocks,
                      dst_num_blocks, num_kv_heads, head_dim, block_size, cache_dtype, stream);
}

namespace {

// pa_decode, and pa_decode_append when k_new is not null (k_pool_w /
// v_pool_w: the same pools as k_cache / v_cache, writable; null for pa_decode).
pa_status decode_impl(void* out, const void* q, const void* k_new, const void* v_new,
                      void* k_pool_w, void* v_pool_w,
                      const void* k_cache, const void* v_cache, const int32_t* block_tables,
                      int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                      int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                      int64_t num_blocks, float scale, pa_dtype q_dtype, pa_dtype src_dtype,
                      pa_dtype cache_dtype, const float* k_scale, const float* v_scale,
                      int partition_size, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || max_context_len < 0 ||
      max_blocks_per_seq < 1 || num_blocks < 1 || partition_size < PA_PARTITION_AUTO_MERGED)
    return PA_ERR_INVALID_ARG;
  const bool merged = partition_size == PA_PARTITION_AUTO_MERGED;
  const bool balanced = merged || partition_size == PA_PARTITION_AUTO;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (!(std::isfinite(scale) && scale > 0.0f)) return PA_ERR_INVALID_ARG;
  Elem qe, ce;
  if (!to_elem(q_dtype, &qe) || !to_elem(cache_dtype, &ce)) return PA_ERR_INVALID_ARG;
  if (!supported_dim(head_dim) || !supported_block(block_size)) return PA_ERR_UNSUPPORTED;
  const bool combo_ok = (qe == Elem::F32 && ce == Elem::F32) || (qe == Elem::BF16 && ce == Elem::BF16) ||
                        (qe == Elem::BF16 && (is_fp8(ce) || ce == Elem::I4));
  if (!combo_ok) return PA_ERR_UNSUPPORTED;
  if (partition_size > 0 && partition_size % kStepTokens != 0) return PA_ERR_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if (partition_size <= 0 && !out) return PA_ERR_INVALID_ARG;
  if (is_fp8(ce) && (!k_scale || !v_scale)) return PA_ERR_INVALID_ARG;
  if (num_seqs > 65535 || num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;

  const int group = num_q_heads / num_kv_heads;
  const bool valu_group = group == 1 || group == 2 || group == 4 || group == 8;
  const int force = forced_path();
  bool use_mfma;
  if (ce == Elem::F32) {
    if (force == 2 || !valu_group) return PA_ERR_UNSUPPORTED;
    use_mfma = false;
  } else if (ce == Elem::I4) {  // matrix-core kernels only, any G <= 16
    if (force == 1 || group > 16) return PA_ERR_UNSUPPORTED;
    use_mfma = true;
  } else if (force == 1) {
    if (!valu_group) return PA_ERR_UNSUPPORTED;
    use_mfma = false;
  } else if (force == 2) {
    if (group > 16) return PA_ERR_UNSUPPORTED;
    use_mfma = true;
  } else {
    // bf16 and FP8 caches run on the matrix-core kernels for every group
    // size, multi-head attention (G = 1) included: their persistent
    // streaming grid keeps more of the context in flight than the
    // vector-unit kernels (measured on MI355X, 64-head bf16 batch at
    // G = 1: 518 us vs 540 us; the same batch sharing a 2048-token prefix:
    // 424 us vs 456 us)
    if (group > 16) return PA_ERR_UNSUPPORTED;
    use_mfma = true;
  }

  const bool append = k_new != nullptr;
  Elem se = Elem::BF16;
  if (append) {
    if (!v_new || !to_elem(src_dtype, &se)) return PA_ERR_INVALID_ARG;
    if (se != Elem::F32 && se != Elem::BF16) return PA_ERR_UNSUPPORTED;
    if (ce != se && !is_fp8(ce) && ce != Elem::I4) return PA_ERR_UNSUPPORTED;
  }
  // bf16 cache, balanced split, matrix-core kernels: the decode launch
  // appends the newest tokens itself (their rows go into the operand
  // registers of the step that reads them and into the pool after the
  // wavefront's ring has drained).  Otherwise the append is a launch of its
  // own, before the decode's.  PA_SEPARATE_APPEND=1 forces the two launches
  // (cross-checks and timing).
  const bool fuse_append = append && use_mfma && ce == Elem::BF16 && se == Elem::BF16 &&
                           partition_size == PA_PARTITION_AUTO && !separate_append_forced();
  pa::DecodeArgs a;
  std::memset(&a, 0, sizeof a);
  a.out = out; a.q = q; a.k_cache = k_cache; a.v_cache = v_cache;
  a.block_tables = block_tables; a.context_lens = context_lens;
  a.k_scale = k_scale; a.v_scale = v_scale;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  const long long cap = (long long)max_blocks_per_seq * block_size;
  a.cap_len = (int)std::min<long long>(cap, INT32_MAX);
  // lengths are clamped to max_context_len only, as pa_decode_reduce clamps
  // them, so every partition the merge counts has a state; tokens past the
  // table row (cap_len) are never read, and a range lying wholly past it
  // leaves the empty state
  a.max_len = max_context_len;
  a.num_seqs = num_seqs; a.num_q_heads = num_q_heads; a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.partition = balanced ? pa::kAuto : partition_size;
  a.scale = scale;
  a.max_parts = 1;
  int num_counters = 0;
  if (partition_size != 0) {
    Layout l;
    if (!workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                          partition_size, &l))
      return balanced ? PA_ERR_HIP : PA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < l.total || (reinterpret_cast<uintptr_t>(workspace) & 255))
      return PA_ERR_WORKSPACE;
    char* w = static_cast<char*>(workspace);
    a.header = reinterpret_cast<int*>(w);
    if (merged) {
      a.counters = reinterpret_cast<int*>(w + l.counters_off);
      num_counters = l.slices_max;
    }
    w += l.head_bytes;
    a.part_out = reinterpret_cast<float*>(w);
    a.part_max = reinterpret_cast<float*>(w + l.out_bytes);
    a.part_sum = reinterpret_cast<float*>(w + l.out_bytes + l.max_bytes);
    a.max_parts = l.max_parts;
    a.cus = balanced ? l.cus : device_cus();
    a.waves_per_cu = auto_waves_override();
    // fixed partitions stream when their state rows fit the kernel's int row
    // index -- except INT4, whose streaming variant spills registers and
    // measured slower than one wavefront per partition (269 vs 261 us on
    // the 131K-token batch)
    a.stream_fixed = !balanced && a.cus > 0 && !fixed_grid_forced() && ce != Elem::I4 &&
                     (long long)num_seqs * num_q_heads * l.max_parts < INT32_MAX;
  }
  if (num_seqs == 0) return PA_OK;
  if (log_enabled())
    std::fprintf(stderr, "[pagedattn] decode path=%s S=%d Hq=%d Hkv=%d G=%d D=%d B=%d P=%d parts=%d cus=%d append=%s\n",
                 use_mfma ? "mfma" : "valu", num_seqs, num_q_heads, num_kv_heads, group, head_dim,
                 block_size, partition_size, a.max_parts, a.cus,
                 fuse_append ? "in the decode launch" : (append ? "separate launch" : "no"));
  if (fuse_append) {
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_pool_w = k_pool_w;
    a.v_pool_w = v_pool_w;
  } else if (append) {
    pa::WriteArgs w;
    std::memset(&w, 0, sizeof w);
    w.k_new = k_new; w.v_new = v_new;
    w.k_cache = k_pool_w; w.v_cache = v_pool_w;
    w.tables = block_tables; w.lens = context_lens;
    w.k_scale = k_scale; w.v_scale = v_scale;
    w.num_slots = num_blocks * block_size;
    w.num_tokens = num_seqs; w.num_kv_heads = num_kv_heads;
    w.max_blocks = max_blocks_per_seq; w.max_len = max_context_len;
    w.zero_counters = a.counters;  // the decode below counts arrivals from zero
    w.num_counters = num_counters;
    const hipError_t e = pa::launch_cache_write(w, se, ce, head_dim, block_size, stream);
    if (e != hipSuccess) return from_hip(e);
  }
  hipError_t e = use_mfma ? pa::launch_decode_mfma(a, ce, head_dim, block_size, stream)
                          : pa::launch_decode_valu(a, qe, ce, head_dim, block_size, stream);
  return from_hip(e);
}

}  // namespace

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, int max_blocks_per_seq,
                    const int32_t* context_lens, int max_context_len, int num_seqs,
                    int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                    int64_t num_blocks, float scale, pa_dtype q_dtype, pa_dtype cache_dtype,
                    const float* k_scale, const float* v_scale, int partition_size,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(out, q, nullptr, nullptr, nullptr, nullptr, k_cache, v_cache, block_tables,
                     max_blocks_per_seq,
                     context_lens, max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                     block_size, num_blocks, scale, q_dtype, PA_BF16, cache_dtype, k_scale, v_scale,
                     partition_size, workspace, workspace_bytes, stream);
}

pa_status pa_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                           void* k_cache, void* v_cache, const int32_t* block_tables,
                           int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int block_size, int64_t num_blocks, float scale, pa_dtype q_dtype,
                           pa_dtype src_dtype, pa_dtype cache_dtype, const float* k_scale,
                           const float* v_scale, int partition_size, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (!k_new || !v_new) return PA_ERR_INVALID_ARG;
  return decode_impl(out, q, k_new, v_new, k_cache, v_cache, k_cache, v_cache, block_tables,
                     max_blocks_per_seq,
                     context_lens, max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                     block_size, num_blocks, scale, q_dtype, src_dtype, cache_dtype, k_scale, v_scale,
                     partition_size, workspace, workspace_bytes, stream);
}

pa_status pa_decode_reduce(void* out, const void* workspace, size_t workspace_bytes,
                           const int32_t* context_lens, int max_context_len, int num_seqs,
                           int num_q_heads, int num_kv_heads, int head_dim, int partition_size,
                           pa_dtype out_dtype, hipStream_t stream) {
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || max_context_len < 0 ||
      (partition_size <= 0 && partition_size != PA_PARTITION_AUTO &&
       partition_size != PA_PARTITION_AUTO_MERGED))
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  Elem oe;
  if (!to_elem(out_dtype, &oe)) return PA_ERR_INVALID_ARG;
  if (is_fp8(oe) || !supported_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  if (partition_size > 0 && partition_size % kStepTokens != 0) return PA_ERR_UNSUPPORTED;
  if (num_seqs > 65535) return PA_ERR_UNSUPPORTED;
  if (num_q_heads / num_kv_heads > 16 && partition_size < 0) return PA_ERR_UNSUPPORTED;
  if (!out || !workspace || !context_lens) return PA_ERR_INVALID_ARG;
  Layout l;
  if (!workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                        partition_size, &l))
    return partition_size < 0 ? PA_ERR_HIP : PA_ERR_INVALID_ARG;
  if (workspace_bytes < l.total || (reinterpret_cast<uintptr_t>(workspace) & 255)) return PA_ERR_WORKSPACE;
  if (num_seqs == 0 || partition_size == PA_PARTITION_AUTO_MERGED) return PA_OK;  // merged by the decode
  const char* w = static_cast<const char*>(workspace);
  pa::ReduceArgs a;
  std::memset(&a, 0, sizeof a);
  a.out = out;
  a.header = reinterpret_cast<const int*>(w);
  w += l.head_bytes;
  a.part_out = reinterpret_cast<const float*>(w);
  a.part_max = reinterpret_cast<const float*>(w + l.out_bytes);
  a.part_sum = reinterpret_cast<const float*>(w + l.out_bytes + l.max_bytes);
  a.context_lens = context_lens;
  a.max_len = max_context_len;
  a.num_seqs = num_seqs; a.num_q_heads = num_q_heads; a.num_kv_heads = num_kv_heads;
  a.partition = partition_size; a.max_parts = l.max_parts; a.slices_max = l.slices_max;
  if (partition_size == PA_PARTITION_AUTO)
    return from_hip(pa::launch_auto_fixup(a, oe, head_dim, stream));
  return from_hip(pa::launch_reduce(a, oe, head_dim, stream));
}

pa_status pa_prefill_chunk(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, int max_blocks_per_seq,
                           const int32_t* context_lens, int max_context_len,
                           const int32_t* query_start, int num_query_tokens, int max_query_len,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int block_size, int64_t num_blocks, float scale, pa_dtype q_dtype,
                           pa_dtype cache_dtype, const float* k_scale, const float* v_scale,
                           int partition_size, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  if (num_seqs < 0 || num_query_tokens < 0 || max_query_len < 0 || num_q_heads < 1 ||
      num_kv_heads < 1 || max_context_len < 0 || max_blocks_per_seq < 1 || num_blocks < 1 ||
      partition_size < 0)
    return (partition_size == PA_PARTITION_AUTO || partition_size == PA_PARTITION_AUTO_MERGED)
               ? PA_ERR_UNSUPPORTED : PA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (!(std::isfinite(scale) && scale > 0.0f)) return PA_ERR_INVALID_ARG;
  Elem qe, ce;
  if (!to_elem(q_dtype, &qe) || !to_elem(cache_dtype, &ce)) return PA_ERR_INVALID_ARG;
  if (!supported_dim(head_dim) || !supported_block(block_size)) return PA_ERR_UNSUPPORTED;
  if (qe != Elem::BF16 || ce == Elem::F32) return PA_ERR_UNSUPPORTED;
  if (partition_size > 0 && partition_size % kStepTokens != 0) return PA_ERR_UNSUPPORTED;
  const int group = num_q_heads / num_kv_heads;
  if (group > 16 || (group & (group - 1)) != 0) return PA_ERR_UNSUPPORTED;
  {  // one workgroup per (partition, query tile, KV head, sequence), padded to whole XCD rounds
    const long long tiles = pa::prefill_query_tiles(group, max_query_len,
                                                    pa::prefill_max_column_tiles(ce, head_dim));
    const long long parts = partition_size > 0
        ? std::max(1LL, ((long long)max_context_len + partition_size - 1) / partition_size) : 1;
    const long long pairs = ((long long)num_seqs * num_kv_heads + pa::kXcds - 1) / pa::kXcds * pa::kXcds;
    if (num_seqs > 65535 || pairs * parts * tiles > INT32_MAX) return PA_ERR_UNSUPPORTED;
  }
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PA_ERR_INVALID_ARG;
  if (partition_size == 0 && !out) return PA_ERR_INVALID_ARG;
  if (is_fp8(ce) && (!k_scale || !v_scale)) return PA_ERR_INVALID_ARG;

  pa::PrefillArgs p;
  std::memset(&p, 0, sizeof p);
  pa::DecodeArgs& a = p.d;
  a.out = out; a.q = q; a.k_cache = k_cache; a.v_cache = v_cache;
  a.block_tables = block_tables; a.context_lens = context_lens;
  a.k_scale = k_scale; a.v_scale = v_scale;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  const long long cap = (long long)max_blocks_per_seq * block_size;
  a.cap_len = (int)std::min<long long>(cap, INT32_MAX);
  a.max_len = max_context_len;  // as the decode: pa_prefill_reduce counts partitions alike
  a.num_seqs = num_seqs; a.num_q_heads = num_q_heads; a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.partition = partition_size;
  a.scale = scale;
  a.max_parts = 1;
  p.query_start = query_start;
  p.max_query_len = max_query_len;
  if (partition_size > 0) {
    Layout l;
    if (!workspace_layout(num_query_tokens, num_q_heads, num_kv_heads, head_dim, max_context_len,
                          partition_size, &l))
      return PA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < l.total || (reinterpret_cast<uintptr_t>(workspace) & 255))
      return PA_ERR_WORKSPACE;
    char* w = static_cast<char*>(workspace);
    a.part_out = reinterpret_cast<float*>(w);
    a.part_max = reinterpret_cast<float*>(w + l.out_bytes);
    a.part_sum = reinterpret_cast<float*>(w + l.out_bytes + l.max_bytes);
    a.max_parts = l.max_parts;
  }
  if (num_seqs == 0 || max_query_len == 0 || num_query_tokens == 0) return PA_OK;
  return from_hip(pa::launch_prefill_mfma(p, ce, head_dim, block_size, stream));
}

pa_status pa_prefill_reduce(void* out, const void* workspace, size_t workspace_bytes,
                            const int32_t* context_lens, int max_context_len,
                            const int32_t* query_start, int num_query_tokens, int max_query_len,
                            int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                            int partition_size, pa_dtype out_dtype, hipStream_t stream) {
  if (num_seqs < 0 || num_query_tokens < 0 || max_query_len < 0 || num_q_heads < 1 ||
      num_kv_heads < 1 || max_context_len < 0 || partition_size <= 0)
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  Elem oe;
  if (!to_elem(out_dtype, &oe)) return PA_ERR_INVALID_ARG;
  if (is_fp8(oe) || !supported_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  if (partition_size % kStepTokens != 0) return PA_ERR_UNSUPPORTED;
  if (num_seqs > 65535 || max_query_len > 65535) return PA_ERR_UNSUPPORTED;
  if (!out || !workspace || !context_lens || !query_start) return PA_ERR_INVALID_ARG;
  Layout l;
  if (!workspace_layout(num_query_tokens, num_q_heads, num_kv_heads, head_dim, max_context_len,
                        partition_size, &l))
    return PA_ERR_INVALID_ARG;
  if (workspace_bytes < l.total || (reinterpret_cast<uintptr_t>(workspace) & 255)) return PA_ERR_WORKSPACE;
  if (num_seqs == 0 || max_query_len == 0 || num_query_tokens == 0) return PA_OK;
  const char* w = static_cast<const char*>(workspace);
  pa::ReduceArgs a;
  std::memset(&a, 0, sizeof a);
  a.out = out;
  a.part_out = reinterpret_cast<const float*>(w);
  a.part_max = reinterpret_cast<const float*>(w + l.out_bytes);
  a.part_sum = reinterpret_cast<const float*>(w + l.out_bytes + l.max_bytes);
  a.context_lens = context_lens;
  a.max_len = max_context_len;
  a.num_seqs = num_seqs; a.num_q_heads = num_q_heads; a.num_kv_heads = num_kv_heads;
  a.partition = partition_size; a.max_parts = l.max_parts;
  a.query_start = query_start;
  a.max_query_len = max_query_len;
  return from_hip(pa::launch_reduce(a, oe, head_dim, stream));
}

// ---------------------------------------------------------------------------
// pa_decode_noalloc: the balanced split's workspace in a static device array
// ---------------------------------------------------------------------------

}  // extern "C"

// Scratch for pa_decode_noalloc.  Each GPU the library runs on holds its own
// copy at its own address, until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address is
// looked up per device (hipGetSymbolAddress) and only that address is used.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current.
pa_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return from_hip(e != hipSuccess ? e : hipErrorInvalidSymbol);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_decode_noalloc(void* out, const void* q, const void* k_new,
                                       const void* v_new, void* k_cache, void* v_cache,
                                       const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* context_lens, int max_context_len,
                                       int num_seqs, int num_q_heads, int num_kv_heads,
                                       int head_dim, int block_size, int64_t num_blocks,
                                       float scale, pa_dtype q_dtype, pa_dtype src_dtype,
                                       pa_dtype cache_dtype, const float* k_scale,
                                       const float* v_scale, hipStream_t stream) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens ||
      (k_new == nullptr) != (v_new == nullptr))
    return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
      max_context_len < 0 || num_q_heads % num_kv_heads != 0)
    return PA_ERR_INVALID_ARG;
  Layout l;
  if (!workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                        PA_PARTITION_AUTO, &l))
    return PA_ERR_HIP;  // the arguments passed above: the device could not be queried
  if (l.total > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  pa_status st = scratch_of_current_device(&ws);
  if (st != PA_OK) return st;
  st = decode_impl(out, q, k_new, v_new, k_cache, v_cache, k_cache, v_cache, block_tables,
                   max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                   num_kv_heads, head_dim, block_size, num_blocks, scale, q_dtype,
                   k_new ? src_dtype : PA_BF16, cache_dtype, k_scale, v_scale, PA_PARTITION_AUTO,
                   ws, PA_NOALLOC_SCRATCH_BYTES, stream);
  if (st != PA_OK) return st;
  return pa_decode_reduce(out, ws, PA_NOALLOC_SCRATCH_BYTES, context_lens, max_context_len,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, PA_PARTITION_AUTO,
                          q_dtype, stream);
}
