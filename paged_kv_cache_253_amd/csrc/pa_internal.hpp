// Internal interface between the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Element types: FP8 is E4M3FN, E5M2 the other FP8 format, I4 the 4-bit
// integer codes with a float32 scale per (token, KV head) in each tile.
enum class Elem : int { F32 = 0, BF16 = 1, FP8 = 2, E5M2 = 3, I4 = 4 };
inline bool is_fp8(Elem e) { return e == Elem::FP8 || e == Elem::E5M2; }

// Bytes of one (block, KV head) tile of a pool.
__host__ __device__ constexpr int64_t tile_bytes(Elem e, int head_dim, int block_size) {
  if (e == Elem::I4) return (int64_t)block_size * (head_dim / 2 + 4);
  const int elt = e == Elem::F32 ? 4 : (e == Elem::BF16 ? 2 : 1);
  return (int64_t)block_size * head_dim * elt;
}

// Balanced split: most persistent wavefronts per compute unit any decode
// kernel uses (sizes the workspace and the merge grid), minimum slice length
// in 32-token steps, and the XCD count used to group slices.
constexpr int kAutoMaxWavesPerCU = 8;
constexpr int kAutoMinSteps = 4;
constexpr int kXcds = 8;
// Balanced-split workspace header: the decode's wavefront count W as the
// int32 at word kHdrSlices, then from byte kHdrRecordsBytes one 16-byte
// merge record per slice (see pa_split.hpp), then (256-byte aligned) one
// int32 arrival counter per slice for the merge inside the decode launch
// (see pa_merge.hpp).
constexpr int kHdrSlices = 0;
constexpr int kHdrRecordsBytes = 256;
constexpr int kMergeRecordBytes = 16;

// Split modes (DecodeArgs::partition): > 0 fixed partitions of that many
// tokens, 0 unsplit, kAuto balanced slices (the merge inside the decode
// launch when DecodeArgs::counters is set).
constexpr int kAuto = -1;
constexpr int kAutoMerged = -2;  // ABI value of the balanced split merged in the decode launch

// Everything a decode launch needs; passed by value as the kernel argument.
struct DecodeArgs {
  void* out;                    // [S][Hq][D] q type (unsplit launches)
  const void* q;                // [S][Hq][D]
  const void* k_cache;          // [nb][Hkv][D/X][B][X], X elements = 16 bytes
  const void* v_cache;          // [nb][Hkv][D][B]
  const int32_t* block_tables;  // [S][max_blocks]
  const int32_t* context_lens;  // [S]
  const float* k_scale;         // [Hkv] (FP8 cache) or null
  const float* v_scale;
  float* part_out;              // [S][Hq][max_parts][D] (split launches)
  float* part_max;              // [S][Hq][max_parts]
  float* part_sum;
  int64_t num_blocks;
  int max_blocks;               // table row length
  int max_len;                  // clamp for context_lens when planning ranges
  int cap_len;                  // tokens the table rows can address (max_blocks * B)
  int num_seqs, num_q_heads, num_kv_heads, group;
  int partition;                // tokens per partition, 0 = unsplit, kAuto = balanced
  int max_parts;                // partitions per sequence slot in the workspace
  int slices;                   // balanced split: persistent wavefronts (set by the launcher)
  int cus;                      // balanced split: compute units of the device
  int waves_per_cu;             // balanced split: 0 = the kernel's own choice
  int stream_fixed;             // fixed partitions on the persistent streaming grid (matrix-core
                                // kernels; else one wavefront per partition)
  int* header;                  // balanced split: workspace header (W, merge records)
  const void* k_new;            // [S][Hkv][D] bf16: the decode launch appends each sequence's
  const void* v_new;            // newest token itself (bf16 cache, balanced split); else null
  void* k_pool_w;               // with k_new: the pools the rows go to (k_cache, v_cache)
  void* v_pool_w;
  int* counters;                // balanced split merged in the decode launch: [slices_max]
                                // arrival counters, zero on entry and on exit; else null
  float scale;
};

// Several query tokens per sequence: sequence b's query rows are
// query_start[b] .. query_start[b+1]-1 of q / out (its last cached tokens).
// d.num_seqs is the sequence count; d.out, d.q and the partial states are
// indexed by query row instead of sequence.
struct PrefillArgs {
  DecodeArgs d;
  const int32_t* query_start;   // [S + 1]
  int max_query_len;
  int tiles;                    // query tiles per (sequence, KV head) (set by the launcher)
};

// Column tiles (16 MFMA columns each) of a multi-query wavefront, and the
// query tiles of a sequence, for group size G and the longest query run.
// A bf16 cache with head_dim 128 stops at 2 column tiles (4 would spill).
inline int prefill_max_column_tiles(Elem cache, int head_dim) {
  return ((cache == Elem::BF16 || cache == Elem::I4) && head_dim == 128) ? 2 : 4;
}
inline int prefill_column_tiles(int group, int max_query_len, int max_tiles) {
  const long long cols = (long long)group * max_query_len;
  const int nt = cols <= 16 ? 1 : (cols <= 32 ? 2 : 4);
  return nt < max_tiles ? nt : max_tiles;
}
inline int prefill_query_tiles(int group, int max_query_len, int max_tiles) {
  const int rows_per_tile = 16 * prefill_column_tiles(group, max_query_len, max_tiles) / group;
  return (max_query_len + rows_per_tile - 1) / rows_per_tile;
}

// Chunked prefill with query runs long enough to fill a workgroup of the
// LDS-shared kernel (bf16 caches; prefill_lds.hip).
bool prefill_uses_lds(Elem cache, int group, int max_query_len);
hipError_t launch_prefill_lds(const PrefillArgs& p, int head_dim, int block_size, hipStream_t stream);

struct WriteArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int64_t* slots;         // per token, or null: token n is sequence n's newest token
  const int32_t* tables;        // with slots null: [num_tokens][max_blocks] block tables
  const int32_t* lens;          // with slots null: [num_tokens] context lengths (incl. the new token)
  const float* k_scale;
  const float* v_scale;
  int64_t num_slots;            // num_blocks * block_size
  int num_tokens, num_kv_heads;
  int max_blocks, max_len;      // with slots null: table row length, clamp for lens
  int* zero_counters;           // if set: [num_counters] ints cleared by this launch (the
  int num_counters;             // merge counters of the decode launch that follows)
};

// Whole-block copies from (src_k, src_v) to (dst_k, dst_v): the same pools
// for copy-on-write, a device pool and a pinned host pool for swapping.
struct CopyArgs {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  const int64_t* mapping;       // [num_pairs][2] (src, dst) block ids
  int64_t src_blocks, dst_blocks;
  int64_t block_bytes;          // one block of one pool: Hkv tiles
  int num_pairs;
};

struct ReduceArgs {
  void* out;
  const float* part_out;
  const float* part_max;
  const float* part_sum;
  const int32_t* context_lens;
  int max_len, num_seqs, num_q_heads, num_kv_heads, partition, max_parts;
  int slices_max;               // balanced split: upper bound of the decode's wavefront count
  const int* header;            // balanced split: W and merge records written by the decode
  const int32_t* query_start;   // several query tokens per sequence: [S + 1], else null
  int max_query_len;
};

// Each launcher returns hipErrorInvalidValue for a shape it has no kernel
// for (the caller checks shapes first), else the launch status.
hipError_t launch_decode_mfma(const DecodeArgs& a, Elem cache, int head_dim, int block_size,
                              hipStream_t stream);
hipError_t launch_decode_valu(const DecodeArgs& a, Elem q, Elem cache, int head_dim,
                              int block_size, hipStream_t stream);
hipError_t launch_cache_write(const WriteArgs& a, Elem src, Elem cache, int head_dim,
                              int block_size, hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, Elem out, int head_dim, hipStream_t stream);
hipError_t launch_auto_fixup(const ReduceArgs& a, Elem out, int head_dim, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);
hipError_t launch_prefill_mfma(const PrefillArgs& a, Elem cache, int head_dim, int block_size,
                               hipStream_t stream);

}  // namespace pa
