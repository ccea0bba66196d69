// Internal interface between the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum class Elem : int { F32 = 0, BF16 = 1, FP8 = 2 };

// Everything a decode launch needs; passed by value as the kernel argument.
struct DecodeArgs {
  void* out;                    // [S][Hq][D] q type (unsplit launches)
  const void* q;                // [S][Hq][D]
  const void* k_cache;          // [nb][Hkv][B][D]
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
  int max_len;                  // clamp for context_lens (host bound and table capacity)
  int num_seqs, num_q_heads, num_kv_heads, group;
  int partition;                // tokens per partition, 0 = unsplit
  int max_parts;                // partitions per sequence slot in the workspace
  float scale;
};

struct WriteArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int64_t* slots;
  const float* k_scale;
  const float* v_scale;
  int64_t num_slots;            // num_blocks * block_size
  int num_tokens, num_kv_heads;
};

struct ReduceArgs {
  void* out;
  const float* part_out;
  const float* part_max;
  const float* part_sum;
  const int32_t* context_lens;
  int max_len, num_seqs, num_q_heads, partition, max_parts;
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

}  // namespace pa
