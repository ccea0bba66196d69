// Slot-mapped append of new K/V rows into the paged pool.
//
// Token n goes to block slot / B at offset slot % B ("vLLM & High-Throughput
// Serving", section 2, block-table equation on a flat slot number), one row
// per KV head: one 16-byte piece per head-dimension chunk in the chunked K
// tile (element d at chunk d / X, lane d % X of the token, X elements = 16
// bytes), one element per dimension row in the dimension-major V tile.
// Same-type caches copy bits; FP8 caches store the E4M3FN or E5M2 code of
// x / scale[h]; an INT4 cache gives every (token, KV head) row its own scale
// absmax / 7 (the encodings are in pa_append.hpp).
#include "pa_append.hpp"
#include "pa_device.hpp"
#include "pa_internal.hpp"
#include "pa_split.hpp"

namespace pa {
namespace {

// One wavefront per (token, KV head).  All of a lane's loads (its share of
// the new rows, and the slot) are issued before the first store, so the
// wavefront waits for one memory round trip.  FROM_TABLE: token n is
// sequence n's newest token and its slot comes from the block table.
template <typename ST, Elem CE, int D, int BS, bool FROM_TABLE>
__global__ __launch_bounds__(64) void cache_write_kernel(const WriteArgs a) {
  const int n = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  if (a.zero_counters) {  // the following decode launch's merge counters
    const int stride = gridDim.x * gridDim.y * 64;
    for (int i = (h * gridDim.x + n) * 64 + lane; i < a.num_counters; i += stride) a.zero_counters[i] = 0;
  }
  const ST* kn = reinterpret_cast<const ST*>(a.k_new) + ((int64_t)n * a.num_kv_heads + h) * D;
  const ST* vn = reinterpret_cast<const ST*>(a.v_new) + ((int64_t)n * a.num_kv_heads + h) * D;
  NewRow<ST> row;
  load_row<ST, CE, D>(row, kn, vn, lane);
  int64_t slot;
  if constexpr (FROM_TABLE)
    slot = newest_slot<BS>(a.tables, a.max_blocks, clamp_len(a.lens[n], a.max_len), n,
                           a.num_slots / BS);
  else
    slot = a.slots[n];
  if (slot < 0 || slot >= a.num_slots) return;  // padding token, or out of the pool
  const int64_t blk = slot / BS;
  const int off = (int)(slot % BS);
  const int64_t tile = (blk * a.num_kv_heads + h) * tile_bytes(CE, D, BS);
  const bool fp8 = CE == Elem::FP8 || CE == Elem::E5M2;
  store_row<ST, CE, D, BS>(row, reinterpret_cast<char*>(a.k_cache) + tile,
                           reinterpret_cast<char*>(a.v_cache) + tile, off,
                           fp8 ? a.k_scale[h] : 0.f, fp8 ? a.v_scale[h] : 0.f, lane);
}

template <typename ST, Elem CE, int D, int BS>
hipError_t launch(const WriteArgs& a, hipStream_t s) {
  dim3 grid(a.num_tokens, a.num_kv_heads);
  if (a.tables)
    hipLaunchKernelGGL((cache_write_kernel<ST, CE, D, BS, true>), grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((cache_write_kernel<ST, CE, D, BS, false>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

template <typename ST, Elem CE>
hipError_t by_shape(const WriteArgs& a, int head_dim, int block_size, hipStream_t s) {
  if (head_dim == 128 && block_size == 16) return launch<ST, CE, 128, 16>(a, s);
  if (head_dim == 128 && block_size == 32) return launch<ST, CE, 128, 32>(a, s);
  if (head_dim == 64 && block_size == 16) return launch<ST, CE, 64, 16>(a, s);
  if (head_dim == 64 && block_size == 32) return launch<ST, CE, 64, 32>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_cache_write(const WriteArgs& a, Elem src, Elem cache, int head_dim,
                              int block_size, hipStream_t stream) {
  if (src == Elem::F32 && cache == Elem::F32) return by_shape<float, Elem::F32>(a, head_dim, block_size, stream);
  if (src == Elem::BF16 && cache == Elem::BF16) return by_shape<__bf16, Elem::BF16>(a, head_dim, block_size, stream);
  if (src == Elem::F32 && cache == Elem::FP8) return by_shape<float, Elem::FP8>(a, head_dim, block_size, stream);
  if (src == Elem::BF16 && cache == Elem::FP8) return by_shape<__bf16, Elem::FP8>(a, head_dim, block_size, stream);
  if (src == Elem::F32 && cache == Elem::E5M2) return by_shape<float, Elem::E5M2>(a, head_dim, block_size, stream);
  if (src == Elem::BF16 && cache == Elem::E5M2) return by_shape<__bf16, Elem::E5M2>(a, head_dim, block_size, stream);
  if (src == Elem::F32 && cache == Elem::I4) return by_shape<float, Elem::I4>(a, head_dim, block_size, stream);
  if (src == Elem::BF16 && cache == Elem::I4) return by_shape<__bf16, Elem::I4>(a, head_dim, block_size, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
