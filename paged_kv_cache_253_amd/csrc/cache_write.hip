// Slot-mapped append of new K/V rows into the paged pool.
//
// Token n goes to block slot / B at offset slot % B ("vLLM & High-Throughput
// Serving", section 2, block-table equation on a flat slot number), one row
// per KV head: one 16-byte piece per head-dimension chunk in the chunked K
// tile (element d at chunk d / X, lane d % X of the token, X elements = 16
// bytes), one element per dimension row in the dimension-major V tile.  Same-type caches copy bits;
// an FP8 cache stores the E4M3FN code of x / scale[h] (binary32 quotient,
// then nearest-even E4M3 or E5M2 with saturation).
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return (float)x; }

template <typename ST, Elem CE, int D, int BS>
__global__ __launch_bounds__(64) void cache_write_kernel(const WriteArgs a) {
  const int n = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t slot = a.slots[n];
  if (slot < 0 || slot >= a.num_slots) return;  // padding token, or out of the pool
  const int64_t blk = slot / BS;
  const int off = (int)(slot % BS);
  const int64_t tile = (blk * a.num_kv_heads + h) * (int64_t)(BS * D);  // in elements
  constexpr int X = CE == Elem::F32 ? 4 : (CE == Elem::BF16 ? 8 : 16);  // K chunk width
  auto kidx = [&](int d) { return ((d / X) * BS + off) * X + d % X; };
  const ST* kn = reinterpret_cast<const ST*>(a.k_new) + ((int64_t)n * a.num_kv_heads + h) * D;
  const ST* vn = reinterpret_cast<const ST*>(a.v_new) + ((int64_t)n * a.num_kv_heads + h) * D;
  if constexpr (CE == Elem::FP8 || CE == Elem::E5M2) {
    const float ks = a.k_scale[h], vs = a.v_scale[h];
    uint8_t* kc = reinterpret_cast<uint8_t*>(a.k_cache) + tile;
    uint8_t* vc = reinterpret_cast<uint8_t*>(a.v_cache) + tile;
    auto enc = [](float x) -> uint8_t {
      if constexpr (CE == Elem::E5M2) return (uint8_t)f32_to_e5m2_sat(x);
      else return (uint8_t)f32_to_e4m3_sat(x);
    };
    for (int d = threadIdx.x; d < D; d += 64) {
      kc[kidx(d)] = enc(__fdiv_rn(to_f32(kn[d]), ks));
      vc[d * BS + off] = enc(__fdiv_rn(to_f32(vn[d]), vs));
    }
  } else {
    ST* kc = reinterpret_cast<ST*>(a.k_cache) + tile;
    ST* vc = reinterpret_cast<ST*>(a.v_cache) + tile;
    for (int d = threadIdx.x; d < D; d += 64) {
      kc[kidx(d)] = kn[d];
      vc[d * BS + off] = vn[d];
    }
  }
}

template <typename ST, Elem CE, int D, int BS>
hipError_t launch(const WriteArgs& a, hipStream_t s) {
  dim3 grid(a.num_tokens, a.num_kv_heads);
  hipLaunchKernelGGL((cache_write_kernel<ST, CE, D, BS>), grid, dim3(64), 0, s, a);
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
  return hipErrorInvalidValue;
}

}  // namespace pa
