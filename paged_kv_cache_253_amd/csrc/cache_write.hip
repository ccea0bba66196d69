// Slot-mapped append of new K/V rows into the paged pool.
//
// Token n goes to block slot / B at offset slot % B ("vLLM & High-Throughput
// Serving", section 2, block-table equation on a flat slot number), one row
// per KV head: one 16-byte piece per head-dimension chunk in the chunked K
// tile (element d at chunk d / X, lane d % X of the token, X elements = 16
// bytes), one element per dimension row in the dimension-major V tile.  Same-type caches copy bits;
// an FP8 cache stores the E4M3FN code of x / scale[h] (binary32 quotient,
// then nearest-even E4M3 or E5M2 with saturation).  An INT4 cache gives
// every (token, KV head) row its own scale absmax / 7 and stores the
// nearest-even codes of x / scale (cache_write_i4).
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

// INT4 append: one wavefront per (token, KV head).  Lane l (l < D/2) owns
// byte l%4 of octet l/4 of the row, i.e. elements e = 8*(l/4) + l%4 and
// e + 4.  The row's absmax is an all-reduce over the wavefront.  K bytes
// belong to this token alone and are stored whole; a V byte holds two
// tokens (one nibble each), so V nibbles are replaced with atomic AND/OR
// on their 32-bit word, which lets tokens of one octet be appended in the
// same launch.
template <typename ST, int D, int BS>
__global__ __launch_bounds__(64) void cache_write_i4(const WriteArgs a) {
  const int n = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t slot = a.slots[n];
  if (slot < 0 || slot >= a.num_slots) return;  // padding token, or out of the pool
  const int64_t blk = slot / BS;
  const int off = (int)(slot % BS);
  constexpr int kCodeBytes = BS * D / 2;
  const int64_t tile = (blk * a.num_kv_heads + h) * (int64_t)(BS * (D / 2 + 4));  // bytes
  const ST* kn = reinterpret_cast<const ST*>(a.k_new) + ((int64_t)n * a.num_kv_heads + h) * D;
  const ST* vn = reinterpret_cast<const ST*>(a.v_new) + ((int64_t)n * a.num_kv_heads + h) * D;
  const int lane = threadIdx.x;
  const bool act = lane < D / 2;
  const int e0 = 8 * (lane >> 2) + (lane & 3);
  const float k0 = act ? to_f32(kn[e0]) : 0.f, k1 = act ? to_f32(kn[e0 + 4]) : 0.f;
  const float v0 = act ? to_f32(vn[e0]) : 0.f, v1 = act ? to_f32(vn[e0 + 4]) : 0.f;
  const float kmax = xlane<OpMax, 1, 32>(fmaxf(fabsf(k0), fabsf(k1)));
  const float vmax = xlane<OpMax, 1, 32>(fmaxf(fabsf(v0), fabsf(v1)));
  const float ks = __fdiv_rn(kmax, 7.0f), vs = __fdiv_rn(vmax, 7.0f);
  auto code = [](float x, float s) -> uint32_t { return s > 0.f ? (uint32_t)i4_code(x, s) & 15u : 0u; };
  uint8_t* kc = reinterpret_cast<uint8_t*>(a.k_cache) + tile;
  uint8_t* vc = reinterpret_cast<uint8_t*>(a.v_cache) + tile;
  if (act) {
    // K: octet o = lane/4 holds dimensions 8o .. 8o+7, in chunk row o/4 at
    // bytes 4*(o%4) .. of the token's 16 bytes
    const int o = lane >> 2;
    kc[((o >> 2) * BS + off) * 16 + 4 * (o & 3) + (lane & 3)] = (uint8_t)(code(k0, ks) | (code(k1, ks) << 4));
    // V: dimension rows e0 and e0 + 4; the token is element off % 8 of octet
    // off / 8 of the row: byte (off % 8) % 4, high nibble iff off % 8 >= 4
    const int shift = 8 * ((off & 7) & 3) + 4 * ((off & 7) >> 2);
    const uint32_t mask = ~(15u << shift);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = e0 + 4 * j;
      uint32_t* w = reinterpret_cast<uint32_t*>(vc + row * (BS / 2) + (off >> 3) * 4);
      atomicAnd(w, mask);
      atomicOr(w, code(j ? v1 : v0, vs) << shift);
    }
  }
  if (lane == 0) {
    reinterpret_cast<float*>(kc + kCodeBytes)[off] = ks;
    reinterpret_cast<float*>(vc + kCodeBytes)[off] = vs;
  }
}

template <typename ST, Elem CE, int D, int BS>
hipError_t launch(const WriteArgs& a, hipStream_t s) {
  dim3 grid(a.num_tokens, a.num_kv_heads);
  if constexpr (CE == Elem::I4)
    hipLaunchKernelGGL((cache_write_i4<ST, D, BS>), grid, dim3(64), 0, s, a);
  else
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
  if (src == Elem::F32 && cache == Elem::I4) return by_shape<float, Elem::I4>(a, head_dim, block_size, stream);
  if (src == Elem::BF16 && cache == Elem::I4) return by_shape<__bf16, Elem::I4>(a, head_dim, block_size, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
