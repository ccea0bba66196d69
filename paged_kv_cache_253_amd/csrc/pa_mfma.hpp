// Matrix-core operand helpers shared by the paged attention kernels
// (gfx950, wave64, v_mfma_f32_16x16x32_bf16).
//
// MFMA operand layouts (16x16x32, wave64; checked on hardware): lane l holds
// row/column l % 16 and k-slots 8*(l/16) .. 8*(l/16)+7 of A and B; the f32
// result row is 4*(l/16) + r (r = 0..3), column l % 16.
//
// A 32-token step is two QK groups: group m holds tokens 16m .. 16m+15 as
// its rows, so the A operand of one head-dim chunk is 16 tokens x 4 chunk
// rows of the chunked K tile (one contiguous KiB at block size 16).  Lane l
// then holds the scores of tokens 4*(l/16) + r and 16 + 4*(l/16) + r (r =
// 0..3), while its PV k-slots need tokens 8*(l/16) .. +7: p_operand moves
// them there with two lane swaps.
#pragma once

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace mfma {

constexpr int kStep = 32;  // tokens per step

// Cache element kinds of the matrix-core kernels.  The two FP8 kinds share
// the 1-byte layout and differ only in how a code widens to bf16.
constexpr int kBF16 = 0, kE4M3 = 1, kE5M2 = 2;
template <int CK>
constexpr bool one_byte() { return CK != kBF16; }

template <int CK, int D, int BS>
struct Cfg {
  static constexpr bool FP8 = one_byte<CK>();
  static constexpr int kElt = FP8 ? 1 : 2;
  static constexpr int kChunks = D / 32;            // QK MFMAs per token group
  static constexpr int kDTiles = D / 16;            // PV MFMAs per step
  static constexpr int kKLoads = FP8 ? D / 64 : D / 32;  // 16-byte K loads per token group
  static constexpr int kChunkRow = BS * 16;         // bytes of one K chunk row (16 B per token)
  static constexpr int kRowV = BS * kElt;           // bytes of one V row (dimension)
  static constexpr int kTile = BS * D * kElt;       // bytes of one (block, head) tile
  static constexpr int kBlocksPerStep = kStep / BS;
};

template <bool FP8>
struct VRaw;
template <>
struct VRaw<false> { u32x4 w; };  // 8 bf16 tokens
template <>
struct VRaw<true> { u32x2 w; };   // 8 e4m3 tokens

template <int CK, int D, int BS>
struct StepBuf {
  using C = Cfg<CK, D, BS>;
  u32x4 k[2][C::kKLoads];
  VRaw<C::FP8> v[C::kDTiles];
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

// 8 FP8 codes of kind CK (two words) -> 8 bf16, order kept (exact)
template <int CK>
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  bf16x2 a, b, c, d;
  if constexpr (CK == kE5M2) {
    bf8x4_to_bf16(w0, a, b);
    bf8x4_to_bf16(w1, c, d);
  } else {
    fp8x4_to_bf16(w0, a, b);
    fp8x4_to_bf16(w1, c, d);
  }
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// K operand of QK chunk c for token group m (from a buffer with k[2][..])
template <int CK, class Buf>
__device__ __forceinline__ bf16x8 k_operand(const Buf& sb, int m, int c) {
  if constexpr (one_byte<CK>()) {
    const u32x4 w = sb.k[m][c >> 1];
    return (c & 1) ? fp8x8_to_bf16x8<CK>(w[2], w[3]) : fp8x8_to_bf16x8<CK>(w[0], w[1]);
  } else {
    return as_bf16x8(sb.k[m][c]);
  }
}

// Softmax weights in QK register order (p[0..3]: tokens 4*grp + r, p[4..7]:
// tokens 16 + 4*grp + r) -> PV B operand in k-slot order (tokens 8*grp ..
// 8*grp + 7).  Packed bf16 pairs A (first four) and B (last four) of lanes
// in rows 0..3 are exchanged: permlane32_swap leaves rows 0,1 with A of
// rows {0,2},{1,3} and rows 2,3 with B of rows {0,2},{1,3}; permlane16_swap
// then gives row k the two quarters of tokens 8k .. 8k + 7.
__device__ __forceinline__ bf16x8 p_operand(const float* p) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bf16x2 t;
    t[0] = (__bf16)p[2 * i];
    t[1] = (__bf16)p[2 * i + 1];
    w[i] = __builtin_bit_cast(uint32_t, t);
  }
  const auto x0 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
  const auto x1 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
  const auto y0 = __builtin_amdgcn_permlane16_swap(x0[0], x0[1], false, false);
  const auto y1 = __builtin_amdgcn_permlane16_swap(x1[0], x1[1], false, false);
  const u32x4 r = {y0[0], y1[0], y0[1], y1[1]};
  return __builtin_bit_cast(bf16x8, r);
}

// The token of QK result register i (0..7) of lane row grp, within a step.
__device__ __forceinline__ int qk_token(int grp, int i) { return 4 * grp + (i & 3) + 16 * (i >> 2); }

template <int CK>
__device__ __forceinline__ bf16x8 v_operand(const VRaw<one_byte<CK>()>& r) {
  if constexpr (one_byte<CK>()) return fp8x8_to_bf16x8<CK>(r.w[0], r.w[1]);
  else return as_bf16x8(r.w);
}

// Zero the V elements of k-slots whose token is past the range end.
template <bool FP8>
__device__ __forceinline__ void mask_v(VRaw<FP8>& r, int valid) {  // valid = tokens kept, 0..8
  if constexpr (FP8) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      int n = valid - 4 * w;
      uint32_t keep = n >= 4 ? 0xffffffffu : (n <= 0 ? 0u : (0xffffffffu >> (32 - 8 * n)));
      r.w[w] &= keep;
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      int n = valid - 2 * w;
      uint32_t keep = n >= 2 ? 0xffffffffu : (n == 1 ? 0x0000ffffu : 0u);
      r.w[w] &= keep;
    }
  }
}

}  // namespace mfma
}  // namespace pa
