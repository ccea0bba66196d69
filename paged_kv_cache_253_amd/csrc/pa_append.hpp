// Appending one new token's K and V rows (one KV head) into the tiles of its
// block ("vLLM & High-Throughput Serving", section 2: a token lives at offset
// slot % B of block slot / B), as one wavefront.
//
// Split in two so that a wavefront can issue the loads of several rows
// before it stores any (one memory round trip instead of one per row):
// load_row reads a lane's share of the row, store_row encodes and writes it.
//
// Encodings (the pool formats):
//  * same type (f32 / bf16 cache): bits copied; K chunk q (X elements = 16
//    bytes) of the token goes whole to chunk row q of the K tile.
//  * FP8 (E4M3FN or E5M2): code of x / scale[h] (binary32 quotient, nearest
//    even, saturating).
//  * INT4: the row gets its own scale absmax / 7 (binary32), codes are the
//    nearest-even quotients clamped to [-7, 7]; K octet o (dimensions 8o ..
//    8o+7) sits at bytes 4(o % 4) .. of the token's 16 bytes in chunk row
//    o / 4, dimension i's V nibble of token j at byte i·B/2 + (j / 8)·4 +
//    j % 4 (high nibble iff j % 8 >= 4), the scales after the codes.
#pragma once

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return (float)x; }

// A lane's share of one new row.  Same-type caches: K chunk `lane` (lanes <
// D / X) and V elements lane + 64 i.  FP8: K and V elements lane + 64 i.
// INT4: elements e0 and e0 + 4 of K and V, e0 = 8 (lane / 4) + lane % 4
// (lanes < D / 2; the others hold zeros).
template <typename ST>
struct NewRow {
  u32x4 kchunk;
  ST k[2], v[2];
};

template <Elem CE>
constexpr bool same_type_cache() { return CE == Elem::F32 || CE == Elem::BF16; }

template <typename ST, Elem CE, int D>
__device__ __forceinline__ void load_row(NewRow<ST>& r, const ST* kn, const ST* vn, int lane) {
  constexpr int PER = (D + 63) / 64;
  if constexpr (CE == Elem::I4) {
    const int e0 = 8 * (lane >> 2) + (lane & 3);
    const int ea = lane < D / 2 ? e0 : 0;  // every lane loads inside the row
    r.k[0] = kn[ea]; r.k[1] = kn[ea + 4];
    r.v[0] = vn[ea]; r.v[1] = vn[ea + 4];
  } else {
    if constexpr (same_type_cache<CE>()) {
      constexpr int X = 16 / (int)sizeof(ST);
      r.kchunk = *reinterpret_cast<const u32x4*>(kn + min(lane, D / X - 1) * X);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int d = min(lane + 64 * i, D - 1);  // clamped: no load is conditional
      if constexpr (!same_type_cache<CE>()) r.k[i] = kn[d];
      r.v[i] = vn[d];
    }
  }
}

// Store row r at offset `off` of the K and V tiles kt, vt (bytes) of its
// block and KV head.  ks, vs: the head's FP8 scales (ignored otherwise).
// Every lane of the wavefront must call it (INT4 reduces over the lanes).
template <typename ST, Elem CE, int D, int BS>
__device__ __forceinline__ void store_row(const NewRow<ST>& r, char* kt, char* vt, int off, float ks,
                                          float vs, int lane) {
  constexpr int PER = (D + 63) / 64;
  if constexpr (same_type_cache<CE>()) {
    constexpr int X = 16 / (int)sizeof(ST);
    ST* kc = reinterpret_cast<ST*>(kt);
    ST* vc = reinterpret_cast<ST*>(vt);
    if (lane < D / X) *reinterpret_cast<u32x4*>(kc + ((int64_t)lane * BS + off) * X) = r.kchunk;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int d = lane + 64 * i;
      if (d < D) vc[d * BS + off] = r.v[i];
    }
  } else if constexpr (CE == Elem::FP8 || CE == Elem::E5M2) {
    constexpr int X = 16;
    uint8_t* kc = reinterpret_cast<uint8_t*>(kt);
    uint8_t* vc = reinterpret_cast<uint8_t*>(vt);
    auto enc = [](float x) -> uint8_t {
      if constexpr (CE == Elem::E5M2) return (uint8_t)f32_to_e5m2_sat(x);
      else return (uint8_t)f32_to_e4m3_sat(x);
    };
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int d = lane + 64 * i;
      if (d < D) {
        kc[((d / X) * BS + off) * X + d % X] = enc(__fdiv_rn(to_f32(r.k[i]), ks));
        vc[d * BS + off] = enc(__fdiv_rn(to_f32(r.v[i]), vs));
      }
    }
  } else {  // INT4
    constexpr int kCodeBytes = BS * D / 2;
    const bool act = lane < D / 2;
    const int e0 = 8 * (lane >> 2) + (lane & 3);
    const float k0 = act ? to_f32(r.k[0]) : 0.f, k1 = act ? to_f32(r.k[1]) : 0.f;
    const float v0 = act ? to_f32(r.v[0]) : 0.f, v1 = act ? to_f32(r.v[1]) : 0.f;
    const float kmax = xlane<OpMax, 1, 32>(fmaxf(fabsf(k0), fabsf(k1)));
    const float vmax = xlane<OpMax, 1, 32>(fmaxf(fabsf(v0), fabsf(v1)));
    const float ksc = __fdiv_rn(kmax, 7.0f), vsc = __fdiv_rn(vmax, 7.0f);
    auto code = [](float x, float s) -> uint32_t { return s > 0.f ? (uint32_t)i4_code(x, s) & 15u : 0u; };
    uint8_t* kc = reinterpret_cast<uint8_t*>(kt);
    uint8_t* vc = reinterpret_cast<uint8_t*>(vt);
    if (act) {
      // K: octet o = lane / 4, byte lane % 4 of it
      const int o = lane >> 2;
      kc[((o >> 2) * BS + off) * 16 + 4 * (o & 3) + (lane & 3)] =
          (uint8_t)(code(k0, ksc) | (code(k1, ksc) << 4));
      // V: a byte holds two tokens, so the token's nibble is replaced with
      // atomic AND/OR on its 32-bit word (tokens of one octet may be
      // appended by different wavefronts at once)
      const int shift = 8 * ((off & 7) & 3) + 4 * ((off & 7) >> 2);
      const uint32_t mask = ~(15u << shift);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = e0 + 4 * j;
        uint32_t* w = reinterpret_cast<uint32_t*>(vc + row * (BS / 2) + (off >> 3) * 4);
        atomicAnd(w, mask);
        atomicOr(w, code(j ? v1 : v0, vsc) << shift);
      }
    }
    if (lane == 0) {
      reinterpret_cast<float*>(kc + kCodeBytes)[off] = ksc;
      reinterpret_cast<float*>(vc + kCodeBytes)[off] = vsc;
    }
  }
}

// Pool slot of sequence b's newest token (position L - 1, L = its context
// length clamped to [0, max_len]) from its block-table row, or -1 when it
// has none: L = 0, the position is past the row, or the entry is outside
// the pool.
template <int BS>
__device__ __forceinline__ int64_t newest_slot(const int32_t* tables, int max_blocks, int len,
                                               int b, int64_t num_blocks) {
  if (len <= 0) return -1;
  const int pos = len - 1;
  if (pos / BS >= max_blocks) return -1;
  const int p = tables[(int64_t)b * max_blocks + pos / BS];
  if (p < 0 || (int64_t)p >= num_blocks) return -1;
  return (int64_t)p * BS + pos % BS;
}

}  // namespace pa
