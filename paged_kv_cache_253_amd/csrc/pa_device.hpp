// Device-side helpers shared by the paged decode kernels (gfx950, wave64).
//
// Element types, exact widening conversions, the FP8 E4M3FN encoder used by
// the cache append, and cross-lane reductions built on DPP row operations
// and the gfx950 permlane swaps (no LDS round trip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// element conversions (all exact)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Four E4M3FN codes packed in a word -> four floats.  gfx950's converter
// reads the OCP E4M3FN format (checked on hardware against the format
// definition for all 256 codes).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* out) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  out[0] = lo[0]; out[1] = lo[1]; out[2] = hi[0]; out[3] = hi[1];
}

// Four E4M3FN codes -> four bf16 (exact: 3 mantissa bits fit in 7, and every
// E4M3 exponent including subnormals is a normal bf16 exponent).
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t w, bf16x2& lo, bf16x2& hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
}

// Four E5M2 codes packed in a word -> four floats / four bf16 (exact: every
// E5M2 value, subnormals and infinities included, is a bf16 and a float).
// gfx950's "bf8" converters read the OCP E5M2 format (checked on hardware
// against the format definition for all 256 codes).
__device__ __forceinline__ void bf8x4_to_f32(uint32_t w, float* out) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_bf8(w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_bf8(w, true);
  out[0] = lo[0]; out[1] = lo[1]; out[2] = hi[0]; out[3] = hi[1];
}

__device__ __forceinline__ void bf8x4_to_bf16(uint32_t w, bf16x2& lo, bf16x2& hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, true);
}

// Round a float to an E5M2 code: nearest, ties to even, magnitudes that
// round above 57344 (the largest finite value) saturate to it, NaN stays
// NaN.  The spacing is 2^-16 below 2^-14 (subnormals) and 2^(e-2) in
// binade 2^e.
__device__ __forceinline__ uint32_t f32_to_e5m2_sat(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = __uint_as_float(u & 0x7fffffffu);
  if (!(a == a)) return sign | 0x7fu;
  if (a >= 57344.0f) return sign | 0x7bu;
  if (a < 6.103515625e-05f) {  // below 2^-14: multiples of 2^-16; rint(4) = 4 is code 0x04
    return sign | (uint32_t)__builtin_rintf(a * 65536.0f);
  }
  int e = (int)((u >> 23) & 0xffu) - 127;                 // binade of a, -14..15
  float q = __builtin_rintf(__builtin_ldexpf(a, 2 - e));  // 4..8
  uint32_t code = (uint32_t)(((e + 15) << 2) + (int)q - 4);  // q == 8 carries into e
  return sign | (code > 0x7bu ? 0x7bu : code);             // the carry above 57344 saturates
}

// Round a float to an E4M3FN code: nearest, ties to even, magnitudes at or
// above 448 saturate to 448, NaN stays NaN.  Written from the format: the
// spacing is 2^-9 below 2^-6 (subnormals) and 2^(e-3) in binade 2^e.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = __uint_as_float(u & 0x7fffffffu);
  if (!(a == a)) return sign | 0x7fu;
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9; rint(8) = 8 is code 0x08
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  int e = (int)((u >> 23) & 0xffu) - 127;  // binade of a, -6..8
  float q = __builtin_rintf(__builtin_ldexpf(a, 3 - e));  // 8..16
  return sign | (uint32_t)(((e + 7) << 3) + (int)q - 8);  // q == 16 carries into e
}

// ---------------------------------------------------------------------------
// INT4 codes
// ---------------------------------------------------------------------------

// Bias of the widened INT4 operands: a code c becomes the bf16 136 + c.
constexpr float kI4Bias = 136.0f;

// One octet word of INT4 codes (byte i: element i in the low nibble,
// element i + 4 in the high nibble, two's complement) -> eight bf16 holding
// 136 + code, in element order.  XOR with 8 turns each nibble into c + 8
// (0..15); a bf16 with high byte 0x43 and low byte u is exactly 128 + u for
// u < 128, so one byte permute per pair builds the bit patterns.  Exact; the
// consumer subtracts the bias in float32.
__device__ __forceinline__ u32x4 i4x8_biased_words(uint32_t w) {
  // offset codes (code + 8 = code ^ 8), one per byte; each line is one
  // three-input bitwise instruction after the shift
  const uint32_t lo = (w & 0x0F0F0F0Fu) ^ 0x08080808u;         // elements 0..3
  const uint32_t hi = ((w >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;  // elements 4..7
  constexpr uint32_t k43 = 0x43434343u;
  // v_perm_b32: selector byte 0..3 picks a byte of the second operand, 4..7
  // of the first; {b0, 0x43, b1, 0x43} and {b2, 0x43, b3, 0x43}
  return u32x4{__builtin_amdgcn_perm(k43, lo, 0x04010400u), __builtin_amdgcn_perm(k43, lo, 0x04030402u),
               __builtin_amdgcn_perm(k43, hi, 0x04010400u), __builtin_amdgcn_perm(k43, hi, 0x04030402u)};
}

// INT4 code of x under scale s (s > 0): x / s rounded once in binary32,
// then to the nearest integer, ties to even, kept within -7..7.
__device__ __forceinline__ int i4_code(float x, float s) {
  const float q = __builtin_rintf(__fdiv_rn(x, s));
  return (int)fminf(fmaxf(q, -7.0f), 7.0f);
}

// ---------------------------------------------------------------------------
// cross-lane combine.  DPP row controls (within 16-lane rows):
//   0xB1 quad_perm[1,0,3,2]  (partner = lane ^ 1)
//   0x4E quad_perm[2,3,0,1]  (partner = lane ^ 2)
//   0x141 row_half_mirror    (lane i <-> 7 - i inside each 8)
//   0x140 row_mirror         (lane i <-> 15 - i inside each 16)
// After combining over partners 1 and 2 every quad holds one value, so the
// mirrors pair whole quads / half-rows; that is all an all-reduce needs.
// Across rows the gfx950 permlane swaps exchange lane l with l ^ 16 and
// l ^ 32 in one VALU instruction.
// ---------------------------------------------------------------------------

struct OpSum { __device__ static float f(float a, float b) { return a + b; } };
struct OpMax { __device__ static float f(float a, float b) { return fmaxf(a, b); } };
// NaN-propagating maximum (v_maximum3_f32): unlike fmaxf it needs no
// quieting of its inputs, so a tree of them is one instruction per level.
// For softmax scores, which hold no NaN unless the inputs did.
struct OpMaxP {
  __device__ static float f(float a, float b) { return __builtin_elementwise_maximum(a, b); }
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// {x, x of lane ^ 16} (in lane-dependent order): permlane16_swap of x with
// itself leaves one copy of x and brings in the partner's.
template <class Op>
__device__ __forceinline__ float combine16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return Op::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <class Op>
__device__ __forceinline__ float combine32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return Op::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}


// Combine x over lane partners at distances LO, 2*LO, ..., HI (powers of two,
// LO <= HI <= 32).  Exact all-reduce over groups of 2*HI lanes when the
// values are already uniform within groups of LO lanes.
template <class Op, int LO, int HI>
__device__ __forceinline__ float xlane(float x) {
  if constexpr (LO <= 1 && HI >= 1) x = Op::f(x, dpp<0xB1>(x));
  if constexpr (LO <= 2 && HI >= 2) x = Op::f(x, dpp<0x4E>(x));
  if constexpr (LO <= 4 && HI >= 4) x = Op::f(x, dpp<0x141>(x));
  if constexpr (LO <= 8 && HI >= 8) x = Op::f(x, dpp<0x140>(x));
  if constexpr (LO <= 16 && HI >= 16) x = combine16<Op>(x);
  if constexpr (LO <= 32 && HI >= 32) x = combine32<Op>(x);
  return x;
}

__device__ __forceinline__ int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// KV tiles are read once per decode: stream them with non-temporal loads,
// which keep them from displacing reusable lines in the caches (measured on
// MI355X: random 4 KiB tiles read at ~6.9 TB/s this way, ~6.1 TB/s with
// ordinary loads).
template <typename T>
__device__ __forceinline__ T stream_load(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}

// Wave-uniform "any lane true".
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

}  // namespace pa
