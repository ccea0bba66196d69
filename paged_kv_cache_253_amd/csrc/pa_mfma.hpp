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
//
// The k-slots of QK chunk c map to head dimensions per cache kind (q_dim):
// any map works as long as q and K use the same one, so each kind takes the
// one its K loads deliver.
//
// INT4 caches: K and V codes widen to bf16 136 + code (exact; see
// i4x8_biased_words) and the bias is removed in float32: a score is
// s_k(t) * (S - 136 * sum_d q_d) with S the MFMA result, and the PV
// operand carries p(t) * s_v(t), whose own sum (one extra MFMA against a
// row of ones) gives the 136 * sum_t p(t) s_v(t) to subtract from the
// output.  Every token's two scales sit at the end of its tile.
#pragma once

#include <cfloat>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace mfma {

constexpr int kStep = 32;  // tokens per step

// Cache element kinds of the matrix-core kernels.  The two FP8 kinds share
// the 1-byte layout and differ only in how a code widens to bf16.
constexpr int kBF16 = 0, kE4M3 = 1, kE5M2 = 2, kI4 = 3;
template <int CK>
constexpr bool one_byte() { return CK == kE4M3 || CK == kE5M2; }

template <int CK, int D, int BS>
struct Cfg {
  static constexpr bool FP8 = one_byte<CK>();
  static constexpr bool I4 = CK == kI4;
  static constexpr int kElt = FP8 ? 1 : 2;          // bytes per element (bf16 / FP8)
  static constexpr int kChunks = D / 32;            // QK MFMAs per token group
  static constexpr int kDTiles = D / 16;            // PV MFMAs per step
  // K loads per token group and lane: 16 bytes each (INT4: D/8 bytes, one load)
  static constexpr int kKLoads = I4 ? 1 : (FP8 ? D / 64 : D / 32);
  static constexpr int kChunkRow = BS * 16;         // bytes of one K chunk row (16 B per token)
  static constexpr int kRowV = I4 ? BS / 2 : BS * kElt;  // bytes of one V row (dimension)
  static constexpr int kCodeBytes = I4 ? BS * D / 2 : BS * D * kElt;
  static constexpr int kTile = I4 ? BS * (D / 2 + 4) : kCodeBytes;  // one (block, head) tile
  static constexpr int kBlocksPerStep = kStep / BS;
};

// Raw K words of one token group (per lane).
template <int CK, int D>
struct KWord { using T = u32x4; };
template <>
struct KWord<kI4, 64> { using T = u32x2; };

// Raw V words of one PV tile (per lane: 8 tokens of one dimension).
template <int CK>
struct VRaw { u32x4 w; };     // 8 bf16
template <>
struct VRaw<kE4M3> { u32x2 w; };
template <>
struct VRaw<kE5M2> { u32x2 w; };
template <>
struct VRaw<kI4> { uint32_t w; };

// Per-token scales of an INT4 step, in QK register order: k[0] / v[0] for
// tokens 4*grp + r, k[1] / v[1] for tokens 16 + 4*grp + r.
template <int CK>
struct TokScales {};
template <>
struct TokScales<kI4> { f32x4 k[2], v[2]; };

template <int CK, int D, int BS>
struct StepBuf {
  using C = Cfg<CK, D, BS>;
  typename KWord<CK, D>::T k[2][C::kKLoads];
  VRaw<CK> v[C::kDTiles];
  TokScales<CK> ts;
};

// Head dimension of k-slot 0 of QK chunk c for lane group grp (8 contiguous
// dimensions follow it).
template <int CK, int D>
__device__ __forceinline__ int q_dim(int grp, int c) {
  if constexpr (CK == kI4) return (D / 4) * grp + 8 * c;                  // one D/8-byte load
  else if constexpr (one_byte<CK>()) return (c >> 1) * 64 + grp * 16 + (c & 1) * 8;
  else return c * 32 + grp * 8;
}

// Byte offsets of a lane's data inside the step's tiles: K (token col of
// group 0, its k-slot dimensions) and V (dimension col of PV tile 0, tokens
// 8*grp .. +7 of the step, in tile vblk of the step).
template <int CK, int D, int BS>
struct LaneOffsets {
  uint32_t koff, voff;
  int vblk;
  __device__ __forceinline__ LaneOffsets(int grp, int col) {
    using C = Cfg<CK, D, BS>;
    if constexpr (CK == kI4) {
      const int dim0 = (D / 4) * grp;
      koff = (uint32_t)(((dim0 / 32) * BS + col) * 16 + (dim0 % 32) / 2);
    } else {
      koff = (uint32_t)((grp * BS + col) * 16);
    }
    vblk = (BS == 16) ? (grp >> 1) : 0;
    const int vtok = (BS == 16) ? 8 * (grp & 1) : 8 * grp;
    voff = (uint32_t)(col * C::kRowV) + (CK == kI4 ? (uint32_t)(vtok / 2) : (uint32_t)(vtok * C::kElt));
  }
};

// Issue one step's tile loads.  tile0 / tile1: byte offsets of the (block,
// head) tiles of the step's first and second 16 tokens (equal at block size
// 32).  Every call issues the same number of loads.
template <int CK, int D, int BS>
__device__ __forceinline__ void load_step(StepBuf<CK, D, BS>& sb, const char* kc, const char* vc,
                                          int64_t tile0, int64_t tile1, const LaneOffsets<CK, D, BS>& lo,
                                          int grp) {
  using C = Cfg<CK, D, BS>;
  using KW = typename KWord<CK, D>::T;
  const char* kp0 = kc + tile0 + lo.koff;
  const char* kp1 = (BS == 16) ? kc + tile1 + lo.koff : kp0 + 16 * 16;
  const char* vp = vc + (lo.vblk ? tile1 : tile0) + lo.voff;
#pragma unroll
  for (int j = 0; j < C::kKLoads; ++j) {
    sb.k[0][j] = stream_load<KW>(kp0 + j * 4 * C::kChunkRow);
    sb.k[1][j] = stream_load<KW>(kp1 + j * 4 * C::kChunkRow);
  }
#pragma unroll
  for (int dt = 0; dt < C::kDTiles; ++dt) {
    if constexpr (CK == kI4) sb.v[dt].w = stream_load<uint32_t>(vp + dt * 16 * C::kRowV);
    else if constexpr (C::FP8) sb.v[dt].w = stream_load<u32x2>(vp + dt * 16 * C::kRowV);
    else sb.v[dt].w = stream_load<u32x4>(vp + dt * 16 * C::kRowV);
  }
  if constexpr (CK == kI4) {
    const int64_t s0 = tile0 + C::kCodeBytes + 16 * grp;
    const int64_t s1 = (BS == 16) ? tile1 + C::kCodeBytes + 16 * grp : s0 + 64;
    sb.ts.k[0] = stream_load<f32x4>(kc + s0);
    sb.ts.k[1] = stream_load<f32x4>(kc + s1);
    sb.ts.v[0] = stream_load<f32x4>(vc + s0);
    sb.ts.v[1] = stream_load<f32x4>(vc + s1);
  }
}

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
  if constexpr (CK == kI4) {
    return as_bf16x8(i4x8_biased_words(sb.k[m][0][c]));
  } else if constexpr (one_byte<CK>()) {
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

// QK result register i (0..7) of lane row grp holds token 4 * grp +
// qk_token_off(i) of the step.
__device__ __forceinline__ constexpr int qk_token_off(int i) { return (i & 3) + 16 * (i >> 2); }

template <int CK>
__device__ __forceinline__ bf16x8 v_operand(const VRaw<CK>& r) {
  if constexpr (CK == kI4) return as_bf16x8(i4x8_biased_words(r.w));
  else if constexpr (one_byte<CK>()) return fp8x8_to_bf16x8<CK>(r.w[0], r.w[1]);
  else return as_bf16x8(r.w);
}

// Zero the V elements of k-slots whose token is past the range end.  INT4
// needs none: its codes are finite and those tokens' weights are zero.
template <int CK>
__device__ __forceinline__ void mask_v(VRaw<CK>& r, int valid) {  // valid = tokens kept, 0..8
  if constexpr (one_byte<CK>()) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      int n = valid - 4 * w;
      uint32_t keep = n >= 4 ? 0xffffffffu : (n <= 0 ? 0u : (0xffffffffu >> (32 - 8 * n)));
      r.w[w] &= keep;
    }
  } else if constexpr (CK == kBF16) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      int n = valid - 2 * w;
      uint32_t keep = n >= 2 ? 0xffffffffu : (n == 1 ? 0x0000ffffu : 0u);
      r.w[w] &= keep;
    }
  }
}

// 2^x on the transcendental unit (v_exp_f32) without the library's range
// reduction: results below 2^-126 may flush to zero, far below what any
// softmax weight here can contribute (the largest weight of a row is 1).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Lazy rescaling: the reference maximum m_run (and with it the
// accumulators) moves only when a score exceeds it by more than kLazyLog2
// in log2 units, so a weight can reach 2^kLazyLog2 = 256 instead of 1 (a
// bf16 weight keeps its relative precision at any magnitude).  Each lane
// keeps the running maximum of its own scores (m_lane) and compares it with
// the column's threshold thr = m_run + kLazyLog2 / c2, so the cross-lane
// maximum is taken only when some column moves, and once at the end of a
// range (settle), which leaves the range's state (maximum, sum, output) the
// plain one.  The weights' offset mc = m_run * c2 and thr change only when
// m_run does.
constexpr float kLazyLog2 = 8.0f;

// The softmax's log2 factor c2 = scale * log2(e) (times an FP8 K scale), so
// that a weight is 2^((z - m) * c2) for a score z in q.k units.  A K scale
// of 0 (a head whose keys were all zero) would make c2 0 and a masked score
// -inf * 0 = NaN; the smallest normal float instead leaves every finite
// weight exactly 1, as c2 = 0 would, and every masked one 0.
__device__ __forceinline__ float log2_factor(float scale, float kscale) {
  return fmaxf(scale * kscale * kLog2e, FLT_MIN);
}

struct LaneSoftmax {
  float m_run;   // reference maximum of the column's scores (q.k units)
  float m_lane;  // the largest score this lane has seen
  float thr;     // m_run + span: a score above it would weigh more than 2^kLazyLog2
  float mc;      // m_run * c2 (0 while m_run is -inf: every weight is then 0)
  float span;    // kLazyLog2 / c2
  float l_run;   // this lane's share of sum 2^((z - m_run) * c2)

  __device__ __forceinline__ void reset(float c2) {
    m_run = m_lane = thr = -INFINITY;
    mc = 0.f;
    l_run = 0.f;
    span = kLazyLog2 * __builtin_amdgcn_rcpf(c2);
  }

  // Move m_run to the column maximum m_col (this lane's column; all lanes
  // call), rescaling what has been accumulated.
  template <int NDT, bool SUMS>
  __device__ __forceinline__ void move_to(float m_col, float c2, f32x4* acc, f32x4& accb) {
    if (m_col > m_run) {
      // with m_run -inf nothing has been accumulated (every weight so far
      // was 0), and (m_run - m_col) * c2 would be NaN at c2 = 0
      if (m_run != -INFINITY) {
        const float alpha = exp2_fast((m_run - m_col) * c2);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
        if constexpr (SUMS) accb *= alpha;
      }
      m_run = m_col;
      mc = m_col * c2;
      thr = m_col + span;
    }
  }
};

// The column maximum of m_lane: over the lane groups holding one column
// (and, packed, over the two column halves of a head).
template <bool PK>
__device__ __forceinline__ float column_max(float m_lane) {
  if constexpr (PK) m_lane = OpMaxP::f(m_lane, dpp<0x128>(m_lane));  // row_ror:8 -> column c ^ 8
  return xlane<OpMaxP, 16, 32>(m_lane);
}

// End of a range: the state at its true maximum.
template <int NDT, bool PK>
__device__ __forceinline__ void lazy_settle(LaneSoftmax& st, float c2, f32x4* acc, f32x4& accb) {
  const float m_col = column_max<PK>(st.m_lane);
  if (wave_any(m_col > st.m_run)) st.move_to<NDT, true>(m_col, c2, acc, accb);
}

// Initial QK accumulator: zero, or for INT4 minus the operand bias (136 *
// the sum of the lane column's q, see q_bias), so that the MFMA result is
// already sum_d q_d code_d.
template <int CK>
__device__ __forceinline__ f32x4 qk_init(float qbias) {
  if constexpr (CK == kI4) return f32x4{-qbias, -qbias, -qbias, -qbias};
  else return f32x4{0.f, 0.f, 0.f, 0.f};
}

// QK results (QK register order, accumulated from qk_init) -> scores in q.k
// units.  INT4: apply each token's own K scale.  Other kinds: unchanged (an
// FP8 K scale is folded into the log2 factor).
template <int CK, class Buf>
__device__ __forceinline__ void qk_scores(float* z, const Buf& sb) {
  if constexpr (CK == kI4) {
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] *= sb.ts.k[i >> 2][i & 3];
  }
}

// One online-softmax step over the 8 scores a lane holds (QK register
// order, q.k units): update the lane's running maximum and sum, rescale the
// accumulators when a column's reference maximum moves (LaneSoftmax), and
// return the PV weights operand.  c2 = softmax scale * log2(e) (times an FP8 K scale), so
// a weight is 2^(z*c2 - m*c2).  Only a partial step (one holding tokens
// outside the range) reads lim: score register i is kept iff its token's
// offset from the lane's first token, qk_token_off(i), is at most lim (a
// lane that keeps nothing passes -1).  The comparisons are made where they
// are used, so a full step carries no mask.  INT4: the weights carry each
// token's V scale, and accb their column sums.
template <int CK, int NDT, class Buf>
__device__ __forceinline__ bf16x8 softmax_step(float* z, bool partial, int lim, const Buf& sb,
                                               float c2, LaneSoftmax& st, f32x4* acc, f32x4& accb) {
  if (partial) {
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = qk_token_off(i) <= lim ? z[i] : -INFINITY;
  }
  using M = OpMaxP;
  st.m_lane = M::f(M::f(M::f(z[0], z[1]), M::f(z[2], z[3])),
                   M::f(M::f(z[4], z[5]), M::f(M::f(z[6], z[7]), st.m_lane)));
  if (wave_any(st.m_lane > st.thr)) st.move_to<NDT, CK == kI4>(column_max<false>(st.m_lane), c2, acc, accb);
  // a masked score is -inf, so its weight is exp2(-inf) = 0 -- also in a
  // column that has seen only masked scores (mc 0 there, not -inf * c2)
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = exp2_fast(fmaf(z[i], c2, -st.mc));
#pragma unroll
  for (int i = 0; i < 8; ++i) st.l_run += p[i];
  if constexpr (CK == kI4) {
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pv[i] = p[i] * sb.ts.v[i >> 2][i & 3];
    if (partial) {  // a scale outside the range may be anything, NaN included
#pragma unroll
      for (int i = 0; i < 8; ++i) pv[i] = qk_token_off(i) <= lim ? pv[i] : 0.f;
    }
    return p_operand(pv);
  } else {
    return p_operand(p);
  }
}

// bf16 1.0 in every k-slot: the A operand whose product with the PV weights
// is their column sums.
__device__ __forceinline__ bf16x8 ones_operand() {
  const u32x4 w = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  return as_bf16x8(w);
}

// 136 * sum of this lane column's q over all head dimensions (the lanes of
// one column hold disjoint dimension sets; all lanes must call).
template <int NC>
__device__ __forceinline__ float q_bias(const bf16x8* q) {
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) s += (float)q[c][e];
  return kI4Bias * xlane<OpSum, 16, 32>(s);
}

// ---------------------------------------------------------------------------
// Column-packed INT4 steps (G <= 8 query heads per KV head).  Unpacked, a
// step's QK fills G of the 16 MFMA columns and every lane runs the softmax
// on 8 scores of which 16 - G columns are padding.  Packed, columns 0..7
// carry the G heads for the step's first 16 tokens and columns 8..15 the
// same heads for its last 16: each lane holds 4 scores, and the per-token
// work (scales, exponentials, sums) halves at the same MFMA count.
//
// QK (K rows as the A operand): the 32 k-slots split into two segments of
// 16 (lane groups 0,1 and 2,3); A row r of segment s is token 16 s + pi(r),
// and the q operand of column c is zero outside segment c / 8, so column c
// only sees tokens 16 (c / 8) + pi(r).  Lane group bit grp & 1 selects the
// head-dimension half a lane supplies: MFMA i takes dimensions
// (D/2) (grp & 1) + 8 i .. + 7, i.e. word i of the lane's K row.  With
// pi(4g + j) = 8 (g & 1) + 4 (g >> 1) + j, lane (g, c) ends with the
// scores of tokens 16 (c / 8) + 8 (g & 1) + 4 (g >> 1) + j (j = 0..3), and
// the PV weights operand needs one permlane32 swap per register pair.
//
// PV (V rows as the A operand, as unpacked): the weights operand of column
// c is zero outside the k-slots of its token half, so columns c and c + 8
// accumulate the two halves of every step; pk_fold sums them at the end.
// ---------------------------------------------------------------------------

template <int D, int BS>
struct PkBuf {
  u32x4 k[D / 64];       // the lane's K row: D/2 head dimensions, D/16 octet words
  VRaw<kI4> v[D / 16];   // as unpacked
  f32x4 sk, sv;          // K and V scales of the lane's 4 score tokens
};

// A row r of a segment -> its token within the 16-token half.
__device__ __forceinline__ int pk_row_token(int r) { return 8 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

// First token (within the step) of the 4 scores lane (grp, col) holds.
__device__ __forceinline__ int pk_score_token(int grp, int col) {
  return 16 * (col >> 3) + 8 * (grp & 1) + 4 * (grp >> 1);
}

// Head dimension of k-slot 0 of QK MFMA i for lane group grp.
template <int D>
__device__ __forceinline__ int pk_q_dim(int grp, int i) { return (D / 2) * (grp & 1) + 8 * i; }

// The lane supplies the q operand of its column (else zeros).
__device__ __forceinline__ bool pk_active(int grp, int col) { return (grp >> 1) == (col >> 3); }

template <int D, int BS>
struct PkOffsets {
  uint32_t koff, soff;
  bool kblk, sblk;  // second tile of the step (block size 16)
  LaneOffsets<kI4, D, BS> v;
  __device__ __forceinline__ PkOffsets(int grp, int col) : v(grp, col) {
    const int ktok = 16 * (grp >> 1) + pk_row_token(col);  // the lane's K row token
    const int chunk = (D / 64) * (grp & 1);                // first 32-dimension chunk
    const int t0 = pk_score_token(grp, col);
    if constexpr (BS == 16) {
      koff = (uint32_t)((chunk * BS + (ktok & 15)) * 16);
      kblk = ktok >= 16;
      soff = (uint32_t)(Cfg<kI4, D, BS>::kCodeBytes + 4 * (t0 & 15));
      sblk = t0 >= 16;
    } else {
      koff = (uint32_t)((chunk * BS + ktok) * 16);
      kblk = false;
      soff = (uint32_t)(Cfg<kI4, D, BS>::kCodeBytes + 4 * t0);
      sblk = false;
    }
  }
};

template <int D, int BS>
__device__ __forceinline__ void load_step_pk(PkBuf<D, BS>& sb, const char* kc, const char* vc, int64_t tile0,
                                             int64_t tile1, const PkOffsets<D, BS>& lo) {
  using C = Cfg<kI4, D, BS>;
  const char* kp = kc + (lo.kblk ? tile1 : tile0) + lo.koff;
#pragma unroll
  for (int j = 0; j < D / 64; ++j) sb.k[j] = stream_load<u32x4>(kp + j * BS * 16);
  const char* vp = vc + (lo.v.vblk ? tile1 : tile0) + lo.v.voff;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) sb.v[dt].w = stream_load<uint32_t>(vp + dt * 16 * C::kRowV);
  const int64_t st = (lo.sblk ? tile1 : tile0) + lo.soff;
  sb.sk = stream_load<f32x4>(kc + st);
  sb.sv = stream_load<f32x4>(vc + st);
}

template <class Buf>
__device__ __forceinline__ bf16x8 k_operand_pk(const Buf& sb, int i) {
  return as_bf16x8(i4x8_biased_words(sb.k[i >> 2][i & 3]));
}

// One online-softmax step over the lane's 4 scores (q.k units, bias
// removed, K scales not yet applied): as softmax_step, with the column
// maximum taken over both column halves of a head, and the PV weights
// operand zero outside the lane's token half.  Partial step: score j is
// kept iff j <= lim.
template <int NDT, class Buf>
__device__ __forceinline__ bf16x8 softmax_step_pk(float* z, bool partial, int lim, const Buf& sb,
                                                  float c2, LaneSoftmax& st, f32x4* acc, f32x4& accb,
                                                  bool active) {
  using M = OpMaxP;
#pragma unroll
  for (int j = 0; j < 4; ++j) z[j] *= sb.sk[j];
  if (partial) {
#pragma unroll
    for (int j = 0; j < 4; ++j) z[j] = j <= lim ? z[j] : -INFINITY;
  }
  st.m_lane = M::f(M::f(z[0], z[1]), M::f(M::f(z[2], z[3]), st.m_lane));
  if (wave_any(st.m_lane > st.thr)) st.move_to<NDT, true>(column_max<true>(st.m_lane), c2, acc, accb);
  float p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) p[j] = exp2_fast(fmaf(z[j], c2, -st.mc));
#pragma unroll
  for (int j = 0; j < 4; ++j) st.l_run += p[j];
  float pv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pv[j] = p[j] * sb.sv[j];
  if (partial) {  // a scale outside the range may be anything, NaN included
#pragma unroll
    for (int j = 0; j < 4; ++j) pv[j] = j <= lim ? pv[j] : 0.f;
  }
  uint32_t w[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    bf16x2 t;
    t[0] = (__bf16)pv[2 * i];
    t[1] = (__bf16)pv[2 * i + 1];
    w[i] = __builtin_bit_cast(uint32_t, t);
  }
  // lanes 0..31 keep their own pair and take that of lane + 32 (tokens + 4);
  // lanes 32..63 take that of lane - 32 (tokens - 4) and keep their own
  const auto x0 = __builtin_amdgcn_permlane32_swap(w[0], w[0], false, false);
  const auto x1 = __builtin_amdgcn_permlane32_swap(w[1], w[1], false, false);
  const u32x4 r = active ? u32x4{x0[0], x1[0], x0[1], x1[1]} : u32x4{0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, r);
}

// Sum the two column halves of a head (columns c and c ^ 8).
__device__ __forceinline__ float pk_fold(float x) { return x + dpp<0x128>(x); }

}  // namespace mfma
}  // namespace pa
