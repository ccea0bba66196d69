// Shared pieces of the multi-query (chunked prefill / speculative verify)
// kernels: the work-item map, the per-wavefront column tiles with their
// QK / causal-mask / online-softmax / PV step, and a query tile's context
// range.  The kernels themselves: prefill_mfma.hip (one wavefront per query
// tile) and prefill_lds.hip (wavefronts of a workgroup sharing each step's
// tiles through LDS).
#pragma once

#include "pa_device.hpp"
#include "pa_internal.hpp"
#include "pa_mfma.hpp"
#include "pa_split.hpp"

namespace pa {
namespace prefill {

using namespace mfma;

// Work item -> (pair = b * Hkv + h, partition, tile-or-group): pair p runs
// on XCD p % kXcds; its items (partition-major) take consecutive slots.
struct Item {
  int b, h, part, sub;
  bool ok;
};
__device__ __forceinline__ Item locate_item(const DecodeArgs& a, int per_part) {
  const int parts = a.partition ? a.max_parts : 1;
  const int items = parts * per_part;
  const int xcd = (int)(blockIdx.x % kXcds);
  const int slot = (int)(blockIdx.x / kXcds);
  const int pair = (slot / items) * kXcds + xcd;
  Item it;
  it.ok = pair < a.num_seqs * a.num_kv_heads;
  const int inner = slot % items;
  it.part = inner / per_part;
  it.sub = inner % per_part;
  it.h = pair % a.num_kv_heads;
  it.b = pair / a.num_kv_heads;
  return it;
}

// The NT column tiles of one wavefront: query rows i0 .. i1-1 of sequence b
// (positions first_pos + i), KV head h; their q operands, running softmax
// states and output accumulators.
//
// The online softmax is the decode's (LaneSoftmax: lazy rescaling checked
// per lane, masks from a per-lane token limit), with less work per step, as
// these kernels issue many steps per byte read:
// * bf16 and FP8: the exp-sum of a column comes from the matrix cores, as
//   the product of a ones operand with the step's weights operand (so it
//   sums the same bf16 weights the PV product does); INT4, whose weights
//   operand carries the V scales, sums its weights on the vector unit.
// * Whether a step needs masks is decided per column tile from scalars: the
//   smallest position of its valid rows against the step's last token.
template <int CK, int D, int BS, int NT>
struct Columns {
  using C = Cfg<CK, D, BS>;
  int pos[NT];
  int pos_min[NT];                    // wave-uniform: smallest valid position (INT_MAX: no valid row)
  bool cvalid[NT];
  size_t qrow[NT];                    // row of q / out (query token * Hq + query head)
  bf16x8 qop[NT][C::kChunks];
  f32x4 acc[NT][C::kDTiles];
  // bf16 / FP8: exp-sums of the columns (every register); INT4: column sums
  // of the PV weights (the exp-sums are st.l_run)
  f32x4 sums[NT];
  LaneSoftmax st[NT];
  float qbias[NT];

  // columns: query token qi = i0 + c / G, head g = c % G
  __device__ __forceinline__ void init(const DecodeArgs& a, int r0, int i0, int i1, int first_pos,
                                       int h, int col, int grp, float c2) {
    const int G = a.group;
    const __bf16* qbase = reinterpret_cast<const __bf16*>(a.q);
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      const int c = ct * 16 + col;
      const int qi = i0 + c / G;
      cvalid[ct] = qi < i1;
      pos[ct] = first_pos + qi;
      // the tile's first column holds its smallest position
      const int qi0 = __builtin_amdgcn_readfirstlane(i0 + (ct * 16) / G);
      pos_min[ct] = qi0 < __builtin_amdgcn_readfirstlane(i1)
                        ? __builtin_amdgcn_readfirstlane(first_pos) + qi0 : INT_MAX;
      qrow[ct] = (size_t)(r0 + (cvalid[ct] ? qi : i0)) * a.num_q_heads + (size_t)h * G + (c % G);
#pragma unroll
      for (int cc = 0; cc < C::kChunks; ++cc) {
        if (cvalid[ct]) {
          qop[ct][cc] = *reinterpret_cast<const bf16x8*>(qbase + qrow[ct] * D + q_dim<CK, D>(grp, cc));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) qop[ct][cc][e] = (__bf16)0.0f;
        }
      }
      // the query operands land here: otherwise the compiler, seeing loads
      // into them before the step loop, waits at their first use in every
      // step for all loads in flight, the ones issued ahead for later steps
      // included (an empty asm statement that reads them, no memory clobber)
#pragma unroll
      for (int cc = 0; cc < C::kChunks; ++cc) asm volatile("" : : "v"(qop[ct][cc]));
      st[ct].reset(c2);
      sums[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      qbias[ct] = 0.f;
      if constexpr (C::I4) qbias[ct] = q_bias<C::kChunks>(qop[ct]);
#pragma unroll
      for (int dt = 0; dt < C::kDTiles; ++dt) acc[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // One 32-token step starting at token `base`; tokens at or past t1 are
  // outside this wavefront's range.  kPermRows: the QK A operand's rows
  // come permuted (row r of sb.k[0] is token 8 (r / 4) + r % 4, of sb.k[1]
  // that + 4), so score register i of lane row grp is token 8 grp + i: the
  // scores then sit in the PV weights operand's k-slot order and need no
  // exchange between lanes.
  template <bool kPermRows = false>
  __device__ __forceinline__ void step(StepBuf<CK, D, BS>& sb, int base, int t1, int grp, float c2) {
    static_assert(!(kPermRows && C::I4), "INT4 weights carry token scales in QK register order");
    f32x4 s0[NT], s1[NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) { s0[ct] = qk_init<CK>(qbias[ct]); s1[ct] = s0[ct]; }
#pragma unroll
    for (int c = 0; c < C::kChunks; ++c) {
      const bf16x8 ka = k_operand<CK>(sb, 0, c);
      const bf16x8 kb = k_operand<CK>(sb, 1, c);
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        s0[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qop[ct][c], s0[ct], 0, 0, 0);
        s1[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qop[ct][c], s1[ct], 0, 0, 0);
      }
    }
    if (base + kStep > t1) {  // PV k-slots of this lane: tokens 8*grp .. +7
      const int vvalid = min(max(t1 - (base + 8 * grp), 0), 8);
#pragma unroll
      for (int dt = 0; dt < C::kDTiles; ++dt) mask_v<CK>(sb.v[dt], vvalid);
    }
    bf16x8 pop[NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      float z[8] = {s0[ct][0], s0[ct][1], s0[ct][2], s0[ct][3],
                    s1[ct][0], s1[ct][1], s1[ct][2], s1[ct][3]};
      qk_scores<CK>(z, sb);
      // a valid row stops inside the step (its position, or the range end)
      const bool partial = min(t1 - 1, pos_min[ct]) < base + kStep - 1;
      // kept: offsets from the lane's first token up to the last token this
      // column may see (none for a padding column)
      const int zlim = cvalid[ct] ? min(t1 - 1, pos[ct]) - base - (kPermRows ? 8 : 4) * grp : -1;
      if (partial) {
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = (kPermRows ? i : qk_token_off(i)) <= zlim ? z[i] : -INFINITY;
      }
      using M = OpMaxP;
      LaneSoftmax& s = st[ct];
      s.m_lane = M::f(M::f(M::f(z[0], z[1]), M::f(z[2], z[3])),
                      M::f(M::f(z[4], z[5]), M::f(M::f(z[6], z[7]), s.m_lane)));
      if (wave_any(s.m_lane > s.thr))
        s.move_to<C::kDTiles, true>(column_max<false>(s.m_lane), c2, acc[ct], sums[ct]);
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = exp2_fast(fmaf(z[i], c2, -s.mc));
      if constexpr (C::I4) {
#pragma unroll
        for (int i = 0; i < 8; ++i) s.l_run += p[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] *= sb.ts.v[i >> 2][i & 3];
        if (partial) {  // a scale outside the range may be anything, NaN included
#pragma unroll
          for (int i = 0; i < 8; ++i) p[i] = qk_token_off(i) <= zlim ? p[i] : 0.f;
        }
      }
      if constexpr (kPermRows) {
#pragma unroll
        for (int i = 0; i < 8; ++i) pop[ct][i] = (__bf16)p[i];
      } else {
        pop[ct] = p_operand(p);
      }
    }
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt) {
      const bf16x8 vop = v_operand<CK>(sb.v[dt]);
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
        acc[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[ct], acc[ct][dt], 0, 0, 0);
    }
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
      sums[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_operand(), pop[ct], sums[ct], 0, 0, 0);
  }

  // One row per valid column: the output, or the partition's softmax state.
  __device__ __forceinline__ void finish(const DecodeArgs& a, int part, int grp, float c2,
                                         float vscale) {
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      lazy_settle<C::kDTiles, false>(st[ct], c2, acc[ct], sums[ct]);
      const float l_tot = C::I4 ? xlane<OpSum, 16, 32>(st[ct].l_run) : sums[ct][0];
      if (!cvalid[ct]) continue;
      const float inv = l_tot > 0.f ? vscale / l_tot : 0.f;  // a row with no token writes zeros
      if constexpr (C::I4) {  // remove the operand bias: 136 * sum_t p(t) s_v(t)
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[ct][dt][r] = fmaf(-kI4Bias, sums[ct][0], acc[ct][dt][r]);
      }
      if (a.partition == 0) {
        __bf16* o = reinterpret_cast<__bf16*>(a.out) + qrow[ct] * D;
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt) {
          bf16x2 lo, hi;
          lo[0] = (__bf16)(acc[ct][dt][0] * inv); lo[1] = (__bf16)(acc[ct][dt][1] * inv);
          hi[0] = (__bf16)(acc[ct][dt][2] * inv); hi[1] = (__bf16)(acc[ct][dt][3] * inv);
          u32x2 w = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
          *reinterpret_cast<u32x2*>(o + dt * 16 + grp * 4) = w;
        }
      } else {
        const size_t row = qrow[ct] * a.max_parts + part;
        float* o = a.part_out + row * D;
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt)
          *reinterpret_cast<f32x4*>(o + dt * 16 + grp * 4) = acc[ct][dt] * inv;
        if (grp == 0) {
          a.part_max[row] = st[ct].m_run * (c2 * kLn2);  // natural units: scale * q.k
          a.part_sum[row] = l_tot;
        }
      }
    }
  }
};

// Query rows and context range of query tile `tile` of sequence b: rows
// i0 .. i1-1 (empty if i0 >= nq), tokens [t0, t1) of partition `part`.
struct TileRange {
  int r0, nq, i0, i1, first_pos, t0, t1, len;
  int need;  // tokens the tile's rows reach, before the table row's end cuts them
};
__device__ __forceinline__ TileRange tile_range(const PrefillArgs& args, int b, int tile, int part,
                                                int rows_per_tile) {
  const DecodeArgs& a = args.d;
  TileRange t;
  t.len = clamp_len(a.context_lens[b], a.max_len);
  t.r0 = args.query_start[b];
  t.nq = max(args.query_start[b + 1] - t.r0, 0);
  t.i0 = tile * rows_per_tile;
  t.i1 = min(t.i0 + rows_per_tile, t.nq);
  t.first_pos = t.len - t.nq;         // position of query token 0 (negative only if nq > len)
  // tokens the tile needs: 0 .. position of its last query token, none at
  // or past the end of the table row
  t.need = min(t.first_pos + t.i1, t.len);
  const int t_end = min(t.need, a.cap_len);
  t.t0 = 0;
  t.t1 = t_end;
  if (a.partition > 0) {
    t.t0 = part * a.partition;
    t.t1 = min(t.t0 + a.partition, t_end);
  }
  return t;
}


}  // namespace prefill
}  // namespace pa
