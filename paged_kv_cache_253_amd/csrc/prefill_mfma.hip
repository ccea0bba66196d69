// Attention of several new query tokens per sequence over the paged cache,
// on the matrix cores: chunked prefill ("vLLM & High-Throughput Serving",
// section 4: a long prompt fed in chunks next to the decodes) and
// speculative verification ("AI Inference Serving at Scale", section 7:
// the target model scores K drafted tokens in one pass).  Sequence b's
// query tokens are its last Q_b cached tokens; the one at position p
// attends to cached tokens 0..p.
//
// One wavefront owns (context partition, KV head, sequence, query tile).
// The MFMA columns are (query token, query head) pairs: 16 * NT columns,
// i.e. 16 * NT / G query tokens of the group's G heads, in NT column tiles
// of 16.  Each 32-token step loads K and V once and uses them for every
// column tile:
//
//   S^T = K Q^T     2 * (head_dim / 32) * NT MFMAs (rows = tokens)
//   causal mask     token t is kept for a column iff t <= its position
//   online softmax  per column, in the result registers (as the decode)
//   O^T += V^T P^T  (head_dim / 16) * NT MFMAs
//
// The step pipeline, block-table walk and operand layouts are the decode
// kernel's (pa_mfma.hpp).  A tile's context ends at its last query token,
// so later tiles of a long chunk read more of the cache than earlier ones.
#include "pa_device.hpp"
#include "pa_internal.hpp"
#include "pa_mfma.hpp"
#include "pa_split.hpp"

namespace pa {
namespace {

using namespace mfma;

template <int CK, int D, int BS, int NT>
__global__ __launch_bounds__(64) void prefill_mfma(const PrefillArgs args) {
  constexpr bool FP8 = one_byte<CK>();
  using C = Cfg<CK, D, BS>;
  const DecodeArgs& a = args.d;
  const int part = blockIdx.x;
  const int tile = blockIdx.y / a.num_kv_heads;
  const int h = blockIdx.y % a.num_kv_heads;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int G = a.group;              // a power of two, <= 16 * NT
  const int rows_per_tile = 16 * NT / G;

  const int len = clamp_len(a.context_lens[b], a.max_len);
  const int r0 = args.query_start[b];
  int nq = args.query_start[b + 1] - r0;
  nq = nq < 0 ? 0 : nq;
  const int i0 = tile * rows_per_tile;
  if (i0 >= nq) return;
  const int i1 = min(i0 + rows_per_tile, nq);
  const int first_pos = len - nq;     // position of query token 0 (negative only if nq > len)
  // tokens this tile needs: 0 .. position of its last query token
  int t_end = min(first_pos + i1, len);
  t_end = min(t_end, a.cap_len);
  int t0 = 0, t1 = t_end;
  if (a.partition > 0) {
    t0 = part * a.partition;
    t1 = min(t0 + a.partition, t_end);
    if (t0 >= t1) return;             // no row of the tile reaches this partition
  }

  // ---- columns: query token qi = i0 + c / G, head g = c % G ---------------
  int pos[NT];
  bool cvalid[NT];
  size_t qrow[NT];                    // row of q / out (query token * Hq + query head)
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    const int c = ct * 16 + col;
    const int qi = i0 + c / G;
    cvalid[ct] = qi < i1;
    pos[ct] = first_pos + qi;
    qrow[ct] = (size_t)(r0 + (cvalid[ct] ? qi : i0)) * a.num_q_heads + (size_t)h * G + (c % G);
  }

  bf16x8 qop[NT][C::kChunks];
  {
    const __bf16* qbase = reinterpret_cast<const __bf16*>(a.q);
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
      for (int c = 0; c < C::kChunks; ++c) {
        const int d0 = q_dim<CK, D>(grp, c);
        if (cvalid[ct]) {
          qop[ct][c] = *reinterpret_cast<const bf16x8*>(qbase + qrow[ct] * D + d0);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) qop[ct][c][e] = (__bf16)0.0f;
        }
      }
  }

  float kscale = 1.0f, vscale = 1.0f;
  if constexpr (FP8) { kscale = a.k_scale[h]; vscale = a.v_scale[h]; }
  const float c2 = a.scale * kscale * kLog2e;  // q.k -> log2 units

  f32x4 acc[NT][C::kDTiles];
  f32x4 accb[NT];  // INT4: column sums of the PV weights
  float m_run[NT], l_run[NT], qbias[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    m_run[ct] = -INFINITY;
    l_run[ct] = 0.f;
    accb[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    qbias[ct] = 0.f;
    if constexpr (C::I4) qbias[ct] = q_bias<C::kChunks>(qop[ct]);
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt) acc[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  if (t0 < t1) {
    // ---- per-lane byte offsets inside a step's tiles (as the decode) -------
    const LaneOffsets<CK, D, BS> lo(grp, col);
    const char* kc = reinterpret_cast<const char*>(a.k_cache);
    const char* vc = reinterpret_cast<const char*>(a.v_cache);
    const int32_t* table = a.block_tables + (size_t)b * a.max_blocks;
    const int nsteps = (t1 - t0 + kStep - 1) / kStep;
    const int lb_first = t0 / BS;
    const int lb_last = (t1 - 1) / BS;
    int chunk_base = lb_first;
    int tbl = (chunk_base + lane <= lb_last) ? table[chunk_base + lane] : 0;
    auto phys_of = [&](int lb) -> int64_t {
      int p = readlane(tbl, lb - chunk_base);
      return (p < 0 || (int64_t)p >= a.num_blocks) ? 0 : (int64_t)p;
    };

    auto issue = [&](StepBuf<CK, D, BS>& sb, int step) {
      const int lb0 = (t0 + step * kStep) / BS;
      const int lb1 = min(lb0 + C::kBlocksPerStep - 1, lb_last);
      if (lb1 - chunk_base >= 64) {  // slide the table window
        chunk_base = lb0;
        tbl = (chunk_base + lane <= lb_last) ? table[chunk_base + lane] : 0;
      }
      const int64_t p0 = phys_of(lb0);
      const int64_t p1 = (C::kBlocksPerStep == 2) ? phys_of(lb1) : p0;
      const int64_t tile0 = (p0 * a.num_kv_heads + h) * C::kTile;
      const int64_t tile1 = (p1 * a.num_kv_heads + h) * C::kTile;
      load_step(sb, kc, vc, tile0, tile1, lo, grp);
    };

    auto compute = [&](StepBuf<CK, D, BS>& sb, int step) {
      const int base = t0 + step * kStep;
      f32x4 s0[NT], s1[NT];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) { s0[ct] = f32x4{0.f, 0.f, 0.f, 0.f}; s1[ct] = s0[ct]; }
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
        const int lim = min(t1 - 1, pos[ct]);  // last token this column may see here
        float z[8] = {s0[ct][0], s0[ct][1], s0[ct][2], s0[ct][3],
                      s1[ct][0], s1[ct][1], s1[ct][2], s1[ct][3]};
        qk_scores<CK>(z, sb, qbias[ct]);
        // the step is full for every real column unless one stops inside it
        const bool partial = wave_any(cvalid[ct] && base + kStep - 1 > lim);
        bool ok[8];
        if (partial) {
#pragma unroll
          for (int i = 0; i < 8; ++i) ok[i] = cvalid[ct] && base + qk_token(grp, i) <= lim;
        }
        pop[ct] = softmax_step<CK, C::kDTiles>(z, partial, ok, sb, c2, m_run[ct], l_run[ct], acc[ct],
                                               accb[ct]);
      }
#pragma unroll
      for (int dt = 0; dt < C::kDTiles; ++dt) {
        const bf16x8 vop = v_operand<CK>(sb.v[dt]);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
          acc[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[ct], acc[ct][dt], 0, 0, 0);
      }
      if constexpr (C::I4) {
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
          accb[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_operand(), pop[ct], accb[ct], 0, 0, 0);
      }
    };

    StepBuf<CK, D, BS> bufA, bufB;
    issue(bufA, 0);
    for (int step = 0; step < nsteps; step += 2) {
      issue(bufB, min(step + 1, nsteps - 1));
      compute(bufA, step);
      if (step + 1 >= nsteps) break;
      issue(bufA, min(step + 2, nsteps - 1));
      compute(bufB, step + 1);
    }
  }

  // ---- epilogue: one row per valid column ----------------------------------
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    const float l_tot = xlane<OpSum, 16, 32>(l_run[ct]);
    if (!cvalid[ct]) continue;
    const float inv = l_tot > 0.f ? vscale / l_tot : 0.f;  // a row with no token writes zeros
    if constexpr (C::I4) {  // remove the operand bias: 136 * sum_t p(t) s_v(t)
#pragma unroll
      for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[ct][dt][r] = fmaf(-kI4Bias, accb[ct][0], acc[ct][dt][r]);
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
        a.part_max[row] = m_run[ct] * (c2 * kLn2);  // natural units: scale * q.k
        a.part_sum[row] = l_tot;
      }
    }
  }
}

template <int CK, int D, int BS, int NT>
hipError_t launch_nt(const PrefillArgs& p, hipStream_t stream) {
  constexpr bool FP8 = one_byte<CK>();
  const DecodeArgs& a = p.d;
  const Elem e = CK == kI4 ? Elem::I4 : (FP8 ? Elem::FP8 : Elem::BF16);  // FP8 kinds alike
  const int tiles = prefill_query_tiles(a.group, p.max_query_len, prefill_max_column_tiles(e, D));
  const int parts = a.partition ? a.max_parts : 1;
  if ((long long)tiles * a.num_kv_heads > 65535) return hipErrorInvalidValue;
  dim3 grid(parts, tiles * a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((prefill_mfma<CK, D, BS, NT>), grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

template <int CK, int D, int BS>
hipError_t launch_shape(const PrefillArgs& p, hipStream_t stream) {
  constexpr int kMaxNT = (!one_byte<CK>() && D == 128) ? 2 : 4;  // as prefill_max_column_tiles
  switch (prefill_column_tiles(p.d.group, p.max_query_len, kMaxNT)) {
    case 1: return launch_nt<CK, D, BS, 1>(p, stream);
    case 2: return launch_nt<CK, D, BS, 2>(p, stream);
    default:
      if constexpr (kMaxNT >= 4) return launch_nt<CK, D, BS, 4>(p, stream);
      return hipErrorInvalidValue;
  }
}

template <int CK>
hipError_t dispatch(const PrefillArgs& p, int head_dim, int block_size, hipStream_t s) {
  if (head_dim == 128 && block_size == 16) return launch_shape<CK, 128, 16>(p, s);
  if (head_dim == 128 && block_size == 32) return launch_shape<CK, 128, 32>(p, s);
  if (head_dim == 64 && block_size == 16) return launch_shape<CK, 64, 16>(p, s);
  if (head_dim == 64 && block_size == 32) return launch_shape<CK, 64, 32>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs& p, Elem cache, int head_dim, int block_size,
                               hipStream_t stream) {
  if (cache == Elem::BF16) return dispatch<kBF16>(p, head_dim, block_size, stream);
  if (cache == Elem::FP8) return dispatch<kE4M3>(p, head_dim, block_size, stream);
  if (cache == Elem::E5M2) return dispatch<kE5M2>(p, head_dim, block_size, stream);
  if (cache == Elem::I4) return dispatch<kI4>(p, head_dim, block_size, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
