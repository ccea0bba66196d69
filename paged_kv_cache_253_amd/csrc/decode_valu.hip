// Paged decode attention on the vector ALUs.
//
// Used where the per-KV-head query group is too small for the matrix cores
// to pay (multi-head attention, G = 1) and for float32 caches.  Same work
// split and pipeline as the MFMA kernel: one wavefront per (sequence, KV
// head, partition), 32-token steps through the block table ("vLLM &
// High-Throughput Serving", section 2), next step's tiles in flight during
// the current one.
//
// QK: K tiles hold 16-byte chunks of the head dimension, token-major per
// chunk.  Lane l takes token l % 16 of a 16-token group and chunk rows
// 4j + l / 16, so each 16-byte load instruction reads four chunk rows of 16
// tokens (4 x 256 contiguous bytes); the four lanes of a token finish its dot
// product with two cross-row swaps, leaving every one of them the score.
// PV: V tiles are dimension-major, so a lane reads VPT consecutive tokens of
// one dimension per 16-byte load and accumulates them with the matching
// softmax weights, which it takes from a 32-entry LDS row per query head.
// Lanes sharing a dimension are summed once at the end.
#include "pa_device.hpp"
#include "pa_internal.hpp"
#include "pa_merge.hpp"
#include "pa_split.hpp"

namespace pa {
namespace {

constexpr int kStep = kStepTokens;
constexpr int kValuWavesPerCU = 4;  // balanced split: persistent wavefronts per CU

template <Elem E> struct ElemBytes;
template <> struct ElemBytes<Elem::F32> { static constexpr int v = 4; };
template <> struct ElemBytes<Elem::BF16> { static constexpr int v = 2; };
template <> struct ElemBytes<Elem::FP8> { static constexpr int v = 1; };
template <> struct ElemBytes<Elem::E5M2> { static constexpr int v = 1; };

// 16 bytes of cache elements -> floats
template <Elem E>
__device__ __forceinline__ void widen16(u32x4 w, float* out) {
  if constexpr (E == Elem::F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
  } else if constexpr (E == Elem::BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { out[2 * i] = bf16lo_to_f32(w[i]); out[2 * i + 1] = bf16hi_to_f32(w[i]); }
  } else if constexpr (E == Elem::E5M2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) bf8x4_to_f32(w[i], out + 4 * i);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) fp8x4_to_f32(w[i], out + 4 * i);
  }
}

template <typename QT>
__device__ __forceinline__ float load_q(const QT* p) { return (float)*p; }

// Where a range's result goes: the final output rows, or partial softmax
// states (row of query head g of the group = row0 + g * row_stride).
struct Target {
  bool final_out;
  size_t row0;
  size_t row_stride;
};

// Attention of the G query heads of KV head h of sequence b over tokens
// [t0, t1) (t0 a multiple of 32).  An empty range -- also one that lies past
// the table row -- writes zero output rows, or the empty softmax state
// (maximum -inf, exp-sum 0, zero row), which the merge weighs 0.
template <typename QT, Elem E, int D, int BS, int G>
__device__ __forceinline__ void attend(const DecodeArgs& a, const int b, const int h, const int t0,
                                       int t1, const Target tgt) {
  constexpr int ELT = ElemBytes<E>::v;
  constexpr int VEC = 16 / ELT;          // elements per 16-byte load
  constexpr int NC = D / VEC;            // 16-byte chunks per K row
  constexpr int CPL = NC / 4;            // K chunks per lane per 16-token group
  constexpr int NK = 2 * CPL;            // K loads per lane per step (two groups)
  constexpr int VPT = VEC;               // tokens per 16-byte V load
  constexpr int CPR = kStep / VPT;       // V loads per dimension per step
  constexpr int NV = D * CPR / 64;       // V loads per lane per step
  constexpr int DSTRIDE = 64 / CPR;      // dimension stride between a lane's V loads
  constexpr int TILE = BS * D * ELT;
  constexpr int BPS = kStep / BS;        // blocks per step
  static_assert(NC % 4 == 0 && NK >= 2 && NV >= 1 && kStep == 32, "shape");

  __shared__ float plds[2][G][kStep];

  const int lane = threadIdx.x;
  t1 = min(t1, a.cap_len);  // never walk past the table row
  QT* out = reinterpret_cast<QT*>(a.out);

  const int tc = lane % CPR;               // V token chunk of this lane
  if (t0 >= t1) {
    const bool dev = a.counters != nullptr;
    if (tc == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int d = i * DSTRIDE + lane / CPR;
          if (tgt.final_out)
            out[((size_t)b * a.num_q_heads + h * G + g) * D + d] = (QT)0.0f;
          else
            state_store(a.part_out + (tgt.row0 + (size_t)g * tgt.row_stride) * D + d, 0.f, dev);
        }
    }
    if (!tgt.final_out && lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const size_t row = tgt.row0 + (size_t)g * tgt.row_stride;
        state_store(a.part_max + row, -INFINITY, dev);
        state_store(a.part_sum + row, 0.f, dev);
      }
    }
    return;
  }

  // q slices of this lane (chunks 4j + kq) for every head of the group
  const int ktok = lane & 15;  // token within a 16-token group
  const int kq = lane >> 4;    // chunk row within each group of four
  float qf[G][CPL][VEC];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const QT* qrow = reinterpret_cast<const QT*>(a.q) + ((size_t)b * a.num_q_heads + h * G + g) * D;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
      for (int e = 0; e < VEC; ++e) qf[g][j][e] = load_q(qrow + (4 * j + kq) * VEC + e);
  }

  float kscale = 1.0f, vscale = 1.0f;
  if constexpr (E == Elem::FP8 || E == Elem::E5M2) { kscale = a.k_scale[h]; vscale = a.v_scale[h]; }
  const float c2 = a.scale * kscale * kLog2e;  // q.k -> log2 units

  // byte offsets inside the step's tiles: load m*CPL + j reads chunk row
  // 4j + kq of token 16m + ktok of the step
  uint32_t koff[NK];
  int kblk[NK];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int tok = 16 * m + ktok;
      kblk[m * CPL + j] = tok / BS;
      koff[m * CPL + j] = ((uint32_t)(4 * j + kq) * BS + (uint32_t)(tok % BS)) * 16;
    }
  const int vtok = tc * VPT;                 // first token of this lane's V chunk
  const int vblk = vtok / BS;
  const uint32_t voff = (uint32_t)(lane / CPR) * BS * ELT + (uint32_t)(vtok % BS) * ELT;

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

  struct Buf { u32x4 k[NK]; u32x4 v[NV]; };

  auto issue = [&](Buf& sb, int step) {
    const int lb0 = (t0 + step * kStep) / BS;
    const int lbl = min(lb0 + BPS - 1, lb_last);
    if (lbl - chunk_base >= 64) {
      chunk_base = lb0;
      tbl = (chunk_base + lane <= lb_last) ? table[chunk_base + lane] : 0;
    }
    int64_t tiles[BPS];
#pragma unroll
    for (int j = 0; j < BPS; ++j) tiles[j] = (phys_of(min(lb0 + j, lbl)) * a.num_kv_heads + h) * TILE;
#pragma unroll
    for (int i = 0; i < NK; ++i)
      sb.k[i] = stream_load<u32x4>(kc + tiles[kblk[i]] + koff[i]);
    const char* vp = vc + tiles[vblk] + voff;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      sb.v[i] = stream_load<u32x4>(vp + (size_t)i * DSTRIDE * BS * ELT);
  };

  float acc[G][NV];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[g][i] = 0.f;
  float m_run[G], l_run[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { m_run[g] = -INFINITY; l_run[g] = 0.f; }

  int parity = 0;
  auto compute = [&](Buf& sb, int step) {
    const int base = t0 + step * kStep;
    const bool partial = base + kStep > t1;
    float s[G][2];  // scores of tokens ktok and 16 + ktok of the step
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float dot[G];
#pragma unroll
      for (int g = 0; g < G; ++g) dot[g] = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        float kv[VEC];
        widen16<E>(sb.k[m * CPL + j], kv);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < VEC; ++e) dot[g] = fmaf(qf[g][j][e], kv[e], dot[g]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) s[g][m] = xlane<OpSum, 16, 32>(dot[g]);
    }
    bool valid[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) valid[m] = !partial || (base + 16 * m + ktok < t1);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      // scores in log2 units: z = s * c2, so exp(scale*q.k - max) = 2^(z - m)
      float mx = -INFINITY;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        s[g][m] = valid[m] ? __fmul_rn(s[g][m], c2) : -INFINITY;
        mx = fmaxf(mx, s[g][m]);
      }
      mx = xlane<OpMax, 1, 8>(mx);  // the 16 lanes of a row hold all 32 tokens
      const float m_new = fmaxf(m_run[g], mx);
      if (wave_any(m_new > m_run[g])) {
        const float alpha = exp2f(m_run[g] - m_new);
        l_run[g] *= alpha;
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[g][i] *= alpha;
        m_run[g] = m_new;
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const float p = valid[m] ? exp2f(s[g][m] - m_run[g]) : 0.f;
        l_run[g] += p;
        if (kq == 0) plds[parity][g][16 * m + ktok] = p;
      }
    }
    __syncthreads();
    // V: tokens vtok .. vtok+VPT-1 of the step, dimension i*DSTRIDE + lane/CPR
    const int vvalid = partial ? min(max(t1 - (base + vtok), 0), VPT) : VPT;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float vv[VPT];
      widen16<E>(sb.v[i], vv);
#pragma unroll
      for (int e = 0; e < VPT; ++e) vv[e] = (e < vvalid) ? vv[e] : 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float sum = acc[g][i];
#pragma unroll
        for (int e = 0; e < VPT; ++e) sum = fmaf(plds[parity][g][vtok + e], vv[e], sum);
        acc[g][i] = sum;
      }
    }
    parity ^= 1;
  };

  Buf bufA, bufB;
  issue(bufA, 0);
  for (int step = 0; step < nsteps; step += 2) {
    issue(bufB, min(step + 1, nsteps - 1));
    compute(bufA, step);
    if (step + 1 >= nsteps) break;
    issue(bufA, min(step + 2, nsteps - 1));
    compute(bufB, step + 1);
  }

  // ---- epilogue -------------------------------------------------------------
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float l_tot = xlane<OpSum, 1, 8>(l_run[g]);  // rows hold equal copies
    const float inv = vscale / l_tot;
    const int hq = h * G + g;
    const size_t row = tgt.row0 + (size_t)g * tgt.row_stride;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float v = acc[g][i];
      if constexpr (CPR > 1) v = xlane<OpSum, 1, CPR / 2>(v);
      v *= inv;
      if (tc == 0) {
        const int d = i * DSTRIDE + lane / CPR;
        if (tgt.final_out) out[((size_t)b * a.num_q_heads + hq) * D + d] = (QT)v;
        else state_store(a.part_out + row * D + d, v, a.counters != nullptr);
      }
    }
    if (!tgt.final_out && lane == 0) {
      state_store(a.part_max + row, m_run[g] * kLn2, a.counters != nullptr);  // natural units
      state_store(a.part_sum + row, l_tot, a.counters != nullptr);
    }
  }
}

template <typename QT, Elem E, int D, int BS, int G>
__global__ __launch_bounds__(64) void decode_valu_grid(const DecodeArgs a) {
  const int part = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int len = clamp_len(a.context_lens[b], a.max_len);
  if (a.partition == 0) {
    attend<QT, E, D, BS, G>(a, b, h, 0, len, Target{true, 0, 0});
    return;
  }
  const int t0 = part * a.partition;
  const int t1 = min(t0 + a.partition, len);
  if (t0 >= t1) return;
  const size_t row0 = ((size_t)b * a.num_q_heads + (size_t)h * G) * a.max_parts + part;
  attend<QT, E, D, BS, G>(a, b, h, t0, t1, Target{false, row0, (size_t)a.max_parts});
}

// MERGE: cut runs merged in this launch (a template parameter so that the
// other launches carry none of its code).
template <typename QT, Elem E, int D, int BS, int G, bool MERGE>
__global__ __launch_bounds__(64) void decode_valu_auto(const DecodeArgs a) {
  if (blockIdx.x == 0 && threadIdx.x == 0) a.header[kHdrSlices] = a.slices;  // for the merge
  const int r = slice_of_wave(blockIdx.x, a.slices);
  const Split sp = plan_split(a.context_lens, a.num_seqs, a.max_len, a.num_kv_heads, a.slices);
  int64_t g, g_end;
  slice_bounds(sp, r, g, g_end);
  MergeRec rec{0, 0, 0, 0};
  if (g >= g_end) {
    if (threadIdx.x == 0) store_merge_rec(a.header, r, rec);
    return;
  }
  int h = (int)(g / sp.per_head);
  int b, i0;
  locate_step(a.context_lens, a.num_seqs, a.max_len, g - (int64_t)h * sp.per_head, b, i0);
  bool first = true;
  CutPiece pieces[2] = {{0, 0, 0, 0, false}, {0, 0, 0, 0, false}};  // first and last runs
  while (g < g_end) {
    const int len = clamp_len(a.context_lens[b], a.max_len);
    const int n = steps_of_len(len);
    pieces[first ? 0 : 1] = CutPiece{g - i0, n, b, h, true};
    const int seg = (int)min((int64_t)(n - i0), g_end - g);
    const int t0 = i0 * kStep;
    const int t1 = min((i0 + seg) * kStep, len);
    if (i0 == 0 && seg == n) {
      attend<QT, E, D, BS, G>(a, b, h, t0, t1, Target{true, 0, 0});
    } else {
      const size_t row0 = ((size_t)r * 2 + (first ? 0 : 1)) * G;
      attend<QT, E, D, BS, G>(a, b, h, t0, t1, Target{false, row0, 1});
      if (i0 == 0) rec = merge_rec_of(sp, r, g, n, b, h, first ? 0 : 1);
    }
    g += seg;
    first = false;
    i0 = 0;
    if (++b == a.num_seqs) { b = 0; ++h; }
  }
  if (threadIdx.x == 0) store_merge_rec(a.header, r, rec);
  if constexpr (MERGE) {  // cut runs merged in this launch by the wavefront finishing last
    const MergeView v{a.out, a.part_out, a.part_max, a.part_sum, a.num_q_heads, G};
    arrive_and_merge<QT, D>(v, a.counters, sp, pieces);
  }
}

template <typename QT, Elem E, int D, int BS, int G>
hipError_t launch_one(const DecodeArgs& a, hipStream_t stream) {
  if (a.partition == kAuto) {
    DecodeArgs b = a;
    b.slices = a.cus * (a.waves_per_cu ? a.waves_per_cu : kValuWavesPerCU);
    if (a.counters)
      hipLaunchKernelGGL((decode_valu_auto<QT, E, D, BS, G, true>), dim3(b.slices), dim3(64), 0, stream, b);
    else
      hipLaunchKernelGGL((decode_valu_auto<QT, E, D, BS, G, false>), dim3(b.slices), dim3(64), 0, stream, b);
  } else {
    const int parts = a.partition ? a.max_parts : 1;
    dim3 grid(parts, a.num_kv_heads, a.num_seqs);
    hipLaunchKernelGGL((decode_valu_grid<QT, E, D, BS, G>), grid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

template <typename QT, Elem E, int D, int BS>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  switch (a.group) {
    case 1: return launch_one<QT, E, D, BS, 1>(a, stream);
    case 2: return launch_one<QT, E, D, BS, 2>(a, stream);
    case 4: return launch_one<QT, E, D, BS, 4>(a, stream);
    case 8: return launch_one<QT, E, D, BS, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename QT, Elem E>
hipError_t launch_shape(const DecodeArgs& a, int head_dim, int block_size, hipStream_t s) {
  if (head_dim == 128 && block_size == 16) return launch_g<QT, E, 128, 16>(a, s);
  if (head_dim == 128 && block_size == 32) return launch_g<QT, E, 128, 32>(a, s);
  if (head_dim == 64 && block_size == 16) return launch_g<QT, E, 64, 16>(a, s);
  if (head_dim == 64 && block_size == 32) return launch_g<QT, E, 64, 32>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_valu(const DecodeArgs& a, Elem q, Elem cache, int head_dim,
                              int block_size, hipStream_t stream) {
  if (q == Elem::F32 && cache == Elem::F32) return launch_shape<float, Elem::F32>(a, head_dim, block_size, stream);
  if (q == Elem::BF16 && cache == Elem::BF16) return launch_shape<__bf16, Elem::BF16>(a, head_dim, block_size, stream);
  if (q == Elem::BF16 && cache == Elem::FP8) return launch_shape<__bf16, Elem::FP8>(a, head_dim, block_size, stream);
  if (q == Elem::BF16 && cache == Elem::E5M2) return launch_shape<__bf16, Elem::E5M2>(a, head_dim, block_size, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
