// Paged decode attention on the matrix cores (bf16, FP8 or INT4 KV cache).
//
// One wavefront owns one (sequence, KV head, context partition).  It walks
// the partition in steps of 32 tokens (two 16-token blocks or one 32-token
// block), reaching each block through the sequence's block table (the
// block-table equation of "vLLM & High-Throughput Serving", section 2), and
// keeps the next step's K and V tiles in flight while it computes the
// current one.  Per step:
//
//   S^T = K q^T      two v_mfma_f32_16x16x32_bf16 chains (tokens 0-15 and
//                    16-31 of the step) over head_dim; rows = tokens,
//                    columns = the G query heads of this KV head (zero
//                    columns beyond G).  K tiles hold 16-byte head-dim
//                    chunks token-major, so the A operand of one chunk
//                    (16 tokens x 4 chunk rows) is one 1 KiB run at B = 16
//   online softmax   per query head, in the MFMA output registers; the step
//                    maximum needs two permlane swaps, no LDS
//   O^T += V^T P^T   head_dim/16 MFMAs; V tiles are stored dimension-major
//                    so each lane's 8 tokens of one dimension are one 16-byte
//                    load; P comes from the S^T registers through one
//                    permlane32 and one permlane16 swap per packed word
//
// MFMA operand layouts (16x16x32, wave64; checked on hardware): lane l holds
// row/column l % 16 and k-slots 8*(l/16) .. 8*(l/16)+7 of A and B; the f32
// result row is 4*(l/16) + r (r = 0..3), column l % 16.  QK row i of group
// m is token 16*m + i, so lane l holds scores of tokens 4*(l/16) + r and
// 16 + 4*(l/16) + r; its PV k-slots need tokens 8*(l/16) .. +7, which the
// two swaps bring in from the lanes 16 and 32 away (p_operand).
//
// The same head mapping (column = query head) holds in S^T and O^T, so every
// softmax statistic a lane keeps is the one its output registers need.
//
// Two entry kernels share the per-range body: a grid of one wavefront per
// (partition, KV head, sequence), and a persistent grid that walks balanced
// slices of the whole batch (see pa_split.hpp).
#include "pa_device.hpp"
#include "pa_internal.hpp"
#include "pa_merge.hpp"
#include "pa_mfma.hpp"
#include "pa_split.hpp"

#include <type_traits>

namespace pa {
namespace {

using namespace mfma;

// Where a range's result goes: the final output rows, or partial softmax
// states (rows of part_out/part_max/part_sum; row of query head g of the
// group = row0 + g * row_stride).
struct Target {
  bool final_out;
  size_t row0;
  size_t row_stride;
};

// Attention of the G query heads of KV head h of sequence b over tokens
// [t0, t1) (t0 a multiple of 32).  An empty range -- also one that lies past
// the table row -- writes zero output rows, or the empty softmax state
// (maximum -inf, exp-sum 0, zero row), which the merge weighs 0.
template <int CK, int D, int BS>
__device__ __forceinline__ void attend(const DecodeArgs& a, const int b, const int h, const int t0,
                                       int t1, const Target tgt) {
  constexpr bool FP8 = one_byte<CK>();
  using C = Cfg<CK, D, BS>;
  t1 = min(t1, a.cap_len);  // never walk past the table row
  const int lane = threadIdx.x;
  const int col = lane & 15;   // query head within the group (QK/PV column)
  const int grp = lane >> 4;   // k-slot group: tokens 8*grp .. 8*grp+7 of a step
  const int G = a.group;
  const int hq = h * G + col;
  const bool head_ok = col < G;

  if (t0 >= t1) {
    if (head_ok && tgt.final_out) {
      __bf16* o = reinterpret_cast<__bf16*>(a.out) + ((size_t)b * a.num_q_heads + hq) * D;
#pragma unroll
      for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[dt * 16 + grp * 4 + r] = (__bf16)0.0f;
    } else if (head_ok) {
      const size_t row = tgt.row0 + (size_t)col * tgt.row_stride;
      float* o = a.part_out + row * D;
#pragma unroll
      for (int dt = 0; dt < C::kDTiles; ++dt)
        *reinterpret_cast<f32x4*>(o + dt * 16 + grp * 4) = f32x4{0.f, 0.f, 0.f, 0.f};
      if (grp == 0) {
        a.part_max[row] = -INFINITY;
        a.part_sum[row] = 0.f;
      }
    }
    return;
  }

  // ---- q operand (B of QK): head `col`, the 8 dims of k-slot group `grp` --
  bf16x8 qop[C::kChunks];
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(a.q) + ((size_t)b * a.num_q_heads + hq) * D;
#pragma unroll
    for (int c = 0; c < C::kChunks; ++c) {
      // dims of chunk c held by this lane; K rows use the same map
      const int d0 = q_dim<CK, D>(grp, c);
      if (head_ok) {
        qop[c] = *reinterpret_cast<const bf16x8*>(qrow + d0);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qop[c][e] = (__bf16)0.0f;
      }
    }
  }

  float kscale = 1.0f, vscale = 1.0f;
  if constexpr (FP8) { kscale = a.k_scale[h]; vscale = a.v_scale[h]; }
  const float c2 = log2_factor(a.scale, kscale);  // q.k -> log2 units
  float qbias = 0.f;
  if constexpr (C::I4) qbias = q_bias<C::kChunks>(qop);

  // ---- per-lane byte offsets inside the step's tiles ----------------------
  // K: QK row col of group m is token 16*m + col of the step; load j of the
  // group reads chunk row 4*j + grp (INT4: the chunk row and half holding
  // dimensions D/4*grp ..).  V: dimension dt*16 + col, tokens 8*grp .. +7.
  const LaneOffsets<CK, D, BS> lo(grp, col);

  const char* kc = reinterpret_cast<const char*>(a.k_cache);
  const char* vc = reinterpret_cast<const char*>(a.v_cache);
  const int32_t* table = a.block_tables + (size_t)b * a.max_blocks;
  const int nsteps = (t1 - t0 + kStep - 1) / kStep;
  const int lb_first = t0 / BS;
  const int lb_last = (t1 - 1) / BS;  // last logical block with a token in range

  // block-table window: lane i holds entry chunk_base + i
  int chunk_base = lb_first;
  int tbl = (chunk_base + lane <= lb_last) ? table[chunk_base + lane] : 0;

  auto phys_of = [&](int lb) -> int64_t {
    int p = readlane(tbl, lb - chunk_base);
    return (p < 0 || (int64_t)p >= a.num_blocks) ? 0 : (int64_t)p;
  };

  auto issue = [&](StepBuf<CK, D, BS>& sb, int step) {
    const int lb0 = (t0 + step * kStep) / BS;
    const int lb1 = min(lb0 + C::kBlocksPerStep - 1, lb_last);
    if (lb1 - chunk_base >= 64) {  // slide the table window (long unsplit ranges)
      chunk_base = lb0;
      tbl = (chunk_base + lane <= lb_last) ? table[chunk_base + lane] : 0;
    }
    const int64_t p0 = phys_of(lb0);
    const int64_t p1 = (C::kBlocksPerStep == 2) ? phys_of(lb1) : p0;
    const int64_t tile0 = (p0 * a.num_kv_heads + h) * C::kTile;
    const int64_t tile1 = (p1 * a.num_kv_heads + h) * C::kTile;
    load_step(sb, kc, vc, tile0, tile1, lo, grp);
  };

  f32x4 acc[C::kDTiles];
#pragma unroll
  for (int dt = 0; dt < C::kDTiles; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 accb = {0.f, 0.f, 0.f, 0.f};  // INT4: column sums of the PV weights
  LaneSoftmax st;  // online softmax of head `col` (lazy rescaling)
  st.reset(c2);

  auto compute = [&](StepBuf<CK, D, BS>& sb, int step) {
    const int base = t0 + step * kStep;
    const bool partial = base + kStep > t1;
    f32x4 s0 = qk_init<CK>(qbias), s1 = s0;
#pragma unroll
    for (int c = 0; c < C::kChunks; ++c) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<CK>(sb, 0, c), qop[c], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<CK>(sb, 1, c), qop[c], s1, 0, 0, 0);
    }
    float z[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    qk_scores<CK>(z, sb);
    // partial step: the lane's scores at token offsets <= zlim are in range
    const int zlim = t1 - base - 1 - 4 * grp;
    if (partial) {
      const int vvalid = min(max(t1 - (base + 8 * grp), 0), 8);  // PV k-slots: tokens 8*grp .. +7
#pragma unroll
      for (int dt = 0; dt < C::kDTiles; ++dt) mask_v<CK>(sb.v[dt], vvalid);
    }
    const bf16x8 pop = softmax_step<CK, C::kDTiles>(z, partial, zlim, sb, c2, st, acc, accb);
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt)
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v_operand<CK>(sb.v[dt]), pop, acc[dt], 0, 0, 0);
    if constexpr (C::I4) accb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_operand(), pop, accb, 0, 0, 0);
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

  // ---- epilogue -------------------------------------------------------------
  lazy_settle<C::kDTiles, false>(st, c2, acc, accb);
  const float l_tot = xlane<OpSum, 16, 32>(st.l_run);
  const float inv = vscale / l_tot;
  if constexpr (C::I4) {  // remove the operand bias: 136 * sum_t p(t) s_v(t)
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[dt][r] = fmaf(-kI4Bias, accb[0], acc[dt][r]);
  }
  if (!head_ok) return;
  if (tgt.final_out) {
    __bf16* o = reinterpret_cast<__bf16*>(a.out) + ((size_t)b * a.num_q_heads + hq) * D;
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt) {
      bf16x2 lo, hi;
      lo[0] = (__bf16)(acc[dt][0] * inv); lo[1] = (__bf16)(acc[dt][1] * inv);
      hi[0] = (__bf16)(acc[dt][2] * inv); hi[1] = (__bf16)(acc[dt][3] * inv);
      u32x2 w = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
      *reinterpret_cast<u32x2*>(o + dt * 16 + grp * 4) = w;
    }
  } else {
    const size_t row = tgt.row0 + (size_t)col * tgt.row_stride;
    float* o = a.part_out + row * D;
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt)
      *reinterpret_cast<f32x4*>(o + dt * 16 + grp * 4) = acc[dt] * inv;
    if (grp == 0) {
      a.part_max[row] = st.m_run * (c2 * kLn2);  // natural units: scale * q.k
      a.part_sum[row] = l_tot;
    }
  }
}

// One wavefront per (partition, KV head, sequence); unsplit launches have a
// single partition covering the whole context.
template <int CK, int D, int BS>
__global__ __launch_bounds__(64) void decode_mfma_grid(const DecodeArgs a) {
  const int part = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int len = clamp_len(a.context_lens[b], a.max_len);
  if (a.partition == 0) {
    attend<CK, D, BS>(a, b, h, 0, len, Target{true, 0, 0});
    return;
  }
  const int t0 = part * a.partition;
  const int t1 = min(t0 + a.partition, len);
  if (t0 >= t1) return;  // the sequence has no such partition
  const size_t row0 = ((size_t)b * a.num_q_heads + (size_t)h * a.group) * a.max_parts + part;
  attend<CK, D, BS>(a, b, h, t0, t1, Target{false, row0, (size_t)a.max_parts});
}

// ---------------------------------------------------------------------------
// Balanced split: one persistent wavefront per SIMD streams its slice of the
// batch as one sequence of 32-token steps, whatever runs (sequence, KV head)
// the steps belong to.  A ring of kRing step slots holds the K, V and q tiles
// of the next steps; the issue side runs kRing - 1 steps ahead of the
// compute side, across run boundaries, so the memory pipeline never drains
// inside a slice.  Every slot issues the same loads, so the wait before a
// slot's compute is exact.  Block-table entries and lengths are read with
// scalar loads (separate wait counter from the tile loads).  A run the slice
// covers whole is finished here; the slice's first and last runs, when cut
// by a slice boundary, leave partial states in rows (2r)*G.. and (2r+1)*G..,
// merged by a separate launch or, when the launch has merge counters, by the
// wavefront that finishes a cut run's last piece (pa_merge.hpp).
// ---------------------------------------------------------------------------

constexpr int kFirst = 1, kLast = 2, kFinal = 4;
// Ring of 3 step slots: each wavefront keeps up to 3 steps of tiles in
// flight (60 loads for bf16 head_dim 128, at the hardware's limit of 63
// outstanding vector memory operations per wavefront, so a deeper ring adds
// nothing but registers; measured equal to a ring of 4 on MI355X).
// Wavefronts per compute unit by step size (measured on MI355X): with 16 KiB
// steps (bf16, head_dim 128) two wavefronts per CU read the scattered tiles
// fastest; fewer, deeper streams beat more, shallower ones there.  Smaller
// steps (FP8 or head_dim 64) do best with four.
#ifndef PA_STREAM_RING
#define PA_STREAM_RING 3  // build-time tuning knob
#endif
constexpr int kRing = PA_STREAM_RING;

// INT4 steps (4.25 KiB at head_dim 128) are the smallest and carry the most
// VALU work per byte: two wavefronts per SIMD (8 per CU, 240 VGPRs each)
// let one wavefront's widening and softmax overlap the other's loads.
template <int CK, int D>
constexpr int stream_waves_per_cu() {
  if (CK == kI4) return 8;
  return kStep * 2 * D * (CK == kBF16 ? 2 : 1) >= 16 * 1024 ? 2 : 4;
}
template <int CK>
constexpr int stream_waves_per_simd() { return CK == kI4 ? 2 : 1; }

// Persistent wavefronts per CU of a launch: the kernel's own choice, except
// multi-head batches (G = 1: one query head per 16-column MFMA, so a step
// carries little work per byte), which stream best with one wavefront per
// SIMD (measured on MI355X, 64-head bf16 batches: 518 vs 535 us at two per
// CU), or the tuning override.
template <int CK, int D>
int launch_waves_per_cu(const DecodeArgs& a) {
  if (a.waves_per_cu) return a.waves_per_cu;
  const int own = stream_waves_per_cu<CK, D>();
  return a.group == 1 && own < 4 ? 4 : own;
}
static_assert(stream_waves_per_cu<kI4, 128>() <= kAutoMaxWavesPerCU, "workspace bound");

typedef const __attribute__((address_space(4))) int32_t* const_i32;
typedef const __attribute__((address_space(4))) float* const_f32;

// The newest token of a run (position L - 1) when a decode step appends it
// itself (bf16 cache): this lane's share of its K and V rows -- the k-slot
// dimensions of each QK chunk, as q, and dimension 16 * dt + col of V --
// its place in the step, and where it is written.
template <int D, bool ON>
struct NewRows {};
template <int D>
struct NewRows<D, true> {
  u32x4 k[D / 32];
  uint32_t v[D / 16];
  int pos;       // token of the step, -1 if the step holds no newest token
  int off;       // offset in its block
  int64_t tile;  // byte offset of its (block, KV head) tile in either pool
};

// Where a step's query operands come from.  Per step (loaded with the
// step's tiles): simple, and no wait at a segment's start, but the loads
// repeat on every step and every slot of the ring holds a copy.  Per
// segment (INT4: one copy, loaded when a segment's first step is about to
// compute): an INT4 step's tiles are a quarter of a bf16 step's, so the
// repeated query loads were as many bytes through the vector memory path as
// the tiles themselves and the copies held the registers the kernel needs;
// the price is one wait for the ring's outstanding loads per segment, which
// costs the bf16 decode more than it saves (measured on MI355X, 70B-shaped
// batch: INT4 127 -> 113 us, bf16 283 -> 341 us).
template <int CK>
constexpr bool q_per_segment() { return CK == kI4; }

template <int CK, int D, bool PER_STEP>
struct StepQ { bf16x8 q[D / 32]; };
template <int CK, int D>
struct StepQ<CK, D, false> {};

template <int CK, int D, int BS, bool APPEND, bool PK>
struct Slot : std::conditional_t<PK, PkBuf<D, BS>, StepBuf<CK, D, BS>>,
              StepQ<CK, D, !q_per_segment<CK>()> {
  using C = Cfg<CK, D, BS>;
  NewRows<D, APPEND> nw;
  // segment descriptor (wave-uniform)
  int base;   // first token of the step
  int t1;     // end of the run's tokens inside this segment
  int b, h;
  int flags;  // kFirst / kLast step of its segment; kFinal output (else partial state)
  int row0;   // partial state: row of the group's first query head
  bool real;  // false: a filler step (loads repeated, nothing computed)
};

// APPEND (bf16 cache, balanced split): the launch also appends every
// sequence's newest token, at the slot its block table gives (pa_decode_append).
// The wavefront that computes a run's last step loads that token's K and V
// rows with the step, puts them into the step's operand registers in place
// of the pool's bytes, and writes them to the pool after its ring has
// drained: no other step reads that block, so the result is bit for bit that
// of an append launch before the decode, without its launch and without
// partial-line stores in the middle of the stream.
//
// MERGE (PA_PARTITION_AUTO_MERGED): cut runs are merged in this launch by
// the wavefront that finishes a run's last piece (pa_merge.hpp).  FIXED:
// fixed partitions (slices of whole partitions).  PK: INT4 with G <= 8,
// column-packed steps (pa_mfma.hpp).  Template parameters so that each
// launch carries only its own mode's code.
template <int CK, int D, int BS, bool APPEND, bool MERGE, bool FIXED, bool PK = false>
__global__ __launch_bounds__(64)
__attribute__((amdgpu_waves_per_eu(stream_waves_per_simd<CK>(), stream_waves_per_simd<CK>())))
void decode_mfma_stream(const DecodeArgs a) {
  constexpr bool FP8 = one_byte<CK>();
  using C = Cfg<CK, D, BS>;
  using S = Slot<CK, D, BS, APPEND, PK>;
  static_assert(!APPEND || CK == kBF16, "the decode appends only into bf16 caches");
  static_assert(!PK || (CK == kI4 && !FIXED), "column packing is for INT4 balanced launches");
  static_assert(!(APPEND && MERGE), "the appending decode uses the separate merge");
  static_assert(!(FIXED && (APPEND || MERGE)), "fixed partitions neither append nor merge");
  const int lane = threadIdx.x;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int G = a.group;
  const int W = a.slices;
  // fixed partitions: steps per partition, and the workspace row stride of
  // a group's query heads (their rows are max_parts apart); 0 / 1 balanced
  const int pst = FIXED ? a.partition / kStepTokens : 0;
  const int rstride = FIXED ? a.max_parts : 1;
  if (blockIdx.x == 0 && lane == 0 && !pst) a.header[kHdrSlices] = W;  // for the merge
  const Split sp = plan_split(a.context_lens, a.num_seqs, a.max_len, a.num_kv_heads, W, pst);
  const int r = slice_of_wave(blockIdx.x, W);
  int64_t g0, g_end;
  slice_bounds(sp, r, g0, g_end);
  if (g0 >= g_end) {
    if (lane == 0 && !pst) store_merge_rec(a.header, r, MergeRec{0, 0, 0, 0});
    return;
  }

  const const_i32 lens = (const_i32)a.context_lens;
  const const_i32 tables = (const_i32)a.block_tables;

  // ---- issue-side cursor over the slice's runs ----------------------------
  // Balanced: `left` counts the slice's steps not yet issued.  Fixed
  // partitions: the slice is whole partitions; `left` counts those not yet
  // started, and each partition is one segment of its run.
  int64_t left = g_end - g0;
  int cb, ci;                 // run (sequence cb, KV head ch) and its step index
  int ch = (int)(g0 / sp.per_head);
  locate_step(a.context_lens, a.num_seqs, a.max_len, g0 - (int64_t)ch * sp.per_head, cb, ci, pst);
  int clen = clamp_len(lens[cb], a.max_len);
  int cn = steps_of_len(clen);
  int cpart = 0;              // fixed partitions: the current partition of the run
  int cseg_start, cseg_end;   // the segment (run part inside the slice), in run steps
  int cflags_run, crow0;
  if (pst) {
    cpart = ci;
    ci = cpart * pst;
    cseg_start = ci;
    cseg_end = min(ci + pst, cn);
    cflags_run = 0;
    crow0 = (cb * a.num_q_heads + ch * G) * a.max_parts + cpart;
    --left;
  } else {
    cseg_start = ci;
    cseg_end = (int)min((int64_t)cn, (int64_t)ci + left);
    cflags_run = (ci == 0 && cseg_end == cn) ? kFinal : 0;
    crow0 = r * 2 * G;  // the slice's first run -> rows (2r)*G..
  }
  int pending = 0;        // real steps issued and not yet computed
  // merge record: only the slice's last run can be cut by the next boundary
  MergeRec rec{0, 0, 0, 0};
  if (!pst && ci == 0 && cseg_end < cn) rec = merge_rec_of(sp, r, g0, cn, cb, ch, 0);
  // the slice's first and last runs (first step, steps, sequence, KV head):
  // the pieces this wavefront may hold of cut runs, for a merge in the launch
  CutPiece pieces[2] = {{g0 - ci, cn, cb, ch, true}, {0, 0, 0, 0, false}};

  // per-lane offsets inside a step's tiles (see attend)
  const LaneOffsets<CK, D, BS> lo(grp, col);
  const PkOffsets<D, BS> plo(grp, col);
  // lanes past the group read a real row; unused
  const int qhead = min(PK ? (col & 7) : col, G - 1);
  const bool pk_on = pk_active(grp, col);  // packed: the lane's q operand is its head's
  const char* kc = reinterpret_cast<const char*>(a.k_cache);
  const char* vc = reinterpret_cast<const char*>(a.v_cache);
  const __bf16* qbase = reinterpret_cast<const __bf16*>(a.q);

  int64_t tile0 = 0, tile1 = 0;  // the last real step's tiles (filler steps reload them)
  const __bf16* qp = qbase;
  constexpr bool QSEG = q_per_segment<CK>();
  constexpr int kQOps = PK ? D / 16 : C::kChunks;  // q operands (one per QK MFMA of a token group)
  bf16x8 qseg[QSEG ? kQOps : 1];  // per segment: the computing segment's query

  auto issue = [&](S& sl) {
    const bool real = pst ? (ci < cseg_end || left > 0) : left > 0;
    sl.real = real;
    if constexpr (APPEND) sl.nw.pos = -1;
    if (real) {
      if (pst && ci == cseg_end) {  // next partition of the slice
        --left;
        if (++cpart * pst >= cn) {  // next run that has a partition
          do {
            if (++cb == a.num_seqs) { cb = 0; ++ch; }
            clen = clamp_len(lens[cb], a.max_len);
          } while (clen == 0);
          cn = steps_of_len(clen);
          cpart = 0;
        }
        ci = cpart * pst;
        cseg_start = ci;
        cseg_end = min(ci + pst, cn);
        crow0 = (cb * a.num_q_heads + ch * G) * a.max_parts + cpart;
      } else if (ci == cseg_end) {  // next run of the slice
        if (++cb == a.num_seqs) { cb = 0; ++ch; }
        clen = clamp_len(lens[cb], a.max_len);
        cn = steps_of_len(clen);
        ci = 0;
        cseg_start = 0;
        cseg_end = (int)min((int64_t)cn, left);
        cflags_run = (cseg_end == cn) ? kFinal : 0;
        crow0 = (r * 2 + 1) * G;
        if (cseg_end < cn) rec = merge_rec_of(sp, r, g_end - left, cn, cb, ch, 1);
        if constexpr (MERGE) pieces[1] = CutPiece{g_end - left, cn, cb, ch, true};
      }
      sl.base = ci * kStepTokens;
      sl.t1 = min(min(cseg_end * kStepTokens, clen), a.cap_len);
      sl.b = cb;
      sl.h = ch;
      sl.flags = cflags_run | (ci == cseg_start ? kFirst : 0) | (ci + 1 == cseg_end ? kLast : 0);
      sl.row0 = crow0;
      // physical blocks of the step (an empty run reads block 0, all masked)
      const int lb0 = sl.base / BS;
      const int lb_last = sl.t1 > 0 ? (sl.t1 - 1) / BS : 0;
      const int64_t row = (int64_t)cb * a.max_blocks;
      int p0 = sl.t1 > sl.base ? tables[row + lb0] : 0;
      int p1 = (C::kBlocksPerStep == 2 && lb0 + 1 <= lb_last) ? tables[row + lb0 + 1] : p0;
      // the run's newest token (position clen - 1) in this step, in a block
      // the table names (else the append writes nothing, as a slot outside
      // the pool)
      const int np = clen - 1;
      const int pn = (np / BS == lb0) ? p0 : p1;
      const bool newest = APPEND && ci + 1 == cn && clen > 0 && np < a.cap_len && pn >= 0 &&
                          (int64_t)pn < a.num_blocks;
      p0 = (p0 < 0 || (int64_t)p0 >= a.num_blocks) ? 0 : p0;
      p1 = (p1 < 0 || (int64_t)p1 >= a.num_blocks) ? 0 : p1;
      tile0 = ((int64_t)p0 * a.num_kv_heads + ch) * C::kTile;
      tile1 = ((int64_t)p1 * a.num_kv_heads + ch) * C::kTile;
      if constexpr (APPEND) {
        if (newest) {
          sl.nw.pos = np - sl.base;
          sl.nw.off = np % BS;
          sl.nw.tile = ((int64_t)pn * a.num_kv_heads + ch) * C::kTile;
          const size_t nrow = ((size_t)cb * a.num_kv_heads + ch) * D;
          const __bf16* kn = reinterpret_cast<const __bf16*>(a.k_new) + nrow;
          const uint16_t* vn = reinterpret_cast<const uint16_t*>(a.v_new) + nrow;
#pragma unroll
          for (int c = 0; c < C::kChunks; ++c)
            sl.nw.k[c] = *reinterpret_cast<const u32x4*>(kn + q_dim<CK, D>(grp, c));
#pragma unroll
          for (int dt = 0; dt < C::kDTiles; ++dt) sl.nw.v[dt] = vn[dt * 16 + col];
        }
      }
      qp = qbase + ((size_t)cb * a.num_q_heads + (size_t)ch * G + qhead) * D;
      ++ci;
      if (!pst) --left;
      ++pending;
    }
    if constexpr (PK) load_step_pk(sl, kc, vc, tile0, tile1, plo);
    else load_step(sl, kc, vc, tile0, tile1, lo, grp);
    if constexpr (!QSEG) {
#pragma unroll
      for (int c = 0; c < C::kChunks; ++c)
        sl.q[c] = *reinterpret_cast<const bf16x8*>(qp + q_dim<CK, D>(grp, c));
    }
  };
  // per segment: the query of the segment whose first step computes next,
  // loaded before the ring's next issue, and used at once (INT4: its operand
  // bias), so that the wait it takes covers only the loads already in flight
  // and no later step waits for it again
  float qbias = 0.f;
  auto load_q = [&](const S& sl) {
    const __bf16* p = qbase + ((size_t)sl.b * a.num_q_heads + (size_t)sl.h * G + qhead) * D;
    if constexpr (PK) {
      const bf16x8 zero = {};
#pragma unroll
      for (int i = 0; i < kQOps; ++i) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(p + pk_q_dim<D>(grp, i));
        qseg[i] = pk_on ? v : zero;
      }
    } else {
#pragma unroll
      for (int c = 0; c < (QSEG ? C::kChunks : 0); ++c)
        qseg[c] = *reinterpret_cast<const bf16x8*>(p + q_dim<CK, D>(grp, c));
    }
    if constexpr (QSEG) {
      static_assert(!QSEG || C::I4, "a per-segment query must be used where it is loaded");
      qbias = q_bias<kQOps>(qseg);
    }
  };

  // ---- finished segments ----------------------------------------------------
  // A finished segment's G output rows (and, for a cut run, its maxima and
  // sums) wait in LDS and are written after the ring has drained, or when
  // the buffer is full.  A wavefront's memory operations retire in order, so
  // a global store issued while the ring's loads are in flight holds up
  // every younger load until the write completes: a bubble of about one
  // memory latency per finished segment (measured on MI355X: ~4 us each,
  // 17 us of 284 on the 70B-shaped batch).  The G rows are contiguous in
  // out and in the workspace, so they leave as 16-byte stores over all
  // lanes.  Rows are padded by 4 floats so the G writing lanes hit
  // different banks.
  constexpr int kStageRow = D + 4;
  // LDS per wavefront: 16 KiB at eight per CU, 37 KiB at four (four such
  // workgroups, tags and appended-row staging included, stay within the
  // CU's 160 KiB; a slice of 16 fixed partitions at G = 4, head_dim 128,
  // then never flushes mid-stream), 32 KiB at two.
  constexpr int kWaves = stream_waves_per_cu<CK, D>();
  constexpr int kOutFloats = (kWaves >= 8 ? 16384 : (kWaves >= 4 ? 37888 : 32768)) / 4;
  constexpr int kOutSlotsMax = 32;
  __shared__ __attribute__((aligned(16))) float outbuf[kOutFloats];
  __shared__ int outtag[kOutSlotsMax];  // out row of the group's head 0 (final), or -1 - row0 (state)
  const int slot_floats = (G * kStageRow + 2 * G + 3) & ~3;
  const int out_cap = min(kOutSlotsMax, kOutFloats / slot_floats);
  int nout = 0;

  auto flush = [&]() {
    __builtin_amdgcn_wave_barrier();  // the slots were written by other lanes of this wavefront
    for (int sidx = 0; sidx < nout; ++sidx) {
      const int tag = __builtin_amdgcn_readfirstlane(outtag[sidx]);
      const float* src = outbuf + sidx * slot_floats;
      if (tag >= 0) {
        __bf16* o = reinterpret_cast<__bf16*>(a.out) + (size_t)tag * D;
        for (int q = lane; q < G * (D / 8); q += 64) {  // 8 outputs per 16-byte store
          const float* e = src + (q / (D / 8)) * kStageRow + (q % (D / 8)) * 8;
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(e);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(e + 4);
          bf16x8 y;
#pragma unroll
          for (int i = 0; i < 4; ++i) { y[i] = (__bf16)x0[i]; y[4 + i] = (__bf16)x1[i]; }
          *reinterpret_cast<bf16x8*>(o + (size_t)q * 8) = y;
        }
      } else {
        const int row0 = -1 - tag;  // head g of the group at row row0 + g * rstride
        if constexpr (MERGE) {  // merged in this launch, maybe on another XCD: device-scope stores
          float* o = a.part_out + (size_t)row0 * D;
          for (int q = lane; q < G * D; q += 64)
            state_store(o + q, src[(q / D) * kStageRow + q % D], true);
        } else {
          for (int q = lane; q < G * (D / 4); q += 64) {
            const int g = q / (D / 4);
            *reinterpret_cast<f32x4*>(a.part_out + ((size_t)row0 + (size_t)g * rstride) * D +
                                      (q % (D / 4)) * 4) =
                *reinterpret_cast<const f32x4*>(src + g * kStageRow + (q % (D / 4)) * 4);
          }
        }
        if (lane < G) {
          const size_t rl = (size_t)row0 + (size_t)lane * rstride;
          state_store(a.part_max + rl, src[G * kStageRow + lane], MERGE);
          state_store(a.part_sum + rl, src[G * kStageRow + G + lane], MERGE);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();  // reads done before the slots are reused
    nout = 0;
  };

  // ---- appended rows --------------------------------------------------------
  // A newest token's K and V rows wait in LDS, with their tile and offset,
  // and are written after the ring has drained (or when the buffer fills).
  constexpr int kAppMax = APPEND ? 8 : 1;
  __shared__ __attribute__((aligned(16))) uint32_t appk[kAppMax][D / 2];  // K row, bf16 pairs
  __shared__ uint16_t appv[kAppMax][D];                                    // V row
  __shared__ int64_t apptile[kAppMax];
  __shared__ int appoff[kAppMax];
  int napp = 0;
  char* const kw = reinterpret_cast<char*>(a.k_pool_w);  // set when APPEND
  char* const vw = reinterpret_cast<char*>(a.v_pool_w);

  auto flush_app = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_wave_barrier();  // the rows were staged by other lanes of this wavefront
    for (int i = 0; i < napp; ++i) {
      const int64_t tile = apptile[i];
      const int off = appoff[i];
      // K: D/8 pieces of 16 bytes, piece r (dimensions 8r .. 8r + 7) in chunk row r
      if (lane < D / 8)
        *reinterpret_cast<u32x4*>(kw + tile + ((int64_t)lane * BS + off) * 16) =
            *reinterpret_cast<const u32x4*>(&appk[i][lane * 4]);
      // V: dimension d in row d of the dimension-major tile
      for (int d = lane; d < D; d += 64)
        *reinterpret_cast<uint16_t*>(vw + tile + ((int64_t)d * BS + off) * 2) = appv[i][d];
    }
    __builtin_amdgcn_wave_barrier();  // reads done before the rows are reused
    napp = 0;
  };

  // ---- compute side ---------------------------------------------------------
  f32x4 acc[C::kDTiles];
  f32x4 accb = {0.f, 0.f, 0.f, 0.f};  // INT4: column sums of the PV weights
  LaneSoftmax st;
  float c2 = 0.f;

  auto compute = [&](S& sl) {
    const bf16x8* qop;
    if constexpr (QSEG) qop = qseg;
    else qop = sl.q;
    if constexpr (APPEND) {
      // The newest token's rows replace the pool's bytes in the step's
      // registers (K: lanes of its QK row; V: element pos % 8 of the lanes
      // of its k-slot group) and are staged for the write.
      const int tn = sl.nw.pos;
      if (tn >= 0) {
        // value selects on both token groups: a store through a chosen
        // group index would put the ring in scratch memory
        const bool row0 = col == (tn & 15) && tn < 16;
        const bool row1 = col == (tn & 15) && tn >= 16;
#pragma unroll
        for (int c = 0; c < C::kChunks; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sl.k[0][c][e] = row0 ? sl.nw.k[c][e] : sl.k[0][c][e];
            sl.k[1][c][e] = row1 ? sl.nw.k[c][e] : sl.k[1][c][e];
          }
        if (grp == (tn >> 3)) {
          const int wi = (tn & 7) >> 1;
          const int sh = (tn & 1) * 16;
#pragma unroll
          for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (i == wi) sl.v[dt].w[i] = (sl.v[dt].w[i] & ~(0xffffu << sh)) | (sl.nw.v[dt] << sh);
        }
        if (napp == kAppMax) flush_app();  // rare: many runs end in one slice
        if (col == 0) {
#pragma unroll
          for (int c = 0; c < C::kChunks; ++c)
            *reinterpret_cast<u32x4*>(&appk[napp][q_dim<CK, D>(grp, c) / 2]) = sl.nw.k[c];
        }
        if (grp == 0) {
#pragma unroll
          for (int dt = 0; dt < C::kDTiles; ++dt) appv[napp][dt * 16 + col] = (uint16_t)sl.nw.v[dt];
        }
        if (lane == 0) {
          apptile[napp] = sl.nw.tile;
          appoff[napp] = sl.nw.off;
        }
        ++napp;
      }
    }
    if (sl.flags & kFirst) {
#pragma unroll
      for (int dt = 0; dt < C::kDTiles; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      accb = f32x4{0.f, 0.f, 0.f, 0.f};
      float kscale = 1.0f;
      if constexpr (FP8) kscale = ((const_f32)a.k_scale)[sl.h];
      c2 = log2_factor(a.scale, kscale);
      st.reset(c2);
      if constexpr (C::I4 && !QSEG) qbias = q_bias<C::kChunks>(qop);
    }
    const bool partial = sl.base + kStepTokens > sl.t1;
    bf16x8 pop;
    if constexpr (PK) {
      // two accumulation chains over the D/16 words of the lane's K row
      f32x4 s0 = qk_init<CK>(qbias), s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < kQOps; i += 2) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand_pk(sl, i), qop[i], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand_pk(sl, i + 1), qop[i + 1], s1, 0, 0, 0);
      }
      float z[4] = {s0[0] + s1[0], s0[1] + s1[1], s0[2] + s1[2], s0[3] + s1[3]};
      // partial step: score j (token pk_score_token + j) in range iff j <= zlim
      const int zlim = sl.t1 - sl.base - 1 - pk_score_token(grp, col);
      pop = softmax_step_pk<C::kDTiles>(z, partial, zlim, sl, c2, st, acc, accb, pk_on);
    } else {
      f32x4 s0 = qk_init<CK>(qbias), s1 = s0;
#pragma unroll
      for (int c = 0; c < C::kChunks; ++c) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<CK>(sl, 0, c), qop[c], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<CK>(sl, 1, c), qop[c], s1, 0, 0, 0);
      }
      float z[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
      qk_scores<CK>(z, sl);
      const int n = sl.t1 - sl.base;
      const int zlim = n - 1 - 4 * grp;  // partial step: offsets <= zlim in range
      if (partial) {
        const int vvalid = min(max(n - 8 * grp, 0), 8);
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt) mask_v<CK>(sl.v[dt], vvalid);
      }
      pop = softmax_step<CK, C::kDTiles>(z, partial, zlim, sl, c2, st, acc, accb);
    }
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt)
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v_operand<CK>(sl.v[dt]), pop, acc[dt], 0, 0, 0);
    if constexpr (C::I4) accb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_operand(), pop, accb, 0, 0, 0);

    if (sl.flags & kLast) {
      lazy_settle<C::kDTiles, PK>(st, c2, acc, accb);
      float l_tot = xlane<OpSum, 16, 32>(st.l_run);
      if constexpr (PK) {  // columns c and c ^ 8 hold the two token halves of a head
        l_tot = pk_fold(l_tot);
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[dt][r] = pk_fold(acc[dt][r]);
        accb[0] = pk_fold(accb[0]);
      }
      float vscale = 1.0f;
      if constexpr (FP8) vscale = ((const_f32)a.v_scale)[sl.h];
      const float inv = l_tot > 0.f ? vscale / l_tot : 0.f;  // an empty run writes zeros
      if constexpr (C::I4) {  // remove the operand bias: 136 * sum_t p(t) s_v(t)
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[dt][r] = fmaf(-kI4Bias, accb[0], acc[dt][r]);
      }
      if (nout == out_cap) flush();  // rare: many short runs in one slice
      float* dst = outbuf + nout * slot_floats;
      if (col < G) {
        float* row = dst + col * kStageRow;
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt)
          *reinterpret_cast<f32x4*>(row + dt * 16 + grp * 4) = acc[dt] * inv;
        if (!(sl.flags & kFinal) && grp == 0) {
          dst[G * kStageRow + col] = st.m_run * (c2 * kLn2);  // natural units: scale * q.k
          dst[G * kStageRow + G + col] = l_tot;
        }
      }
      if (lane == 0)
        outtag[nout] = (sl.flags & kFinal) ? sl.b * a.num_q_heads + sl.h * G : -1 - sl.row0;
      ++nout;
    }
  };

  // ---- the ring ------------------------------------------------------------
  S ring[kRing];
#pragma unroll
  for (int j = 0; j < kRing - 1; ++j) issue(ring[j]);
  while (pending > 0) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      if (QSEG && ring[j].real && (ring[j].flags & kFirst)) load_q(ring[j]);
      issue(ring[(j + kRing - 1) % kRing]);
      if (ring[j].real) {
        compute(ring[j]);
        --pending;
      }
    }
  }
  flush();
  if constexpr (APPEND) flush_app();
  if (pst) return;
  if (lane == 0) store_merge_rec(a.header, r, rec);
  if constexpr (MERGE) {  // cut runs merged in this launch by the wavefront finishing last
    const MergeView v{a.out, a.part_out, a.part_max, a.part_sum, a.num_q_heads, G};
    arrive_and_merge<__bf16, D>(v, a.counters, sp, pieces);
  }
}

template <int CK, int D, int BS>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  if (a.k_new) {  // the decode appends the newest tokens itself (bf16, balanced split)
    if constexpr (CK == kBF16) {
      if (a.partition != kAuto || a.counters) return hipErrorInvalidValue;
      DecodeArgs b = a;
      b.slices = a.cus * launch_waves_per_cu<CK, D>(a);
      hipLaunchKernelGGL((decode_mfma_stream<CK, D, BS, true, false, false>), dim3(b.slices), dim3(64), 0, stream, b);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (a.partition == kAuto || (a.partition > 0 && a.stream_fixed)) {
    DecodeArgs b = a;
    b.slices = a.cus * launch_waves_per_cu<CK, D>(a);
    if (a.partition > 0) {
      if constexpr (CK != kI4)  // INT4 fixed partitions take the grid (host side)
        hipLaunchKernelGGL((decode_mfma_stream<CK, D, BS, false, false, true>), dim3(b.slices), dim3(64), 0, stream, b);
      else
        return hipErrorInvalidValue;
    } else if (CK == kI4 && a.group <= 8) {  // column-packed INT4 steps
      if (a.counters)
        hipLaunchKernelGGL((decode_mfma_stream<CK, D, BS, false, true, false, CK == kI4>), dim3(b.slices), dim3(64), 0, stream, b);
      else
        hipLaunchKernelGGL((decode_mfma_stream<CK, D, BS, false, false, false, CK == kI4>), dim3(b.slices), dim3(64), 0, stream, b);
    } else if (a.counters)
      hipLaunchKernelGGL((decode_mfma_stream<CK, D, BS, false, true, false>), dim3(b.slices), dim3(64), 0, stream, b);
    else
      hipLaunchKernelGGL((decode_mfma_stream<CK, D, BS, false, false, false>), dim3(b.slices), dim3(64), 0, stream, b);
  } else {
    const int parts = a.partition ? a.max_parts : 1;
    dim3 grid(parts, a.num_kv_heads, a.num_seqs);
    hipLaunchKernelGGL((decode_mfma_grid<CK, D, BS>), grid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

template <int CK>
hipError_t dispatch_shape(const DecodeArgs& a, int head_dim, int block_size, hipStream_t s) {
  if (head_dim == 128 && block_size == 16) return launch<CK, 128, 16>(a, s);
  if (head_dim == 128 && block_size == 32) return launch<CK, 128, 32>(a, s);
  if (head_dim == 64 && block_size == 16) return launch<CK, 64, 16>(a, s);
  if (head_dim == 64 && block_size == 32) return launch<CK, 64, 32>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, Elem cache, int head_dim, int block_size,
                              hipStream_t stream) {
  if (cache == Elem::BF16) return dispatch_shape<kBF16>(a, head_dim, block_size, stream);
  if (cache == Elem::FP8) return dispatch_shape<kE4M3>(a, head_dim, block_size, stream);
  if (cache == Elem::E5M2) return dispatch_shape<kE5M2>(a, head_dim, block_size, stream);
  if (cache == Elem::I4) return dispatch_shape<kI4>(a, head_dim, block_size, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
