// Merge of a cut run's partial softmax states (balanced split).
//
// A run (sequence b, KV head h) that slice boundaries cut leaves one state
// per slice holding a piece of it: slices r_first .. r_first + nparts - 1,
// piece 0 in state slot k_first of slice r_first, every later piece in slot 0
// of its slice (rows ((2 * slice + slot) * G + g) of the workspace).  A state
// is the piece's maximum score m, its exp-sum l relative to m and its
// normalised output o; with M the largest m, piece j weighs
// w_j = l_j * exp(m_j - M) and the output is sum_j w_j * o_j / sum_j w_j:
// every piece's exp terms put on the common scale, i.e. softmax over the
// whole run.
//
// merge_cut_run is the one routine both merges use -- the separate merge
// launch (pa_decode_reduce) and the merge inside the decode launch -- so a
// run's output bits do not depend on which of them ran.  Per query head:
// the maximum and weight sum are cross-lane reductions with piece j on lane
// j, and the rows are accumulated in piece order with fused multiply-adds.
#pragma once

#include <type_traits>

#include "pa_device.hpp"
#include "pa_internal.hpp"
#include "pa_split.hpp"

namespace pa {

// merge_cut_run's paths for runs of up to 64 pieces: NH query heads at a
// time, their pieces' rows in rounds of NP -- runs of at most 4 pieces 8
// heads and one round of rows, longer ones (a run cut by the dynamic tail's
// small chunks) 4 heads and rounds of 16 pieces.
constexpr int kMergeFastPieces = 4;
constexpr int kMergeFastHeads = 8;
constexpr int kMergeMidPieces = 16;
constexpr int kMergeMidHeads = 4;

// Partial states that a wavefront of the same launch may read from another
// XCD (the merge inside the decode launch) are stored and loaded at device
// scope: each access is coherent at the device level by itself (written
// through, or read past, the non-coherent per-XCD caches), so neither side
// needs an agent-scope fence, which on gfx950 writes back or invalidates the
// whole L2 of its XCD (measured on MI355X: ~20 us more per 8B-shaped decode
// launch with a release fence per wavefront and an acquire per merge).
__device__ __forceinline__ void state_store(float* p, float v, bool device_scope) {
  if (device_scope) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool DEVICE_SCOPE>
__device__ __forceinline__ float state_load(const float* p) {
  if constexpr (DEVICE_SCOPE)
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}

struct MergeView {
  void* out;               // [S][Hq][D] output rows
  const float* part_out;   // workspace state rows
  const float* part_max;
  const float* part_sum;
  int num_q_heads, group;
};

// Query heads gq0, gq0 + gq_step, ... of the cut run, by one wavefront.
// DEVICE_SCOPE: the states were stored by this launch (state_store).
template <typename OT, int D, bool DEVICE_SCOPE>
__device__ __forceinline__ void merge_cut_run(const MergeView& v, int b, int h, int r_first,
                                              int k_first, int nparts, int gq0, int gq_step) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int G = v.group;
  auto row_of = [&](int j, int gq) -> size_t {  // piece j of the run, in slice order
    const int rr = r_first + j;
    return ((size_t)rr * 2 + (j == 0 ? k_first : 0)) * G + gq;
  };
  auto emit = [&](int gq, const float* acc, float total) {
    OT* o = reinterpret_cast<OT*>(v.out) + ((size_t)b * v.num_q_heads + (size_t)h * G + gq) * D;
    const float inv = 1.0f / total;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[lane + 64 * e] = (OT)(acc[e] * inv);
  };

  // Runs of up to 64 pieces, NH query heads at a time: the pieces' maxima
  // and exp-sums in one round (piece j on lane j), then the rows in rounds
  // of NP pieces, accumulated in piece order with the weights on those
  // lanes; every head's arithmetic is the general path's, in the same order.
  auto merge_heads = [&](auto np_tag, auto nh_tag) {
    constexpr int NP = decltype(np_tag)::value;
    constexpr int NH = decltype(nh_tag)::value;
    const bool mine = lane < nparts;
    for (int gb = gq0; gb < G; gb += gq_step * NH) {
      float w[NH], acc[NH][PER];
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        const int gq = min(gb + i * gq_step, G - 1);
        const size_t rl = row_of(mine ? lane : 0, gq);
        const float pm = state_load<DEVICE_SCOPE>(v.part_max + rl);
        const float ps = state_load<DEVICE_SCOPE>(v.part_sum + rl);
        const float mx = xlane<OpMax, 1, 32>(mine ? pm : -INFINITY);
        w[i] = mine ? ps * __expf(pm - mx) : 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[i][e] = 0.f;
      }
      for (int j0 = 0; j0 < nparts; j0 += NP) {
        float rows[NH][NP][PER];
#pragma unroll
        for (int i = 0; i < NH; ++i) {
          const int gq = min(gb + i * gq_step, G - 1);
#pragma unroll
          for (int j = 0; j < NP; ++j) {
            const float* src = v.part_out + row_of(min(j0 + j, nparts - 1), gq) * D + lane;
#pragma unroll
            for (int e = 0; e < PER; ++e) rows[i][j][e] = state_load<DEVICE_SCOPE>(src + 64 * e);
          }
        }
#pragma unroll
        for (int i = 0; i < NH; ++i) {
#pragma unroll
          for (int j = 0; j < NP; ++j) {
            if (j0 + j < nparts) {
              const float wj = __int_as_float(readlane(__float_as_int(w[i]), j0 + j));
#pragma unroll
              for (int e = 0; e < PER; ++e) acc[i][e] = fmaf(wj, rows[i][j][e], acc[i][e]);
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        const int gq = gb + i * gq_step;
        if (gq < G) emit(gq, acc[i], xlane<OpSum, 1, 32>(w[i]));
      }
    }
  };
  if (nparts <= kMergeFastPieces) {  // the usual cut: 2 or 3 pieces, one round of rows
    merge_heads(std::integral_constant<int, kMergeFastPieces>{}, std::integral_constant<int, kMergeFastHeads>{});
    return;
  }
  if (nparts <= 64) {
    merge_heads(std::integral_constant<int, kMergeMidPieces>{}, std::integral_constant<int, kMergeMidHeads>{});
    return;
  }

  for (int gq = gq0; gq < G; gq += gq_step) {
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float wsum;
    {
      // more than 64 pieces: lanes take the pieces' maxima and exp-sums in
      // parallel
      float mx = -INFINITY;
      for (int j = lane; j < nparts; j += 64)
        mx = fmaxf(mx, state_load<DEVICE_SCOPE>(v.part_max + row_of(j, gq)));
      mx = xlane<OpMax, 1, 32>(mx);
      wsum = 0.f;
      for (int j0 = 0; j0 < nparts; j0 += 64) {
        const int j = j0 + lane;
        const size_t row = row_of(j < nparts ? j : j0, gq);
        const float w = j < nparts ? state_load<DEVICE_SCOPE>(v.part_sum + row) *
                                         __expf(state_load<DEVICE_SCOPE>(v.part_max + row) - mx)
                                   : 0.f;
        wsum += w;
        const int cnt = min(64, nparts - j0);
        for (int jj = 0; jj < cnt; ++jj) {
          const float wj = __int_as_float(readlane(__float_as_int(w), jj));
          const float* src = v.part_out + row_of(j0 + jj, gq) * D + lane;
#pragma unroll
          for (int e = 0; e < PER; ++e) acc[e] = fmaf(wj, state_load<DEVICE_SCOPE>(src + 64 * e), acc[e]);
        }
      }
    }
    emit(gq, acc, xlane<OpSum, 1, 32>(wsum));
  }
}

// Merge inside the decode launch.  A cut run's pieces finish on different
// wavefronts (on any XCD); each wavefront, once its own states are stored,
// counts itself in on the run's counter (indexed by the slice holding piece
// 0), and the one whose arrival completes the count merges the run and
// clears the counter for the next launch.  The states are device-scope
// stores (state_store), and the wavefront waits until all of its stores
// are complete before it counts itself in, so a piece's states are visible
// device-wide before its arrival can be seen; the merging wavefront reads
// them with device-scope loads issued after the count returned.
//
// A piece is described by the run's first step gs and step count n in the
// balanced plan; pieces of uncut runs are ignored.  Up to two pieces per
// call (a slice's first and last runs): their arrivals are issued together.
struct CutPiece {
  int64_t gs;
  int n, b, h;
  bool valid;
};

template <typename OT, int D>
__device__ __forceinline__ void arrive_and_merge(const MergeView& v, int* counters, const Split& sp,
                                                 const CutPiece (&pc)[2]) {
  const int lane = threadIdx.x & 63;
  int r_first[2], nparts[2];
  bool cut[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    cut[i] = false;
    r_first[i] = 0;
    nparts[i] = 0;
    if (pc[i].valid) {
      r_first[i] = slice_of_step(sp, pc[i].gs);
      nparts[i] = slice_of_step(sp, pc[i].gs + pc[i].n - 1) - r_first[i] + 1;
      cut[i] = nparts[i] >= 2;
    }
  }
  if (!cut[0] && !cut[1]) return;
  // every memory operation of this wavefront (its state stores) complete
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int old0 = 0, old1 = 0;
  if (lane == 0) {
    if (cut[0]) old0 = __hip_atomic_fetch_add(counters + r_first[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (cut[1]) old1 = __hip_atomic_fetch_add(counters + r_first[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  old0 = readlane(old0, 0);
  old1 = readlane(old1, 0);
  const bool last0 = cut[0] && old0 == nparts[0] - 1;
  const bool last1 = cut[1] && old1 == nparts[1] - 1;
  if (!last0 && !last1) return;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (!(i == 0 ? last0 : last1)) continue;
    const int k_first = pc[i].gs == (int64_t)r_first[i] * sp.per ? 0 : 1;
    merge_cut_run<OT, D, true>(v, pc[i].b, pc[i].h, r_first[i], k_first, nparts[i], 0, 1);
    if (lane == 0) __hip_atomic_store(counters + r_first[i], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace pa
