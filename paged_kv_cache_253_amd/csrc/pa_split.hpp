// Work split shared by the decode kernels and the merge kernels.
//
// Two ways to cut a batch's contexts into per-wavefront ranges:
//
//  * Fixed partitions (flash decoding): range p of (sequence b, KV head h)
//    covers tokens [p*P, min((p+1)*P, L_b)); one wavefront per range.
//  * Balanced ("auto"): every (b, h) is a run of 32-token steps
//    (ceil(L_b / 32), at least 1 so an empty context still has its zero
//    output written); the runs are laid end to end, KV head major, and a
//    persistent grid of W wavefronts takes W equal consecutive slices.  A
//    (b, h) that one slice covers whole is finished by that wavefront; one
//    that straddles a slice boundary leaves a partial softmax state per
//    slice, merged afterwards.  Each slice has at most two such states: its
//    first run ("head", slot 0) and its last run ("tail", slot 1).  The
//    wavefront that holds a cut run's first piece leaves a merge record
//    for it, so the merge needs neither the plan nor a search.
//  * Fixed partitions on the persistent grid: the same plan counted in
//    whole partitions instead of steps (a run of L tokens has ceil(L / P)
//    of them, none when L = 0), so no partition is cut and every one
//    leaves its state in its own workspace row.
#pragma once

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

constexpr int kStepTokens = 32;

__device__ __forceinline__ int clamp_len(int len, int max_len) {
  return len < 0 ? 0 : (len > max_len ? max_len : len);
}

__device__ __forceinline__ int steps_of_len(int len) {
  return len <= 0 ? 1 : (len + kStepTokens - 1) / kStepTokens;
}

// Work units of a run of len tokens: 32-token steps (pst == 0, balanced
// split) or partitions of pst steps.
__device__ __forceinline__ int units_of_len(int len, int pst) {
  if (pst == 0) return steps_of_len(len);
  const int part = pst * kStepTokens;
  return len <= 0 ? 0 : (len + part - 1) / part;
}

// Inclusive prefix sum over the 64 lanes of the wavefront.
__device__ __forceinline__ int wave_scan_incl(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

struct Split {
  int64_t per_head;  // units (steps, or partitions) of one KV head over the whole batch
  int64_t total;     // units of the batch (all KV heads)
  int64_t per;       // units per slice
  int slices;        // persistent wavefronts W
};

// Every wavefront computes the same plan from the lengths (no device-wide
// communication).  A balanced slice is at least kAutoMinSteps steps, so
// small batches use fewer wavefronts instead of many tiny slices.
__device__ __forceinline__ Split plan_split(const int32_t* lens, int num_seqs, int max_len,
                                            int num_kv_heads, int slices, int pst = 0) {
  const int lane = threadIdx.x & 63;
  int64_t tot = 0;
  for (int c = 0; c < num_seqs; c += 64) {
    const int b = c + lane;
    const int n = b < num_seqs ? units_of_len(clamp_len(lens[b], max_len), pst) : 0;
    tot += readlane(wave_scan_incl(n), 63);
  }
  Split s;
  s.per_head = tot;
  s.total = tot * num_kv_heads;
  s.slices = slices;
  const int64_t even = (s.total + slices - 1) / slices;
  const int64_t least = pst ? 1 : kAutoMinSteps;
  s.per = even > least ? even : least;
  return s;
}

// Steps [g0, g1) of slice c (empty for slices past the batch).
__device__ __forceinline__ void slice_bounds(const Split& s, int c, int64_t& g0, int64_t& g1) {
  g0 = (int64_t)c * s.per;
  g1 = g0 + s.per;
  if (g1 > s.total) g1 = s.total;
  if (g0 > g1) g0 = g1;
}

// Slice holding step g (0 <= g < total).
__device__ __forceinline__ int slice_of_step(const Split& s, int64_t g) { return (int)(g / s.per); }

// Sequence b and unit offset i of unit `rem` (0 <= rem < per_head) of a head.
__device__ __forceinline__ void locate_step(const int32_t* lens, int num_seqs, int max_len,
                                            int64_t rem, int& b_out, int& i_out, int pst = 0) {
  const int lane = threadIdx.x & 63;
  int64_t base = 0;
  for (int c = 0; c < num_seqs; c += 64) {
    const int b = c + lane;
    const int n = b < num_seqs ? units_of_len(clamp_len(lens[b], max_len), pst) : 0;
    const int incl = wave_scan_incl(n);
    const int chunk = readlane(incl, 63);
    if (rem < base + chunk) {
      const uint64_t hit = __builtin_amdgcn_ballot_w64(base + incl > rem);
      const int l = __builtin_ctzll(hit);
      b_out = c + l;
      i_out = (int)(rem - (base + readlane(incl, l) - readlane(n, l)));
      return;
    }
    base += chunk;
  }
  b_out = num_seqs - 1;  // not reached for rem < per_head
  i_out = 0;
}

// Merge record of slice r: the run whose first piece is slice r's last
// segment, when a later slice boundary cuts it -- sequence, KV head, the
// number of slices holding a piece (pieces j >= 1 are the first runs of
// slices r + j), and the state slot of piece 0 in slice r (0 when the run
// is also the slice's first run, else 1).  nparts = 0: no such run.  Every
// wavefront of a balanced launch writes its record, so none survives from
// an earlier launch.
struct MergeRec {
  int b, h, nparts, slot;
};

__device__ __forceinline__ void store_merge_rec(int* header, int r, const MergeRec& m) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 v = {m.b, m.h, m.nparts, m.slot};
  *reinterpret_cast<i32x4*>(reinterpret_cast<char*>(header) + kHdrRecordsBytes +
                            (size_t)r * kMergeRecordBytes) = v;
}

// Record of the run that starts at step gs (its first piece in slice r,
// state slot `slot`) and has n steps, if it runs past slice r.
__device__ __forceinline__ MergeRec merge_rec_of(const Split& s, int r, int64_t gs, int n, int b,
                                                 int h, int slot) {
  const int last = slice_of_step(s, gs + n - 1);
  if (last == r) return MergeRec{0, 0, 0, 0};
  return MergeRec{b, h, last - r + 1, slot};
}

// Slice of wavefront w: slices handled by one XCD (workgroups are dealt to
// the XCDs round-robin) are consecutive, so neighbouring work -- e.g.
// sequences sharing prefix blocks -- meets in one L2.
__device__ __forceinline__ int slice_of_wave(int w, int slices) {
  if (slices % kXcds != 0) return w;
  return (w % kXcds) * (slices / kXcds) + w / kXcds;
}

}  // namespace pa
