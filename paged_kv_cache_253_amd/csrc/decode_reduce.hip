// Merge of partial softmax states into the output.
//
// A partial state of a token range holds its maximum score m, its exp-sum l
// (taken relative to m) and its normalised output o.  With M the largest m
// of a (sequence, query head), range p weighs w_p = l_p * exp(m_p - M) and
// the output is sum_p w_p * o_p / sum_p w_p: each range's exp terms are put
// on the common scale, so the result is softmax over the union of ranges.
// Every merge below adds its ranges in a fixed order (deterministic bits).
//
//  * reduce_kernel: fixed partitions.  One 256-thread workgroup per
//    (sequence, query head); 16-byte loads, D/4 threads per partition row,
//    256/(D/4) rows in flight; the row groups are summed in order at the end.
//  * auto_fixup_kernel: balanced slices.  One workgroup per slice; the
//    slice's merge record (written by the decode, see pa_split.hpp) names
//    the cut run whose first piece it holds, if any, and the workgroup
//    merges all of that run's slice states (merge_cut_run in pa_merge.hpp,
//    the routine the decode kernels use when they merge in their own
//    launch), all of its query heads by one wavefront.
#include "pa_device.hpp"
#include "pa_internal.hpp"
#include "pa_merge.hpp"
#include "pa_split.hpp"

namespace pa {
namespace {

constexpr int kReduceThreads = 256;
constexpr int kWeightChunk = 1024;

template <class Op>
__device__ __forceinline__ float block_combine(float x, float* scratch) {
  x = xlane<Op, 1, 32>(x);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[wave] = x;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int i = 1; i < kReduceThreads / 64; ++i) r = Op::f(r, scratch[i]);
  return r;
}

// MQ: several query tokens per sequence; output row = query token
// query_start[b] + i (grid z = i), whose context is the tokens up to its
// position, L_b - Q_b + i.
template <typename OT, int D, bool MQ>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(const ReduceArgs a) {
  constexpr int TPR = D / 4;                    // threads per partition row
  constexpr int ROWS = kReduceThreads / TPR;    // rows in flight
  __shared__ float wbuf[kWeightChunk];
  __shared__ float part[ROWS][D];
  __shared__ float scratch[kReduceThreads / 64];

  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  int len = clamp_len(a.context_lens[b], a.max_len);
  size_t qrow = b;
  if constexpr (MQ) {
    const int i = blockIdx.z;
    const int r0 = a.query_start[b];
    const int nq = a.query_start[b + 1] - r0;
    if (i >= nq) return;
    qrow = (size_t)(r0 + i);
    len = max(min(len - nq + i + 1, len), 0);
  }
  const int n = (len + a.partition - 1) / a.partition;
  OT* o = reinterpret_cast<OT*>(a.out) + (qrow * a.num_q_heads + hq) * D;
  if (n == 0) {
    if (tid < D) o[tid] = (OT)0.0f;
    return;
  }
  const size_t base = (qrow * a.num_q_heads + hq) * a.max_parts;
  float mx = -INFINITY;
  for (int p = tid; p < n; p += kReduceThreads) mx = fmaxf(mx, a.part_max[base + p]);
  mx = block_combine<OpMax>(mx, scratch);

  const int row = tid / TPR;
  const int q4 = tid % TPR;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int c0 = 0; c0 < n; c0 += kWeightChunk) {
    const int cn = min(kWeightChunk, n - c0);
    for (int p = tid; p < cn; p += kReduceThreads) {
      const float w = a.part_sum[base + c0 + p] * __expf(a.part_max[base + c0 + p] - mx);
      wbuf[p] = w;
      wsum += w;
    }
    __syncthreads();
    const float* src = a.part_out + (base + c0) * D + q4 * 4;
#pragma unroll 4
    for (int p = row; p < cn; p += ROWS)
      acc += wbuf[p] * *reinterpret_cast<const f32x4*>(src + (size_t)p * D);
    __syncthreads();
  }
  const float total = block_combine<OpSum>(wsum, scratch);
  *reinterpret_cast<f32x4*>(&part[row][q4 * 4]) = acc;
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) s += part[r][tid];
    o[tid] = (OT)(s / total);
  }
}

// One wavefront per slice: merge_cut_run loads up to eight heads' states
// per round, and most slices have no cut run to merge (the grid covers the
// most slices a decode can use).
constexpr int kFixupThreads = 64;

template <typename OT, int D>
__global__ __launch_bounds__(kFixupThreads) void auto_fixup_kernel(const ReduceArgs a) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const int r_first = blockIdx.x;  // slice holding the run's first piece
  const int slices = a.header[kHdrSlices];  // as launched by the decode
  const i32x4 rec = *reinterpret_cast<const i32x4*>(reinterpret_cast<const char*>(a.header) +
                                                     kHdrRecordsBytes + (size_t)r_first * kMergeRecordBytes);
  if (r_first >= slices || slices > a.slices_max) return;
  const int b = rec[0], h = rec[1], nparts = rec[2], k_first = rec[3];
  if (nparts < 2) return;  // slice r_first's last run is not cut
  // a workspace no decode has filled must not send the merge out of bounds
  if (nparts > slices - r_first || (unsigned)b >= (unsigned)a.num_seqs ||
      (unsigned)h >= (unsigned)a.num_kv_heads || (unsigned)k_first > 1u)
    return;
  const MergeView v{a.out, a.part_out, a.part_max, a.part_sum, a.num_q_heads,
                    a.num_q_heads / a.num_kv_heads};
  merge_cut_run<OT, D, false>(v, b, h, r_first, k_first, nparts, 0, 1);
}

template <typename OT, int D>
hipError_t launch(const ReduceArgs& a, hipStream_t s) {
  if (a.query_start) {
    if (a.max_query_len < 1) return hipSuccess;
    dim3 grid(a.num_q_heads, a.num_seqs, a.max_query_len);
    hipLaunchKernelGGL((reduce_kernel<OT, D, true>), grid, dim3(kReduceThreads), 0, s, a);
  } else {
    dim3 grid(a.num_q_heads, a.num_seqs);
    hipLaunchKernelGGL((reduce_kernel<OT, D, false>), grid, dim3(kReduceThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <typename OT, int D>
hipError_t launch_fixup(const ReduceArgs& a, hipStream_t s) {
  if (a.slices_max < 2) return hipSuccess;
  hipLaunchKernelGGL((auto_fixup_kernel<OT, D>), dim3(a.slices_max), dim3(kFixupThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, Elem out, int head_dim, hipStream_t stream) {
  if (out == Elem::BF16 && head_dim == 128) return launch<__bf16, 128>(a, stream);
  if (out == Elem::BF16 && head_dim == 64) return launch<__bf16, 64>(a, stream);
  if (out == Elem::F32 && head_dim == 128) return launch<float, 128>(a, stream);
  if (out == Elem::F32 && head_dim == 64) return launch<float, 64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_auto_fixup(const ReduceArgs& a, Elem out, int head_dim, hipStream_t stream) {
  if (out == Elem::BF16 && head_dim == 128) return launch_fixup<__bf16, 128>(a, stream);
  if (out == Elem::BF16 && head_dim == 64) return launch_fixup<__bf16, 64>(a, stream);
  if (out == Elem::F32 && head_dim == 128) return launch_fixup<float, 128>(a, stream);
  if (out == Elem::F32 && head_dim == 64) return launch_fixup<float, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
