// Merge of a split decode's partition states into the output.
//
// One wavefront per (sequence, query head).  With M the largest partition
// maximum, partition p carries weight w_p = sum_p * exp(max_p - M); the
// output is sum_p w_p * out_p / sum_p w_p.  Each partition's exp terms were
// taken relative to its own maximum, so the rescale by exp(max_p - M) puts
// all of them on one scale and the result is softmax over the whole context.
// Partitions are added in increasing p, so the result is deterministic.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

template <typename OT, int D>
__global__ __launch_bounds__(64) void reduce_kernel(const ReduceArgs a) {
  constexpr int PER = D / 64;
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  int len = a.context_lens[b];
  len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
  const int n = (len + a.partition - 1) / a.partition;
  OT* o = reinterpret_cast<OT*>(a.out) + ((size_t)b * a.num_q_heads + hq) * D;
  if (n == 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) o[lane + 64 * e] = (OT)0.0f;
    return;
  }
  const size_t base = ((size_t)b * a.num_q_heads + hq) * a.max_parts;
  float mx = -INFINITY;
  for (int p = lane; p < n; p += 64) mx = fmaxf(mx, a.part_max[base + p]);
  mx = xlane<OpMax, 1, 32>(mx);

  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  for (int p0 = 0; p0 < n; p0 += 64) {
    const int p = p0 + lane;
    const float w = (p < n) ? a.part_sum[base + p] * __expf(a.part_max[base + p] - mx) : 0.f;
    wsum += w;
    const int cnt = min(64, n - p0);
    const float* row = a.part_out + (base + p0) * D + lane;
    for (int j = 0; j < cnt; ++j) {
      const float wj = __int_as_float(readlane(__float_as_int(w), j));
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(wj, row[(size_t)j * D + 64 * e], acc[e]);
    }
  }
  const float total = xlane<OpSum, 1, 32>(wsum);
  const float inv = 1.0f / total;
#pragma unroll
  for (int e = 0; e < PER; ++e) o[lane + 64 * e] = (OT)(acc[e] * inv);
}

template <typename OT, int D>
hipError_t launch(const ReduceArgs& a, hipStream_t s) {
  dim3 grid(a.num_q_heads, a.num_seqs);
  hipLaunchKernelGGL((reduce_kernel<OT, D>), grid, dim3(64), 0, s, a);
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

}  // namespace pa
