// A plain streaming read of a device buffer: the attainable HBM read
// bandwidth of this GPU for a kernel that does nothing but read, measured in
// the same process as the decode so that the decode's achieved bandwidth
// can be stated against it as well as against the published peak.
//
// Every workgroup reads one contiguous share of the buffer, 4 KiB per
// instruction across its 256 lanes (16 bytes each, non-temporal, like the
// decode's tile loads), eight such loads in flight per lane.
#include "pa_device.hpp"
#include "pa_internal.hpp"
#include "pa_measure.h"

namespace pa {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;
constexpr int kReadGroupsPerCU = 8;
constexpr uint32_t kSinkKey = 0x9E3779B9u;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* src, int64_t n16,
                                                                   uint32_t* sink) {
  const int64_t share = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t begin = (int64_t)blockIdx.x * share;
  const int64_t end = begin + share < n16 ? begin + share : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = begin + threadIdx.x;
  for (; i + (int64_t)(kReadUnroll - 1) * kReadThreads < end; i += (int64_t)kReadUnroll * kReadThreads) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = stream_load<u32x4>(src + i + u * kReadThreads);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  for (; i < end; i += kReadThreads) acc ^= stream_load<u32x4>(src + i);
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == kSinkKey) *sink = x;
}

}  // namespace
}  // namespace pa

extern "C" pa_status pa_stream_read(const void* src, size_t bytes, uint32_t* sink,
                                    hipStream_t stream) {
  if (bytes == 0) return PA_OK;
  if (!src || !sink || (reinterpret_cast<uintptr_t>(src) & 15) || (bytes & 15))
    return PA_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return PA_ERR_HIP;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t groups = std::min<int64_t>((int64_t)cus * pa::kReadGroupsPerCU,
                                           (n16 + pa::kReadThreads - 1) / pa::kReadThreads);
  hipLaunchKernelGGL(pa::stream_read_kernel, dim3((unsigned)groups), dim3(pa::kReadThreads), 0,
                     stream, static_cast<const pa::u32x4*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
