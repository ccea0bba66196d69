// Whole-block copies inside the paged pools: the device half of
// copy-on-write.
//
// When a sequence is about to write into a block that other sequences also
// reference, the engine first gives it a private copy of that block and
// copies only that block ("AI Inference Serving at Scale", section 3,
// copy-on-write sharing; "vLLM & High-Throughput Serving", copy-on-write
// prefix caching: a shared block is cloned only when a sequence writes a
// divergent token).  The host side (reference counts, choosing the new
// block) decides the (src, dst) pairs; this kernel moves the bytes.
//
// The same kernel swaps blocks between the device pools and a pool in
// pinned host memory that the GPU addresses directly, for preemption ("How
// LLM Inference Engines Work", the scheduler's swap to CPU memory when the
// GPU is full): one launch moves any number of blocks over the host link.
//
// A block holds every KV head, so in both pools it is one contiguous run of
// num_kv_heads * block_size * head_dim elements.  Each workgroup copies one
// 4 KiB chunk of one pair's K or V block with one 16-byte non-temporal load
// and store per thread: the copy streams HBM at the load/store geometry the
// decode measured fastest, and nothing it moves is reread soon.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kChunkBytes = kCopyThreads * 16;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(const CopyArgs a) {
  const int64_t pair = blockIdx.x;
  const int pool = blockIdx.y;          // 0: K, 1: V
  const int64_t chunk = blockIdx.z;     // 4 KiB chunk of the block
  const int64_t src = a.mapping[2 * pair];
  const int64_t dst = a.mapping[2 * pair + 1];
  // ids outside the pools are skipped; the host validates what it can see
  if (src < 0 || src >= a.src_blocks || dst < 0 || dst >= a.dst_blocks) return;
  const char* from = static_cast<const char*>(pool == 0 ? a.src_k : a.src_v);
  char* to = static_cast<char*>(pool == 0 ? a.dst_k : a.dst_v);
  const int64_t off = chunk * kChunkBytes + (int64_t)threadIdx.x * 16;
  if (off >= a.block_bytes) return;  // a block is a multiple of 1 KiB, not always of 4 KiB
  const u32x4 v = stream_load<u32x4>(from + src * a.block_bytes + off);
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(to + dst * a.block_bytes + off));
}

}  // namespace

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
  const int64_t chunks = (a.block_bytes + kChunkBytes - 1) / kChunkBytes;
  if (a.block_bytes % 16 != 0 || chunks > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.num_pairs, 2, (unsigned)chunks);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
