// Streaming read of a device buffer: the measurement helper behind mtpd_stream_read (not a step of the method).
// It gives the read rate the part sustains for a plain sweep, the denominator beside the 8 TB/s HBM peak, and one
// pass over a buffer much larger than the 4 MB L2 of each XCD plus the 256 MB memory-side cache evicts both with
// clean lines before a cold measurement.
//
// Layout: block b takes 32 KB chunks b, b + grid, b + 2 grid, ... (consecutive chunks go to consecutive blocks and
// so to different XCDs); in a chunk every thread issues its eight 16-byte loads before using any, so a CU holding
// eight such blocks has 256 KB of reads in flight. The loaded words are folded by xor and the result is stored only
// when it equals a key the caller passes (in practice never), which keeps the loads alive without write traffic.
#include "kernels.h"

namespace mtpd {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;
constexpr uint64_t kStreamChunk = (uint64_t)kStreamThreads * kStreamUnroll;  // 16-byte vectors per chunk

__global__ __launch_bounds__(kStreamThreads) void k_stream_read(const uint4* __restrict__ p, uint64_t n16,
                                                                 uint32_t key, uint32_t* __restrict__ sink) {
  uint4 acc = make_uint4(0u, 0u, 0u, 0u);
  for (uint64_t base = (uint64_t)blockIdx.x * kStreamChunk; base < n16; base += (uint64_t)gridDim.x * kStreamChunk) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const uint64_t i = base + (uint64_t)u * kStreamThreads + threadIdx.x;
      v[u] = i < n16 ? p[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      acc.x ^= v[u].x;
      acc.y ^= v[u].y;
      acc.z ^= v[u].z;
      acc.w ^= v[u].w;
    }
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == key) sink[0] = acc.x;
}

}  // namespace

hipError_t launch_stream_read(hipStream_t s, const void* buf, uint64_t bytes, uint32_t key, uint32_t* sink) {
  const uint64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const uint64_t chunks = (n16 + kStreamChunk - 1) / kStreamChunk;
  // eight blocks per CU on the 256 CUs, fewer for small buffers
  const unsigned grid = (unsigned)(chunks < 2048 ? chunks : 2048);
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(kStreamThreads), 0, s, static_cast<const uint4*>(buf), n16, key,
                     sink);
  return hipGetLastError();
}

}  // namespace mtpd
