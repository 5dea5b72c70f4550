// Measurement aid: a plain streaming read of a device buffer, the attainable
// HBM read rate on this device against which the layer's weight stream is
// compared (the layer's own figures stay against the 8 TB/s peak).
//
// Each workgroup reads whole 32 KiB chunks of the buffer, grid-stride: eight
// non-temporal 16-byte loads per lane, each a contiguous 4 KiB of the chunk
// (1 KiB runs per wave), all in flight before the first is used.  What it
// read is folded into one word per workgroup so that no load is dead.
#include "moe_common.h"

namespace moe {

constexpr int kCeilThreads = 256;
constexpr int kCeilUnroll = 8;

__global__ void __launch_bounds__(kCeilThreads)
stream_read_kernel(const u32x4* __restrict__ buf, size_t n16, uint32_t* __restrict__ sink) {
  constexpr size_t kChunk = (size_t)kCeilThreads * kCeilUnroll;   // 16-byte units per chunk
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t c = blockIdx.x; c * kChunk < n16; c += gridDim.x) {
    const size_t base = c * kChunk + threadIdx.x;
    if ((c + 1) * kChunk <= n16) {
      u32x4 v[kCeilUnroll];
#pragma unroll
      for (int u = 0; u < kCeilUnroll; u++) v[u] = __builtin_nontemporal_load(buf + base + u * kCeilThreads);
#pragma unroll
      for (int u = 0; u < kCeilUnroll; u++) acc ^= v[u];
    } else {
      for (size_t i = base; i < n16; i += kCeilThreads) acc ^= __builtin_nontemporal_load(buf + i);
    }
  }
  __shared__ uint32_t s[kCeilThreads];
  s[threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < kCeilThreads; t++) r ^= s[t];
    sink[blockIdx.x] = r;
  }
}

}  // namespace moe

namespace moe_host {

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int groups, hipStream_t s) {
  hipLaunchKernelGGL(moe::stream_read_kernel, dim3(groups), dim3(moe::kCeilThreads), 0, s,
                     static_cast<const moe::u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe_host
