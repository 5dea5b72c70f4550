// Measurement aid: a plain streaming read of a device buffer, the attainable
// HBM read rate on this device against which the layer's weight stream is
// compared (the layer's own figures stay against the 8 TB/s peak).
//
// Each workgroup reads whole 32 KiB chunks of the buffer, grid-stride: eight
// non-temporal 16-byte loads per lane, each a contiguous 4 KiB of the chunk
// (1 KiB runs per wave), all in flight before the first is used.  What it
// read is folded into one word per workgroup so that no load is dead.
#include "lds_dma.h"

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

// Token-tile copies into LDS, as the LDS-staged GEMMs issue them, with no
// arithmetic: one workgroup of 8 waves per CU; the workgroups of one XCD
// (blockIdx % 8) in groups of 16, each group copying the same tile of
// kTileRows rows x row_bytes (the strips of one task tile side by side),
// reps times over, all K steps of all 16-row blocks, 8 copy instructions
// per wave per round and two rounds in flight.  Patterns of one 1 KiB copy:
//   0: 1 KiB contiguous (lane l: bytes 16 l), the packed-weight pattern;
//   1: 16 rows x one 64-byte K step, lane l: row l % 16, piece l / 16 (MFMA
//      lane order);
//   2: the same 16 x 64 bytes, lane l: row l / 4, piece (l % 4) ^ tok_swz
//      (the token-chunk layout of the GEMMs).
constexpr int kTileRows = 160;
constexpr int kCopyGroup = 16;

template <int PATTERN>
__global__ void __launch_bounds__(512, 1)
tile_copy_kernel(const char* __restrict__ buf, int row_bytes, int reps, int groups_per_xcd,
                 uint32_t* __restrict__ sink) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int group = xcd * groups_per_xcd + min(slot / kCopyGroup, groups_per_xcd - 1);
  const char* tile = buf + (size_t)group * kTileRows * row_bytes;
  char* mine = lds + wave * 8192;
  const int nsteps = row_bytes / 64;
  const int rounds = kTileRows / 16 * nsteps / 64;   // 64 chunks per round (8 waves x 8)
  for (int r = 0; r < reps; r++) {
    for (int j = 0; j < rounds; j++) {
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const int c = j * 64 + wave * 8 + u;    // chunk: K step c / 10, row block c % 10
        const char* src;
        if constexpr (PATTERN == 0) {
          src = tile + (size_t)c * 1024 + 16 * lane;
        } else {
          const int st = c / (kTileRows / 16), rb = c % (kTileRows / 16);
          const int row = PATTERN == 1 ? (lane & 15) : tok_copy_row(lane);
          const int piece = PATTERN == 1 ? (lane >> 4) : tok_copy_piece(lane);
          src = tile + (size_t)(rb * 16 + row) * row_bytes + st * 64 + 16 * piece;
        }
        dma16(src, mine + u * 1024);
      }
      wait_vm<8>();
    }
  }
  wait_vm<0>();
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = reinterpret_cast<const uint32_t*>(lds)[wave];
}

}  // namespace moe

namespace moe_host {

size_t tile_copy_bytes(int cus, int row_bytes) {
  return (size_t)(cus / 8 / moe::kCopyGroup) * 8 * moe::kTileRows * row_bytes;
}

hipError_t launch_tile_copy(int pattern, const void* buf, int row_bytes, int reps, uint32_t* sink, int cus,
                            hipStream_t s) {
  constexpr int kLds = 96 * 1024;   // one workgroup per CU
  const int gpx = cus / 8 / moe::kCopyGroup;
  const char* b = static_cast<const char*>(buf);
#define MOE_TC(Pv)                                                                                    \
  {                                                                                                   \
    static bool set = false;                                                                          \
    if (!set) {                                                                                       \
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&moe::tile_copy_kernel<Pv>), \
                                               hipFuncAttributeMaxDynamicSharedMemorySize, kLds);      \
      if (e != hipSuccess) return e;                                                                  \
      set = true;                                                                                     \
    }                                                                                                 \
    hipLaunchKernelGGL((moe::tile_copy_kernel<Pv>), dim3(cus), dim3(512), kLds, s, b, row_bytes, reps, gpx, \
                       sink);                                                                         \
    break;                                                                                            \
  }
  switch (pattern) {
    case 0: MOE_TC(0)
    case 1: MOE_TC(1)
    case 2: MOE_TC(2)
    default: return hipErrorInvalidValue;
  }
#undef MOE_TC
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int groups, hipStream_t s) {
  hipLaunchKernelGGL(moe::stream_read_kernel, dim3(groups), dim3(moe::kCeilThreads), 0, s,
                     static_cast<const moe::u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe_host
