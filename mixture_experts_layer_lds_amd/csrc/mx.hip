// MXFP8 activation quantisation (SGLang tuning guide, block shapes: gfx95
// devices keep MXFP8's [1, 32] blocks).  OCP Microscaling: every 32
// consecutive values of a row share one e8m0 scale 2^s,
//   s = floor(log2(max |v|)) - 8  (8 = the largest e4m3 exponent),
// clamped to [-127, 127] (an all-zero block, or one whose max is below
// 2^-126, takes -127), and hold e4m3 codes of v * 2^-s, rounded to nearest
// even and saturated to +-448.  v * 2^-s is exact in fp32: 2^-s is a normal
// power of two and |v * 2^-s| < 512.
//
// One thread per 32-value block: the block's values arrive in a few 16-byte
// loads, its 32 codes leave in two 16-byte stores and its scale code in one
// byte; consecutive threads take consecutive blocks of a row.
#include "moe_common.h"
#include "decode_route.h"

namespace moe {

constexpr int kMxThreads = 256;

__device__ __forceinline__ int mx_shared_exp(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu);   // biased exponent, sign cleared by the caller
  return e == 0 ? -127 : max(e - 127 - 8, -127);
}

// codes of 32 values with the block exponent s, as 8 dwords
__device__ __forceinline__ void mx_encode32(const float (&v)[32], int s, u32x4& lo, u32x4& hi) {
  const float mul = __uint_as_float((uint32_t)(127 - s) << 23);   // 2^-s, s in [-127, 119]
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; i++)
    w[i] = f32x4_to_e4m3x4_sat(v[4 * i] * mul, v[4 * i + 1] * mul, v[4 * i + 2] * mul,
                               v[4 * i + 3] * mul);
  lo = u32x4{w[0], w[1], w[2], w[3]};
  hi = u32x4{w[4], w[5], w[6], w[7]};
}

// ROUTE (at most 64 pairs): workgroup 0 also does the routing build (the
// x codes do not depend on the routing).
template <bool ROUTE>
__global__ void __launch_bounds__(kMxThreads)
mx_quant_bf16_kernel(const uint16_t* __restrict__ x, long nblocks, uint8_t* __restrict__ xq,
                     uint8_t* __restrict__ sx, moe_host::DecodeRouteOut route, int P) {
  if constexpr (ROUTE) {
    if (blockIdx.x == 0) {
      const int lane = threadIdx.x & 63;
      const DecodeRoute rt = decode_route(route.ids, P, route.E, route.block_m, lane);
      decode_route_write(rt, route, P, threadIdx.x, kMxThreads, lane, threadIdx.x >> 6);
    }
  }
  const long blk = (long)blockIdx.x * kMxThreads + threadIdx.x;
  if (blk >= nblocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + blk * 32);
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const u32x4 q = src[i];
#pragma unroll
    for (int w = 0; w < 4; w++) {
      v[8 * i + 2 * w] = bf16_bits_to_f32(q[w] & 0xffffu);
      v[8 * i + 2 * w + 1] = bf16_bits_to_f32(q[w] >> 16);
    }
  }
#pragma unroll
  for (int i = 0; i < 32; i++) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  const int s = mx_shared_exp(amax);
  u32x4 lo, hi;
  mx_encode32(v, s, lo, hi);
  u32x4* dst = reinterpret_cast<u32x4*>(xq + blk * 32);
  dst[0] = lo;
  dst[1] = hi;
  sx[blk] = (uint8_t)(s + 127);
}

// fp32 rows [P][I] -> codes [P][I] + scale codes [P][I/32], rows below
// expert_offsets[E] (the valid sorted rows).
__global__ void __launch_bounds__(kMxThreads)
mx_requant_kernel(const float* __restrict__ h, int I, const int32_t* __restrict__ expert_offsets,
                  int E, uint8_t* __restrict__ hq, uint8_t* __restrict__ sh) {
  const long blk = (long)blockIdx.x * kMxThreads + threadIdx.x;
  const int per_row = I / 32;
  if (blk >= (long)expert_offsets[E] * per_row) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(h + blk * 32);
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const f32x4 q = src[i];
#pragma unroll
    for (int w = 0; w < 4; w++) v[4 * i + w] = q[w];
  }
#pragma unroll
  for (int i = 0; i < 32; i++) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  const int s = mx_shared_exp(amax);
  u32x4 lo, hi;
  mx_encode32(v, s, lo, hi);
  u32x4* dst = reinterpret_cast<u32x4*>(hq + blk * 32);
  dst[0] = lo;
  dst[1] = hi;
  sh[blk] = (uint8_t)(s + 127);
}

}  // namespace moe

namespace moe_host {

hipError_t launch_mx_quant_bf16(const uint16_t* x, int T, int H, uint8_t* xq, uint8_t* sx, hipStream_t s,
                                const DecodeRouteOut* route, int P) {
  if (route && (P > moe::kDecodeRoutePairs || !route->ids)) return hipErrorInvalidValue;
  const long n = (long)T * (H / 32);
  const dim3 grid((unsigned)((n + moe::kMxThreads - 1) / moe::kMxThreads));
  const DecodeRouteOut ro = route ? *route : DecodeRouteOut{};
  if (route)
    hipLaunchKernelGGL(moe::mx_quant_bf16_kernel<true>, grid, dim3(moe::kMxThreads), 0, s, x, n, xq, sx, ro, P);
  else
    hipLaunchKernelGGL(moe::mx_quant_bf16_kernel<false>, grid, dim3(moe::kMxThreads), 0, s, x, n, xq, sx, ro, P);
  return hipGetLastError();
}

hipError_t launch_mx_requant(const float* h, int P, int I, const int32_t* expert_offsets, int E,
                             uint8_t* hq, uint8_t* sh, hipStream_t s) {
  const long n = (long)P * (I / 32);
  hipLaunchKernelGGL(moe::mx_requant_kernel, dim3((unsigned)((n + moe::kMxThreads - 1) / moe::kMxThreads)),
                     dim3(moe::kMxThreads), 0, s, h, I, expert_offsets, E, hq, sh);
  return hipGetLastError();
}

}  // namespace moe_host
