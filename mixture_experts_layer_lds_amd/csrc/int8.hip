// int8 w8a8 activation quantisation (SGLang tuning guide: the int8_w8a8
// dtype with per-channel quantisation).  Symmetric per-row rule, the fp8
// rule with 127 for 448: scale = fp32(amax/127), inv = fp32(127/amax)
// (divisions in fp64), code = clamp(round_half_even(fp32(v * inv)),
// -127, 127); an all-zero row gets scale 1 and codes 0.
#include "moe_common.h"
#include "decode_route.h"

namespace moe {

constexpr int kI8Threads = 256;

__device__ __forceinline__ void i8_row_scales(float amax, float* scale, float* inv) {
  if (amax > 0.0f) {
    *scale = (float)((double)amax / 127.0);
    *inv = (float)(127.0 / (double)amax);
  } else {
    *scale = 1.0f;
    *inv = 1.0f;
  }
}

// four fp32 values (already multiplied by inv) -> four int8 codes in a dword
__device__ __forceinline__ uint32_t f32x4_to_i8x4(float a, float b, float c, float d) {
  const float v[4] = {a, b, c, d};
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float r = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(v[i]), -127.0f), 127.0f);
    w |= ((uint32_t)(int)r & 0xffu) << (8 * i);
  }
  return w;
}

__device__ __forceinline__ float block_max_i8(float v, float* s_red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = __builtin_fmaxf(__builtin_fmaxf(s_red[0], s_red[1]), __builtin_fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  return r;
}

// x[T][H] bf16 -> xq[T][H] int8 + scale[T]; one workgroup per token.  Also
// clears the row-amax slots zero_rows[t*zk ..) of the token's pairs and
// writes its scale at the sorted row of each of its zk pairs.
// ROUTE (at most 64 pairs): the launch also does the routing build, and the
// sorted rows of each token's zk pairs come from there.
template <bool ROUTE>
__global__ void __launch_bounds__(kI8Threads)
quant_rows_i8_kernel(const uint16_t* __restrict__ x, int H, int8_t* __restrict__ xq,
                     float* __restrict__ scale, float* __restrict__ zero_rows, int zk,
                     const int32_t* __restrict__ pair_pos, float* __restrict__ scale_rows,
                     moe_host::DecodeRouteOut route) {
  __shared__ float s_red[4];
  const int t = blockIdx.x;
  int row_j = 0;   // ROUTE: the sorted row of pair t * zk + lane (lanes < zk)
  if constexpr (ROUTE) {
    const int P = gridDim.x * zk;
    const int lane = threadIdx.x & 63;
    const DecodeRoute rt = decode_route(route.ids, P, route.E, route.block_m, lane);
    if (t == 0) decode_route_write(rt, route, P, threadIdx.x, kI8Threads, lane, threadIdx.x >> 6);
    row_j = __shfl(rt.pos, min(t * zk + lane, P - 1), kWave);
  }
  if (zero_rows && threadIdx.x < zk) zero_rows[(size_t)t * zk + threadIdx.x] = 0.0f;
  const u32x4* row = reinterpret_cast<const u32x4*>(x + (size_t)t * H);
  const int nvec = H / 8;
  float amax = 0.0f;
  for (int i = threadIdx.x; i < nvec; i += kI8Threads) {
    const u32x4 v = row[i];
#pragma unroll
    for (int w = 0; w < 4; w++) {
      amax = __builtin_fmaxf(amax, __builtin_fabsf(bf16_bits_to_f32(v[w] & 0xffffu)));
      amax = __builtin_fmaxf(amax, __builtin_fabsf(bf16_bits_to_f32(v[w] >> 16)));
    }
  }
  amax = block_max_i8(amax, s_red);
  float sc, inv;
  i8_row_scales(amax, &sc, &inv);
  u32x2* out = reinterpret_cast<u32x2*>(xq + (size_t)t * H);
  for (int i = threadIdx.x; i < nvec; i += kI8Threads) {
    const u32x4 v = row[i];
    float f[8];
#pragma unroll
    for (int w = 0; w < 4; w++) {
      f[2 * w] = __fmul_rn(bf16_bits_to_f32(v[w] & 0xffffu), inv);
      f[2 * w + 1] = __fmul_rn(bf16_bits_to_f32(v[w] >> 16), inv);
    }
    u32x2 q;
    q.x = f32x4_to_i8x4(f[0], f[1], f[2], f[3]);
    q.y = f32x4_to_i8x4(f[4], f[5], f[6], f[7]);
    out[i] = q;
  }
  if (threadIdx.x == 0) scale[t] = sc;
  if (scale_rows && threadIdx.x < zk)   // wave 0: lane j holds pair j of the token
    scale_rows[ROUTE ? row_j : pair_pos[(size_t)t * zk + threadIdx.x]] = sc;
}

// fp32 rows h32[r][0..I) of the valid sorted rows -> int8 codes, with the
// row amax found here from the row (h_scale[r] then holds the row scale).
__global__ void __launch_bounds__(kI8Threads)
requant_rows_i8_kernel(const float* __restrict__ h32, int I, const int32_t* __restrict__ expert_offsets,
                       int E, int8_t* __restrict__ hq, float* __restrict__ h_scale) {
  const int r = blockIdx.x;
  if (r >= expert_offsets[E]) return;
  const float amax = row_amax_f32<kI8Threads>(h32 + (size_t)r * I, I);
  float sc, inv;
  i8_row_scales(amax, &sc, &inv);
  const f32x4* row = reinterpret_cast<const f32x4*>(h32 + (size_t)r * I);
  uint32_t* q = reinterpret_cast<uint32_t*>(hq + (size_t)r * I);
  for (int i = threadIdx.x; i < I / 4; i += kI8Threads) {
    const f32x4 v = row[i];
    q[i] = f32x4_to_i8x4(__fmul_rn(v[0], inv), __fmul_rn(v[1], inv), __fmul_rn(v[2], inv),
                         __fmul_rn(v[3], inv));
  }
  if (threadIdx.x == 0) h_scale[r] = sc;
}

}  // namespace moe

namespace moe_host {

hipError_t launch_quant_rows_i8(const uint16_t* x, int T, int H, int8_t* xq, float* scale,
                                float* zero_rows, int zk, const int32_t* pair_pos, float* scale_rows,
                                hipStream_t s, const DecodeRouteOut* route) {
  if (route && ((long)T * zk > moe::kDecodeRoutePairs || !route->ids)) return hipErrorInvalidValue;
  const DecodeRouteOut ro = route ? *route : DecodeRouteOut{};
  if (route)
    hipLaunchKernelGGL(moe::quant_rows_i8_kernel<true>, dim3(T), dim3(moe::kI8Threads), 0, s, x, H, xq, scale,
                       zero_rows, zk, pair_pos, scale_rows, ro);
  else
    hipLaunchKernelGGL(moe::quant_rows_i8_kernel<false>, dim3(T), dim3(moe::kI8Threads), 0, s, x, H, xq, scale,
                       zero_rows, zk, pair_pos, scale_rows, ro);
  return hipGetLastError();
}

hipError_t launch_requant_rows_i8(const float* h32, int P, int I, const int32_t* expert_offsets, int E,
                                  int8_t* hq, float* h_scale, hipStream_t s) {
  hipLaunchKernelGGL(moe::requant_rows_i8_kernel, dim3(P), dim3(moe::kI8Threads), 0, s, h32, I,
                     expert_offsets, E, hq, h_scale);
  return hipGetLastError();
}

}  // namespace moe_host
