// Row-wise stages of the fused MoE layer: per-token FP8 quantisation of the
// hidden states, SiLU-and-mul (+ FP8 requantisation) of the gate-up
// output, and the top-k weighted reduction back to token order
// (HPC-Ops x SGLang blog, section "MoE": gate-up & activation; PDL chaining
// paragraph for the final reduction).
//
// All three are HBM-bound streaming kernels: 16-byte vector loads along the
// contiguous dimension, one workgroup per row, no LDS beyond a 4-wave
// max-reduction.
#include "moe_common.h"
#include "decode_route.h"

namespace moe {

constexpr int kRowThreads = 256;

__device__ __forceinline__ float block_max_256(float v, float* s_red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  float r = __builtin_fmaxf(__builtin_fmaxf(s_red[0], s_red[1]), __builtin_fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  return r;
}

__device__ __forceinline__ float amax8_bf16(const u32x4& v, float amax) {
#pragma unroll
  for (int w = 0; w < 4; w++) {
    amax = __builtin_fmaxf(amax, __builtin_fabsf(bf16_bits_to_f32(v[w] & 0xffffu)));
    amax = __builtin_fmaxf(amax, __builtin_fabsf(bf16_bits_to_f32(v[w] >> 16)));
  }
  return amax;
}

__device__ __forceinline__ u32x2 quant8_bf16(const u32x4& v, float inv) {
  float f[8];
#pragma unroll
  for (int w = 0; w < 4; w++) {
    f[2 * w] = __fmul_rn(bf16_bits_to_f32(v[w] & 0xffffu), inv);
    f[2 * w + 1] = __fmul_rn(bf16_bits_to_f32(v[w] >> 16), inv);
  }
  u32x2 q;
  q.x = f32x4_to_e4m3x4_sat(f[0], f[1], f[2], f[3]);
  q.y = f32x4_to_e4m3x4_sat(f[4], f[5], f[6], f[7]);
  return q;
}

// x[T][H] bf16 -> xq[T][H] e4m3 + scale[T]; H % 8 == 0.  With scale_rows,
// the token's scale is also written at the sorted row of each of its zk pairs.
// NV > 0: the row is read once into registers (H <= NV * 8 * 256), found
// its amax and quantised from there; NV == 0: read twice (any H).
// ROUTE (at most 64 pairs): the launch also does the routing build, and the
// sorted rows of each token's zk pairs come from there.
template <int NV, bool ROUTE = false>
__global__ void __launch_bounds__(kRowThreads)
quant_rows_bf16_kernel(const uint16_t* __restrict__ x, int H, uint8_t* __restrict__ xq,
                       float* __restrict__ scale, float* __restrict__ zero_rows, int zk,
                       const int32_t* __restrict__ pair_pos, float* __restrict__ scale_rows,
                       moe_host::DecodeRouteOut route) {
  __shared__ float s_red[4];
  const int t = blockIdx.x;
  DecodeRoute rt{};
  int row_j = 0;   // ROUTE: the sorted row of pair t * zk + lane (lanes < zk)
  if constexpr (ROUTE) {
    const int P = gridDim.x * zk;
    const int lane = threadIdx.x & 63;
    rt = decode_route(route.ids, P, route.E, route.block_m, lane);
    if (t == 0) decode_route_write(rt, route, P, threadIdx.x, kRowThreads, lane, threadIdx.x >> 6);
    row_j = __shfl(rt.pos, min(t * zk + lane, P - 1), kWave);
  }
  if (zero_rows && threadIdx.x < zk) zero_rows[(size_t)t * zk + threadIdx.x] = 0.0f;
  const u32x4* row = reinterpret_cast<const u32x4*>(x + (size_t)t * H);
  u32x2* out = reinterpret_cast<u32x2*>(xq + (size_t)t * H);
  const int nvec = H / 8;
  float amax = 0.0f, sc, inv;
  if constexpr (NV > 0) {
    u32x4 v[NV];
#pragma unroll
    for (int j = 0; j < NV; j++) {
      const int i = threadIdx.x + j * kRowThreads;
      v[j] = i < nvec ? row[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < NV; j++) amax = amax8_bf16(v[j], amax);
    amax = block_max_256(amax, s_red);
    e4m3_row_scales(amax, &sc, &inv);
#pragma unroll
    for (int j = 0; j < NV; j++) {
      const int i = threadIdx.x + j * kRowThreads;
      if (i < nvec) out[i] = quant8_bf16(v[j], inv);
    }
  } else {
    for (int i = threadIdx.x; i < nvec; i += kRowThreads) amax = amax8_bf16(row[i], amax);
    amax = block_max_256(amax, s_red);
    e4m3_row_scales(amax, &sc, &inv);
    for (int i = threadIdx.x; i < nvec; i += kRowThreads) out[i] = quant8_bf16(row[i], inv);
  }
  if (threadIdx.x == 0) scale[t] = sc;
  if (scale_rows && threadIdx.x < zk)   // wave 0: lane j holds pair j
    scale_rows[ROUTE ? row_j : pair_pos[(size_t)t * zk + threadIdx.x]] = sc;
}

// h[r][n] = SiLU(rs * sum_s g[s][r][n]) * (rs * sum_s g[s][r][I + n]) for the
// valid sorted rows r < expert_offsets[E]; rs is the row's activation scale
// when the partial sums carry only the weight scales, else 1.
__device__ __forceinline__ f32x4 silu_mul4(const float* __restrict__ grow, size_t slice, int S,
                                           int I, int i, float rs) {
  f32x4 gs = *reinterpret_cast<const f32x4*>(grow + 4 * i);
  f32x4 us = *reinterpret_cast<const f32x4*>(grow + I + 4 * i);
  for (int s = 1; s < S; s++) {
    gs += *reinterpret_cast<const f32x4*>(grow + s * slice + 4 * i);
    us += *reinterpret_cast<const f32x4*>(grow + s * slice + I + 4 * i);
  }
  gs *= rs;
  us *= rs;
  f32x4 o;
#pragma unroll
  for (int w = 0; w < 4; w++) o[w] = silu_f32(gs[w]) * us[w];
  return o;
}

// bf16 path: grid (row, column chunk of kActCols); writes bf16 h.
constexpr int kActCols = 2048;

__global__ void __launch_bounds__(kRowThreads)
act_bf16_kernel(const float* __restrict__ g, int S, int P, int I,
                const int32_t* __restrict__ expert_offsets, int E, uint16_t* __restrict__ h) {
  const int r = blockIdx.x;
  if (r >= expert_offsets[E]) return;
  const size_t slice = (size_t)P * 2 * I;
  const float* grow = g + (size_t)r * 2 * I;
  uint16_t* hrow = h + (size_t)r * I;
  const int v0 = blockIdx.y * (kActCols / 4);
  const int v1 = min(I / 4, v0 + kActCols / 4);
#pragma unroll 2
  for (int i = v0 + threadIdx.x; i < v1; i += kRowThreads) {
    const f32x4 o = silu_mul4(grow, slice, S, I, i, 1.0f);
    u32x2 packed;
    packed.x = (uint32_t)f32_to_bf16_bits(o[0]) | ((uint32_t)f32_to_bf16_bits(o[1]) << 16);
    packed.y = (uint32_t)f32_to_bf16_bits(o[2]) | ((uint32_t)f32_to_bf16_bits(o[3]) << 16);
    *reinterpret_cast<u32x2*>(hrow + 4 * i) = packed;
  }
}

// fp8 path: one workgroup per row; the row is computed twice, first for its
// amax, then quantised with the per-row rule (e4m3 codes + fp32 scale).
__global__ void __launch_bounds__(kRowThreads)
act_fp8_kernel(const float* __restrict__ g, int S, int P, int I,
               const int32_t* __restrict__ expert_offsets, int E,
               const float* __restrict__ x_scale, const int32_t* __restrict__ sorted_pairs, int k,
               uint8_t* __restrict__ hq, float* __restrict__ h_scale) {
  __shared__ float s_red[4];
  const int r = blockIdx.x;
  if (r >= expert_offsets[E]) return;   // block-uniform
  const float rs = x_scale ? x_scale[sorted_pairs[r] / k] : 1.0f;
  const size_t slice = (size_t)P * 2 * I;
  const float* grow = g + (size_t)r * 2 * I;
  const int nvec = I / 4;
  float amax = 0.0f;
#pragma unroll 4
  for (int i = threadIdx.x; i < nvec; i += kRowThreads) {
    const f32x4 o = silu_mul4(grow, slice, S, I, i, rs);
#pragma unroll
    for (int w = 0; w < 4; w++) amax = __builtin_fmaxf(amax, __builtin_fabsf(o[w]));
  }
  amax = block_max_256(amax, s_red);
  float sc, inv;
  e4m3_row_scales(amax, &sc, &inv);
  uint32_t* qrow = reinterpret_cast<uint32_t*>(hq + (size_t)r * I);
#pragma unroll 4
  for (int i = threadIdx.x; i < nvec; i += kRowThreads) {
    const f32x4 o = silu_mul4(grow, slice, S, I, i, rs);
    qrow[i] = f32x4_to_e4m3x4_sat(__fmul_rn(o[0], inv), __fmul_rn(o[1], inv),
                                  __fmul_rn(o[2], inv), __fmul_rn(o[3], inv));
  }
  if (threadIdx.x == 0) h_scale[r] = sc;
}

// out[t][:] = bf16( sum_{j ascending, pair valid} w[t][j] * rs[pos] * sum_s y[s][pos][:] ),
// rs = row_scale (the fp8 activation scale of the row when y carries only
// the weight scales) or 1; each term is rounded once after its products and
// once after its sum (no fused multiply-add).
// y is fp32 [S][P][H] (4 columns per thread, 16-byte loads), or bf16 [P][H]
// when Y_BF16 (8 columns per thread, 16-byte loads).  Grid (token, column
// chunk of kRowThreads * columns-per-thread).
// Latency, not bandwidth, sets the time at small T: the token's KM (>= k)
// row indices and weights are workgroup-uniform scalar loads, then every
// row load is issued before the first is added (slots past k and dropped
// pairs read row 0, a valid address, and are skipped), so a call waits
// about one round trip for the rows instead of k.
template <bool Y_BF16, int KM>
__global__ void __launch_bounds__(kRowThreads)
reduce_kernel(const void* __restrict__ yv, int S, int P, const float* __restrict__ topk_w,
              const int32_t* __restrict__ pair_pos, const int32_t* __restrict__ expert_offsets,
              const float* __restrict__ row_scale, int E, int k, int H,
              uint16_t* __restrict__ out) {
#pragma clang fp contract(off)
  constexpr int C = Y_BF16 ? 8 : 4;
  const int t = blockIdx.x;
  const int c0 = (blockIdx.y * kRowThreads + threadIdx.x) * C;   // first column
  if (c0 >= H) return;
  const int valid = expert_offsets[E];
  const size_t slice = (size_t)P * H;
  bool ok[KM];
  size_t at[KM];   // element offset of the row's columns
  float w[KM], rs[KM];
#pragma unroll
  for (int j = 0; j < KM; j++) {
    const int jj = j < k ? j : k - 1;
    const int r = pair_pos[t * k + jj];
    w[j] = topk_w[t * k + jj];
    ok[j] = j < k && r < valid;   // dropped pairs are skipped
    at[j] = (size_t)(ok[j] ? r : 0) * H + c0;
    rs[j] = row_scale ? row_scale[ok[j] ? r : 0] : 1.0f;
  }
  f32x4 a[KM][C / 4];
  if constexpr (Y_BF16) {
    u32x4 raw[KM];
#pragma unroll
    for (int j = 0; j < KM; j++) raw[j] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(yv) + at[j]);
#pragma unroll
    for (int j = 0; j < KM; j++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        a[j][q / 2][2 * (q % 2)] = bf16_bits_to_f32(raw[j][q] & 0xffffu);
        a[j][q / 2][2 * (q % 2) + 1] = bf16_bits_to_f32(raw[j][q] >> 16);
      }
  } else {
    const float* y = static_cast<const float*>(yv);
#pragma unroll
    for (int j = 0; j < KM; j++) a[j][0] = *reinterpret_cast<const f32x4*>(y + at[j]);
    for (int s = 1; s < S; s++) {   // ascending slices, each slice's loads together
      f32x4 b[KM];
#pragma unroll
      for (int j = 0; j < KM; j++) b[j] = *reinterpret_cast<const f32x4*>(y + s * slice + at[j]);
#pragma unroll
      for (int j = 0; j < KM; j++) a[j][0] += b[j];
    }
  }
  float acc[C];
#pragma unroll
  for (int q = 0; q < C; q++) acc[q] = 0.0f;
#pragma unroll
  for (int j = 0; j < KM; j++) {
    if (!ok[j]) continue;
#pragma unroll
    for (int q = 0; q < C; q++) {
      float v = a[j][q / 4][q % 4];
      if (row_scale) v = v * rs[j];
      acc[q] = acc[q] + w[j] * v;
    }
  }
  uint32_t packed[C / 2];
#pragma unroll
  for (int q = 0; q < C / 2; q++)
    packed[q] = (uint32_t)f32_to_bf16_bits(acc[2 * q]) | ((uint32_t)f32_to_bf16_bits(acc[2 * q + 1]) << 16);
  uint16_t* o = out + (size_t)t * H + c0;
  if constexpr (Y_BF16) *reinterpret_cast<u32x4*>(o) = u32x4{packed[0], packed[1], packed[2], packed[3]};
  else *reinterpret_cast<u32x2*>(o) = u32x2{packed[0], packed[1]};
}

template <bool Y_BF16>
static void launch_reduce_t(dim3 grid, const void* y, int S, int P, const float* topk_w,
                            const int32_t* pair_pos, const int32_t* expert_offsets, const float* row_scale,
                            int E, int T, int k, int H, uint16_t* out, hipStream_t s) {
#define MOE_REDUCE_KM(KMv)                                                                              \
  hipLaunchKernelGGL((reduce_kernel<Y_BF16, KMv>), grid, dim3(kRowThreads), 0, s, y, S, P, topk_w,      \
                     pair_pos, expert_offsets, row_scale, E, k, H, out)
  if (k <= 2) MOE_REDUCE_KM(2);
  else if (k <= 4) MOE_REDUCE_KM(4);
  else if (k <= 8) MOE_REDUCE_KM(8);
  else MOE_REDUCE_KM(16);
#undef MOE_REDUCE_KM
}

}  // namespace moe

namespace moe_host {

hipError_t launch_quant_rows_bf16(const uint16_t* x, int T, int H, uint8_t* xq, float* scale,
                                  float* zero_rows, int zk, const int32_t* pair_pos,
                                  float* scale_rows, hipStream_t s, const DecodeRouteOut* route) {
  if (route && ((long)T * zk > moe::kDecodeRoutePairs || !route->ids)) return hipErrorInvalidValue;
  const int per = (H / 8 + moe::kRowThreads - 1) / moe::kRowThreads;   // 16-byte vectors per thread
  const DecodeRouteOut ro = route ? *route : DecodeRouteOut{};
#define MOE_QUANT_NV(NVv)                                                                                 \
  {                                                                                                       \
    if (route)                                                                                            \
      hipLaunchKernelGGL((moe::quant_rows_bf16_kernel<NVv, true>), dim3(T), dim3(moe::kRowThreads), 0, s, \
                         x, H, xq, scale, zero_rows, zk, pair_pos, scale_rows, ro);                       \
    else                                                                                                  \
      hipLaunchKernelGGL((moe::quant_rows_bf16_kernel<NVv, false>), dim3(T), dim3(moe::kRowThreads), 0,  \
                         s, x, H, xq, scale, zero_rows, zk, pair_pos, scale_rows, ro);                    \
  }
  if (per <= 1) MOE_QUANT_NV(1)
  else if (per <= 2) MOE_QUANT_NV(2)
  else if (per <= 4) MOE_QUANT_NV(4)
  else if (per <= 8) MOE_QUANT_NV(8)
  else MOE_QUANT_NV(0)
#undef MOE_QUANT_NV
  return hipGetLastError();
}

hipError_t launch_act(const float* g, int S, int P, int I, const int32_t* expert_offsets, int E,
                      bool fp8, const float* x_scale, const int32_t* sorted_pairs, int k, void* h,
                      float* h_scale, hipStream_t s) {
  if (fp8) {
    hipLaunchKernelGGL(moe::act_fp8_kernel, dim3(P), dim3(moe::kRowThreads), 0, s, g, S, P, I,
                       expert_offsets, E, x_scale, sorted_pairs, k, static_cast<uint8_t*>(h),
                       h_scale);
  } else {
    const dim3 grid(P, (I + moe::kActCols - 1) / moe::kActCols);
    hipLaunchKernelGGL(moe::act_bf16_kernel, grid, dim3(moe::kRowThreads), 0, s, g, S, P, I,
                       expert_offsets, E, static_cast<uint16_t*>(h));
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const void* y, bool y_bf16, int S, int P, const float* topk_w,
                         const int32_t* pair_pos, const int32_t* expert_offsets, const float* row_scale,
                         int E, int T, int k, int H, uint16_t* out, hipStream_t s) {
  const int cols = y_bf16 ? 8 : 4;
  const dim3 grid(T, (H / cols + moe::kRowThreads - 1) / moe::kRowThreads);
  if (y_bf16)
    moe::launch_reduce_t<true>(grid, y, S, P, topk_w, pair_pos, expert_offsets, row_scale, E, T, k, H, out, s);
  else
    moe::launch_reduce_t<false>(grid, y, S, P, topk_w, pair_pos, expert_offsets, row_scale, E, T, k, H, out, s);
  return hipGetLastError();
}

}  // namespace moe_host
