// Precision-aware router GEMM (HPC-Ops x SGLang blog, section "Router
// GEMM: balancing routing precision and throughput", precision-aware BF16
// formulation).  The router keeps fp32 weights W [N][K] while the hidden
// states x [T][K] are bf16; W is split once into a bf16 part cut by
// truncation and a bf16 part holding the residual scaled by 256, so that
// W ~ W_high + W_low / 256, and the scores are two bf16 MFMA products that
// share every activation fragment, accumulated in fp32 and combined with
// the 1/256 scale in the epilogue:
//
//   score[t][n] = x[t] . W_high[n] + (x[t] . W_low[n]) / 256.
//
//  * Split (one-time, at weight load, like the blog's cached weight pair):
//    W_high = the top 16 bits of each fp32 pattern; W_low = RNE bf16 of
//    (W - W_high) * 256, both exact in fp32 before that rounding.  The two
//    parts are stored in the MFMA-fragment order of the expert weights
//    (1 KiB chunks of 16 rows x 64 bytes, ordered block, K step), rows
//    padded with zeros to a multiple of 16.
//  * GEMM: work item = (16*MB tokens, 16*NB experts, K slice s of S).  A
//    workgroup of W waves takes one item and splits its K slice over its
//    waves; each wave streams its x fragments and both weight parts into
//    registers (two register stages of U 64-byte K steps; unconditional
//    loads, token rows past T re-read the last row and are never stored)
//    and issues two MFMAs per (token block, expert block) and step, one per
//    weight part, on the same x fragment.  The waves' sums
//    hi + lo * 2^-8 meet in LDS and are added in ascending wave order.
//    With S > 1 (few tokens: the K split across workgroups puts every CU
//    to work on the weight stream) each slice writes its partial scores to
//    its own [T][N] plane; the planes are added in ascending slice order by
//    a small reduction, or by the router top-k kernel as it loads them.
//    Everything is deterministic.
#include "moe_common.h"

namespace moe {

__global__ void __launch_bounds__(256)
router_split_kernel(const float* __restrict__ w, int N, int K, int Np, uint16_t* __restrict__ hi,
                    uint16_t* __restrict__ lo) {
  const int nsteps = K / 32;
  const long total = (long)(Np / 16) * nsteps * 64;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int lane = (int)(gid & 63);
  const long chunk = gid >> 6;   // (16-row block, K step)
  const int step = (int)(chunk % nsteps);
  const int blk = (int)(chunk / nsteps);
  const int row = blk * 16 + (lane & 15);
  const int k0 = step * 32 + 8 * (lane >> 4);
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    uint32_t hp[2], lp[2];
#pragma unroll
    for (int e = 0; e < 2; e++) {
      const float v = row < N ? w[(long)row * K + k0 + 2 * i + e] : 0.f;
      const uint32_t u = __builtin_bit_cast(uint32_t, v);
      const float high = __builtin_bit_cast(float, u & 0xffff0000u);   // truncation
      hp[e] = u >> 16;
      lp[e] = f32_to_bf16_bits((v - high) * 256.0f);                  // exact residual, RNE
    }
    h[i] = hp[0] | (hp[1] << 16);
    l[i] = lp[0] | (lp[1] << 16);
  }
  *reinterpret_cast<u32x4*>(hi + chunk * 512 + lane * 8) = u32x4{h[0], h[1], h[2], h[3]};
  *reinterpret_cast<u32x4*>(lo + chunk * 512 + lane * 8) = u32x4{l[0], l[1], l[2], l[3]};
}

__device__ __forceinline__ void router_mfma(f32x4& acc, const u32x4& a, const u32x4& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// NT: the weight pair is read once (one token block): non-temporal loads.
// With several token blocks every block re-reads it, and it stays cached.
template <int MB, int NB, int W, int U, bool NT>
__global__ void __launch_bounds__(W * 64)
router_gemm_kernel(moe_host::RouterGemmArgs g) {
  __shared__ f32x4 red[W][MB][NB][64];
  const int lane = threadIdx.x & 63;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nsteps = g.K / 32;
  const int units = nsteps / U;

  // XCD-aware numbering: consecutive items (the expert blocks of one token
  // block and slice, which share its x rows) on the workgroups of one XCD.
  const int G = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd = G / 8, extra = G % 8;
  const int item = (xcd < extra ? xcd * (per_xcd + 1) : extra * (per_xcd + 1) + (xcd - extra) * per_xcd) + slot;
  const int nb = item % g.nb_count;
  const int rest = item / g.nb_count;
  const int tb = rest % g.tb_count;
  const int s = rest / g.tb_count;

  // K units of slice s, then of this wave (every wave gets at least one)
  const int s0 = (int)((long)s * units / g.S), s1 = (int)((long)(s + 1) * units / g.S);
  const int u0 = s0 + (int)((long)(s1 - s0) * wave / W);
  const int u1 = s0 + (int)((long)(s1 - s0) * (wave + 1) / W);
  const int n = u1 - u0;
  const int step0 = u0 * U;

  const char* __restrict__ X = static_cast<const char*>(g.x);
  const size_t row_bytes = (size_t)g.K * 2;
  const char* ap[MB];
#pragma unroll
  for (int b = 0; b < MB; b++) {
    const int t = tb * 16 * MB + b * 16 + lrow;
    ap[b] = X + (size_t)(t < g.T ? t : g.T - 1) * row_bytes + (size_t)step0 * 64 + 16 * lgrp;
  }
  const char* hp[NB];
  const char* lp[NB];
#pragma unroll
  for (int q = 0; q < NB; q++) {
    const size_t off = ((size_t)(nb * NB + q) * nsteps + step0) * 1024 + 16 * lane;
    hp[q] = static_cast<const char*>(g.w_hi) + off;
    lp[q] = static_cast<const char*>(g.w_lo) + off;
  }

  f32x4 ah[MB][NB], al[MB][NB];
#pragma unroll
  for (int b = 0; b < MB; b++)
#pragma unroll
    for (int q = 0; q < NB; q++) ah[b][q] = al[b][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 fx0[U][MB], fh0[U][NB], fl0[U][NB], fx1[U][MB], fh1[U][NB], fl1[U][NB];
  auto load = [&](u32x4 (&fx)[U][MB], u32x4 (&fh)[U][NB], u32x4 (&fl)[U][NB], int unit)
      __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int st = unit * U + u;
#pragma unroll
      for (int q = 0; q < NB; q++) {
        const u32x4* ph = reinterpret_cast<const u32x4*>(hp[q] + (size_t)st * 1024);
        const u32x4* pl = reinterpret_cast<const u32x4*>(lp[q] + (size_t)st * 1024);
        if constexpr (NT) {
          fh[u][q] = __builtin_nontemporal_load(ph);
          fl[u][q] = __builtin_nontemporal_load(pl);
        } else {
          fh[u][q] = *ph;
          fl[u][q] = *pl;
        }
      }
#pragma unroll
      for (int b = 0; b < MB; b++) fx[u][b] = *reinterpret_cast<const u32x4*>(ap[b] + (size_t)st * 64);
    }
  };
  auto compute = [&](const u32x4 (&fx)[U][MB], const u32x4 (&fh)[U][NB], const u32x4 (&fl)[U][NB])
      __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; u++)
#pragma unroll
      for (int b = 0; b < MB; b++)
#pragma unroll
        for (int q = 0; q < NB; q++) {
          router_mfma(ah[b][q], fx[u][b], fh[u][q]);
          router_mfma(al[b][q], fx[u][b], fl[u][q]);
        }
  };
  // Two register stages in turn, no load under a condition (n >= 1).
  load(fx0, fh0, fl0, 0);
  int i = 0;
  for (; i + 2 < n; i += 2) {
    load(fx1, fh1, fl1, i + 1);
    compute(fx0, fh0, fl0);
    load(fx0, fh0, fl0, i + 2);
    compute(fx1, fh1, fl1);
  }
  if (i + 1 < n) {
    load(fx1, fh1, fl1, i + 1);
    compute(fx0, fh0, fl0);
    compute(fx1, fh1, fl1);
  } else {
    compute(fx0, fh0, fl0);
  }

#pragma unroll
  for (int b = 0; b < MB; b++)
#pragma unroll
    for (int q = 0; q < NB; q++) red[wave][b][q][lane] = ah[b][q] + al[b][q] * 0.00390625f;
  __syncthreads();

  // Epilogue of token block b by wave b % W: lane holds expert column
  // (lane % 16) and token rows 4*(lane / 16) + i of each 16 x 16 block.
  float* out = g.out + (size_t)s * g.slice_stride;
  for (int b = wave; b < MB; b += W) {
#pragma unroll
    for (int q = 0; q < NB; q++) {
      f32x4 tot = red[0][b][q][lane];
#pragma unroll
      for (int w = 1; w < W; w++) tot += red[w][b][q][lane];
      const int col = (nb * NB + q) * 16 + lrow;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int t = tb * 16 * MB + b * 16 + 4 * lgrp + r;
        if (t < g.T && col < g.N) out[(size_t)t * g.N + col] = tot[r];
      }
    }
  }
}

// out[i] = sum over s ascending of in[s * stride + i], i < n.
__global__ void __launch_bounds__(256)
router_reduce_kernel(const float* __restrict__ in, int S, long stride, long n, float* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = in[i];
  for (int s = 1; s < S; s++) v += in[s * stride + i];
  out[i] = v;
}

}  // namespace moe

namespace moe_host {

hipError_t launch_router_split(const float* w, int N, int K, void* pair, hipStream_t s) {
  const int Np = (N + 15) / 16 * 16;
  uint16_t* hi = static_cast<uint16_t*>(pair);
  uint16_t* lo = hi + (size_t)Np * K;
  const long threads = (long)(Np / 16) * (K / 32) * 64;
  hipLaunchKernelGGL(moe::router_split_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     w, N, K, Np, hi, lo);
  return hipGetLastError();
}

RouterGemmPlan plan_router_gemm(int T, int N, int K, int cus) {
  RouterGemmPlan p;
  const int Np = (N + 15) / 16 * 16;
  const int units = K / 64;   // two 64-byte K steps per unit
  p.mb = T <= 16 ? 1 : (T <= 32 ? 2 : 4);
  p.tb_count = (T + 16 * p.mb - 1) / (16 * p.mb);
  p.nb = (p.tb_count > 2 && (Np / 16) % 2 == 0) ? 2 : 1;
  p.nb_count = Np / 16 / p.nb;
  p.waves = 4;
  while (p.waves > 1 && units < p.waves) p.waves /= 2;
  // Few items (few tokens): split K across workgroups until the grid
  // covers the CUs, keeping at least one unit per wave.
  const long base = (long)p.tb_count * p.nb_count;
  p.S = 1;
  while (p.S < 16 && base * p.S * 2 <= cus && units / (p.S * 2) >= p.waves) p.S *= 2;
  return p;
}

size_t router_partial_bytes(int T, int N, const RouterGemmPlan& p) {
  return p.S > 1 ? (size_t)p.S * T * N * 4 : 0;
}

hipError_t launch_router_gemm(const void* x, const void* pair, int T, int N, int K,
                              const RouterGemmPlan& p, float* out, hipStream_t s) {
  const int Np = (N + 15) / 16 * 16;
  RouterGemmArgs a;
  a.x = x;
  a.w_hi = pair;
  a.w_lo = static_cast<const char*>(pair) + (size_t)Np * K * 2;
  a.out = out;
  a.T = T;
  a.N = N;
  a.K = K;
  a.S = p.S;
  a.tb_count = p.tb_count;
  a.nb_count = p.nb_count;
  a.slice_stride = (long)T * N;
  const dim3 grid((unsigned)((long)p.S * p.tb_count * p.nb_count));
#define MOE_RG(MB, NB, W)                                                                        \
  if (p.mb == MB && p.nb == NB && p.waves == W) {                                                \
    if (p.tb_count == 1)                                                                         \
      hipLaunchKernelGGL((moe::router_gemm_kernel<MB, NB, W, 2, true>), grid, dim3(W * 64), 0, s, a); \
    else                                                                                         \
      hipLaunchKernelGGL((moe::router_gemm_kernel<MB, NB, W, 2, false>), grid, dim3(W * 64), 0, s, a); \
    return hipGetLastError();                                                                    \
  }
  MOE_RG(1, 1, 4) MOE_RG(2, 1, 4) MOE_RG(4, 1, 4) MOE_RG(4, 2, 4)
  MOE_RG(1, 1, 2) MOE_RG(2, 1, 2) MOE_RG(4, 1, 2) MOE_RG(4, 2, 2)
  MOE_RG(1, 1, 1) MOE_RG(2, 1, 1) MOE_RG(4, 1, 1) MOE_RG(4, 2, 1)
#undef MOE_RG
  return hipErrorInvalidValue;
}

hipError_t launch_router_reduce(const float* partials, int S, int T, int N, float* out, hipStream_t s) {
  const long n = (long)T * N;
  hipLaunchKernelGGL(moe::router_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     partials, S, n, n, out);
  return hipGetLastError();
}

}  // namespace moe_host
