// Grouped expert GEMM for block-scaled fp8 (SGLang tuning guide:
// block_shape [128, 128], DeepSeek-V3's quantisation): e4m3 weights with one
// fp32 scale per 128 x 128 block, e4m3 activations with one per 128-value
// group of a row; register streaming for decode and small batches, in the
// pipeline role of stream_gemm.hip (gate-up through the route index with
// SiLU-and-mul in its epilogue, down to bf16 rows).
//
//  * A K unit is 128 values: two packed 64-byte steps, one full-rate
//    v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales into a fresh
//    accumulator, then acc += unit_sum * (x group scale * w block scale).
//    fp32 block scales are not powers of two, so they cannot ride in the
//    instruction's e8m0 scale operands; the rescale is four FMAs per unit.
//  * Operands swapped against stream_gemm: the weights are the A operand
//    and the token rows the B operand, so a lane's output column is one
//    token (its group scale: one load per unit) and its four output rows
//    are four weight rows of one 128-row block (one block scale, the same
//    address for every lane).  The epilogue then writes four consecutive
//    output columns per lane.
//  * Activation group scales come per sorted row, unit-major ([K/128][P]),
//    written by the quantisation passes.
//  * Per-channel mode (BLOCK false: the fp8 w8a8 layer, one scale per weight
//    row and per token row): the same operand arrangement and 128-value
//    units, and the per-channel epilogue of the fp8 path: gate-up forms
//    SiLU(g * rs * cs_g) * (u * rs * cs_u) in fp32 (the requantisation pass
//    finds each row's amax: folding it here with atomics cost 8% of the
//    gate-up time at T=16); down applies the weight row scales (the row
//    scale is the top-k reduction's).  Four MFMAs of 16x16x32 per 128
//    values become one of 16x16x128.
#include "lds_dma.h"
#include "decode_route.h"

namespace moe {

// NB weight blocks per item: 2 (gate-up: one gate and one up block; down:
// 32 columns), or 4 on 64-row tiles (gate-up: two of each, 32 h columns;
// down: 64 columns), which halves the re-reads of the tile's token rows
// across an expert's column groups.
template <int MB, int W, bool GATEUP, bool BLOCK, int NB = 2>
__global__ void __launch_bounds__(W * 64)
stream_fp8b_kernel(moe_host::StreamArgs g) {
  static_assert(NB == 2 || NB == 4, "two or four weight blocks per item");
  constexpr int NH = GATEUP ? NB / 2 : NB;   // 16-column output blocks per item
  __shared__ f32x4 red[W][MB][NB][64];
  const int lane = threadIdx.x & 63;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int num_tasks = min(g.header[kHdrNumTasks], g.max_tasks);
  const int n_groups = g.N_out / 16 / NH;
  const int total = num_tasks * n_groups;
  const int nsteps = g.K / 64;    // 64-byte steps of e4m3
  const int units = g.K / 128;    // 128-value units = scale groups
  const int upw = units / W;
  const int w_blocks = g.w_rows / 16;
  const int P = g.P;
  const char* __restrict__ A = static_cast<const char*>(g.a);
  const char* __restrict__ B = static_cast<const char*>(g.b);

  const int G = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd = G / 8, extra = G % 8;
  const int vid = (xcd < extra ? xcd * (per_xcd + 1) : extra * (per_xcd + 1) + (xcd - extra) * per_xcd) + slot;

  for (int item = vid; item < total; item += G) {
    const int ti = item / n_groups;
    const int cg = item - ti * n_groups;
    const moe_task_t task = load_task_scalar(g.tasks + ti);
    int blk[NB];
    if constexpr (GATEUP) {
#pragma unroll
      for (int h = 0; h < NH; h++) {
        blk[h] = cg * NH + h;                        // gate rows
        blk[NH + h] = g.N_out / 16 + cg * NH + h;    // the matching up rows
      }
    } else {
#pragma unroll
      for (int q = 0; q < NB; q++) blk[q] = cg * NB + q;
    }
    const int unit0 = wave * upw;
    // token rows (the B operand): past the tile, the tile's first row
    const char* xp[MB];
    const float* xsp[MB];
#pragma unroll
    for (int b = 0; b < MB; b++) {
      const int rb = b * 16 < task.rows ? b : 0;
      const bool in = rb * 16 + lrow < task.rows;
      const int srow = task.row_begin + (in ? rb * 16 + lrow : 0);   // sorted row
      int arow;
      if constexpr (GATEUP) {
        const i32x16_t sp = load16_scalar(g.sorted_pairs + task.row_begin + rb * 16);
        const int p = in ? spread16(sp, lane) : sp[0];
        arow = p / g.topk;
      } else {
        arow = srow;
      }
      xp[b] = A + (size_t)arow * g.K + (size_t)unit0 * 128 + 16 * lgrp;
      xsp[b] = BLOCK ? g.row_scale + (size_t)unit0 * P + srow : g.row_scale + srow;
    }
    const char* wp[NB];
    const float* wsp[NB];
#pragma unroll
    for (int q = 0; q < NB; q++) {
      wp[q] = B + (((size_t)task.expert * w_blocks + blk[q]) * nsteps + (size_t)unit0 * 2) * 1024 + 16 * lane;
      wsp[q] = BLOCK ? g.b_scale + ((size_t)task.expert * (g.w_rows / 128) + (blk[q] * 16) / 128) * units + unit0
                     : g.b_scale + (size_t)task.expert * g.w_rows + blk[q] * 16 + 4 * lgrp;
    }

    f32x4 acc[MB][NB];
#pragma unroll
    for (int m = 0; m < MB; m++)
#pragma unroll
      for (int q = 0; q < NB; q++) acc[m][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 fx0[MB][2], fw0[NB][2], fx1[MB][2], fw1[NB][2];
    float sx0[MB], sw0[NB], sx1[MB], sw1[NB];
    auto load = [&](u32x4 (&fx)[MB][2], u32x4 (&fw)[NB][2], float (&sx)[MB], float (&sw)[NB], int u)
        __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < NB; q++) {
        fw[q][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp[q] + (size_t)u * 2048));
        fw[q][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp[q] + (size_t)u * 2048 + 1024));
        if constexpr (BLOCK) sw[q] = wsp[q][u];
      }
#pragma unroll
      for (int b = 0; b < MB; b++) {
        fx[b][0] = *reinterpret_cast<const u32x4*>(xp[b] + (size_t)u * 128);
        fx[b][1] = *reinterpret_cast<const u32x4*>(xp[b] + (size_t)u * 128 + 64);
        if constexpr (BLOCK) sx[b] = xsp[b][(size_t)u * P];
      }
    };
    auto compute = [&](const u32x4 (&fx)[MB][2], const u32x4 (&fw)[NB][2], const float (&sx)[MB],
                       const float (&sw)[NB]) __attribute__((always_inline)) {
#pragma unroll
      for (int b = 0; b < MB; b++)
#pragma unroll
        for (int q = 0; q < NB; q++) {
          // a fresh accumulator per unit: consecutive MFMAs do not wait on
          // each other's results; the unit sums are added in fp32
          f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
          mfma_fp8_k128(t, fw[q][0], fw[q][1], fx[b][0], fx[b][1]);
          if constexpr (BLOCK) acc[b][q] += t * (sx[b] * sw[q]);
          else acc[b][q] += t;
        }
    };
    load(fx0, fw0, sx0, sw0, 0);
    int i = 0;
    for (; i + 2 < upw; i += 2) {
      load(fx1, fw1, sx1, sw1, i + 1);
      compute(fx0, fw0, sx0, sw0);
      load(fx0, fw0, sx0, sw0, i + 2);
      compute(fx1, fw1, sx1, sw1);
    }
    if (i + 1 < upw) {
      load(fx1, fw1, sx1, sw1, i + 1);
      compute(fx0, fw0, sx0, sw0);
      compute(fx1, fw1, sx1, sw1);
    } else {
      compute(fx0, fw0, sx0, sw0);
    }

#pragma unroll
    for (int m = 0; m < MB; m++)
#pragma unroll
      for (int q = 0; q < NB; q++) red[wave][m][q][lane] = acc[m][q];
    __syncthreads();

    // Epilogue of token block b by wave b % W: lane holds token row
    // 16 b + (lane % 16) and weight rows 4*(lane / 16) + i of each block.
    for (int b = wave; b < MB; b += W) {
      f32x4 tot[NB];
#pragma unroll
      for (int q = 0; q < NB; q++) {
        tot[q] = red[0][b][q][lane];
#pragma unroll
        for (int s = 1; s < W; s++) tot[q] += red[s][b][q][lane];
      }
      const int rr = b * 16 + lrow;
      if constexpr (!BLOCK) {   // per-channel scales: this lane's four weight rows, its token row
#pragma unroll
        for (int q = 0; q < NB; q++) {
          const f32x4 cs = *reinterpret_cast<const f32x4*>(wsp[q]);
          if constexpr (GATEUP) {
            const float rs = *xsp[b];
#pragma unroll
            for (int i4 = 0; i4 < 4; i4++) tot[q][i4] = (tot[q][i4] * rs) * cs[i4];
          } else {
#pragma unroll
            for (int i4 = 0; i4 < 4; i4++) tot[q][i4] = tot[q][i4] * cs[i4];
          }
        }
      }
      if (rr < task.rows) {
        const size_t r = (size_t)(task.row_begin + rr);
        if constexpr (GATEUP) {
#pragma unroll
          for (int h = 0; h < NH; h++) {
            f32x4 hv;
#pragma unroll
            for (int i4 = 0; i4 < 4; i4++) hv[i4] = silu_f32(tot[h][i4]) * tot[NH + h][i4];
            *reinterpret_cast<f32x4*>(static_cast<float*>(g.c) + r * g.N_out + blk[h] * 16 + 4 * lgrp) = hv;
          }
        } else {
#pragma unroll
          for (int q = 0; q < NB; q++) {
            u32x2 v;
            v.x = (uint32_t)f32_to_bf16_bits(tot[q][0]) | ((uint32_t)f32_to_bf16_bits(tot[q][1]) << 16);
            v.y = (uint32_t)f32_to_bf16_bits(tot[q][2]) | ((uint32_t)f32_to_bf16_bits(tot[q][3]) << 16);
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(g.c) + r * g.N_out + blk[q] * 16 + 4 * lgrp) = v;
          }
        }
      }
    }
    __syncthreads();
  }
}

// Per-row group quantisation of 128-value groups (the per-row fp8 rule on
// each group): one thread per 8 values, a group is 16 lanes.  Input bf16
// rows (x, one token per row) or fp32 rows (h, valid sorted rows only).
// Codes to q[row][..]; scales to group_scale[row][g] (when not null) and,
// unit-major, to rows_scale[g][dst_row] for each destination row: the
// sorted rows of the token's zk pairs (x), or the row itself (h).
// ROUTE (token rows, at most 64 pairs): the launch also does the routing
// build, and the sorted rows of each token's zk pairs come from there.
template <bool BF16_IN, bool ROUTE = false>
__global__ void __launch_bounds__(256)
quant_groups_kernel(const void* __restrict__ in, int n, int nrows, const int32_t* __restrict__ expert_offsets,
                    int E, uint8_t* __restrict__ q, float* __restrict__ group_scale,
                    float* __restrict__ rows_scale, int P, int zk, const int32_t* __restrict__ pair_pos,
                    moe_host::DecodeRouteOut route) {
  static_assert(!ROUTE || BF16_IN, "the folded routing build serves the token rows");
  const int r = blockIdx.x;
  __shared__ int s_rows[kMaxTopK];   // ROUTE: sorted rows of this token's pairs
  if constexpr (ROUTE) {
    const int lane = threadIdx.x & 63;
    const DecodeRoute rt = decode_route(route.ids, P, route.E, route.block_m, lane);
    if (r == 0) decode_route_write(rt, route, P, threadIdx.x, 256, lane, threadIdx.x >> 6);
    const int pj = __shfl(rt.pos, min(r * zk + lane, P - 1), kWave);
    if (threadIdx.x < zk) s_rows[threadIdx.x] = pj;
    __syncthreads();
  }
  const int valid = BF16_IN ? nrows : expert_offsets[E];
  if (r >= valid) return;   // block-uniform
  const int nvec = n / 8;
  const int groups = n / 128;
  for (int i = threadIdx.x; i < nvec; i += 256) {
    float v[8];
    if constexpr (BF16_IN) {
      const u32x4 w = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(in) + (size_t)r * n)[i];
#pragma unroll
      for (int k = 0; k < 4; k++) {
        v[2 * k] = bf16_bits_to_f32(w[k] & 0xffffu);
        v[2 * k + 1] = bf16_bits_to_f32(w[k] >> 16);
      }
    } else {
      const f32x4* row = reinterpret_cast<const f32x4*>(static_cast<const float*>(in) + (size_t)r * n);
      const f32x4 a = row[2 * i], b = row[2 * i + 1];
#pragma unroll
      for (int k = 0; k < 4; k++) v[k] = a[k], v[4 + k] = b[k];
    }
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k++) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[k]));
    amax = max16(amax);   // the 16 lanes of one group (256-thread strides keep groups aligned)
    float sc, inv;
    e4m3_row_scales(amax, &sc, &inv);
    u32x2 c;
    c.x = f32x4_to_e4m3x4_sat(__fmul_rn(v[0], inv), __fmul_rn(v[1], inv), __fmul_rn(v[2], inv),
                              __fmul_rn(v[3], inv));
    c.y = f32x4_to_e4m3x4_sat(__fmul_rn(v[4], inv), __fmul_rn(v[5], inv), __fmul_rn(v[6], inv),
                              __fmul_rn(v[7], inv));
    reinterpret_cast<u32x2*>(q + (size_t)r * n)[i] = c;
    if ((i & 15) == 0) {
      const int gidx = i / 16;
      if (group_scale) group_scale[(size_t)r * groups + gidx] = sc;
      if constexpr (BF16_IN) {
        for (int j = 0; j < zk; j++)
          rows_scale[(size_t)gidx * P + (ROUTE ? s_rows[j] : pair_pos[(size_t)r * zk + j])] = sc;
      } else {
        rows_scale[(size_t)gidx * P + r] = sc;
      }
    }
  }
}

template <int MB, int W>
static hipError_t launch_fp8b_t(const moe_host::StreamArgs& a, bool gateup, bool block, int nb, int grid,
                                hipStream_t s) {
  if (block && nb == 4) {
    if constexpr (MB == 4 && W <= 2) {
      if (gateup)
        hipLaunchKernelGGL((stream_fp8b_kernel<MB, W, true, true, 4>), dim3(grid), dim3(W * 64), 0, s, a);
      else
        hipLaunchKernelGGL((stream_fp8b_kernel<MB, W, false, true, 4>), dim3(grid), dim3(W * 64), 0, s, a);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (block) {
    if (gateup)
      hipLaunchKernelGGL((stream_fp8b_kernel<MB, W, true, true>), dim3(grid), dim3(W * 64), 0, s, a);
    else
      hipLaunchKernelGGL((stream_fp8b_kernel<MB, W, false, true>), dim3(grid), dim3(W * 64), 0, s, a);
  } else {
    if (gateup)
      hipLaunchKernelGGL((stream_fp8b_kernel<MB, W, true, false>), dim3(grid), dim3(W * 64), 0, s, a);
    else
      hipLaunchKernelGGL((stream_fp8b_kernel<MB, W, false, false>), dim3(grid), dim3(W * 64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe

namespace moe_host {

hipError_t launch_stream_fp8b(const StreamArgs& a, bool gateup, bool block, int mb, int waves, int grid,
                              hipStream_t s, int nb) {
  if (a.route.ids) return hipErrorInvalidValue;
#define MOE_FP8B_CASE(M, Wv) \
  if (mb == M && waves == Wv) return moe::launch_fp8b_t<M, Wv>(a, gateup, block, nb, grid, s);
  MOE_FP8B_CASE(1, 1) MOE_FP8B_CASE(1, 2) MOE_FP8B_CASE(1, 4) MOE_FP8B_CASE(1, 8)
  MOE_FP8B_CASE(2, 1) MOE_FP8B_CASE(2, 2) MOE_FP8B_CASE(2, 4) MOE_FP8B_CASE(2, 8)
  MOE_FP8B_CASE(4, 1) MOE_FP8B_CASE(4, 2) MOE_FP8B_CASE(4, 4) MOE_FP8B_CASE(4, 8)
#undef MOE_FP8B_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_quant_groups_bf16(const uint16_t* x, int T, int H, uint8_t* xq, float* group_scale,
                                    float* rows_scale, int P, int zk, const int32_t* pair_pos,
                                    hipStream_t s, const DecodeRouteOut* route) {
  if (route && ((long)T * zk > moe::kDecodeRoutePairs || P != T * zk || !route->ids)) return hipErrorInvalidValue;
  const DecodeRouteOut ro = route ? *route : DecodeRouteOut{};
  if (route)
    hipLaunchKernelGGL((moe::quant_groups_kernel<true, true>), dim3(T), dim3(256), 0, s, x, H, T, nullptr, 0, xq,
                       group_scale, rows_scale, P, zk, pair_pos, ro);
  else
    hipLaunchKernelGGL((moe::quant_groups_kernel<true, false>), dim3(T), dim3(256), 0, s, x, H, T, nullptr, 0,
                       xq, group_scale, rows_scale, P, zk, pair_pos, ro);
  return hipGetLastError();
}

hipError_t launch_requant_groups(const float* h, int P, int I, const int32_t* expert_offsets, int E,
                                 uint8_t* hq, float* rows_scale, hipStream_t s) {
  hipLaunchKernelGGL((moe::quant_groups_kernel<false, false>), dim3(P), dim3(256), 0, s, h, I, P, expert_offsets,
                     E, hq, nullptr, rows_scale, P, 1, nullptr, DecodeRouteOut{});
  return hipGetLastError();
}

}  // namespace moe_host
