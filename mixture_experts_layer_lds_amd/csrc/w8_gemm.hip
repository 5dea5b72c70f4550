// Grouped expert GEMM with int8 weights and bf16 activations (w8a16; SGLang
// tuning guide dtype list: int8_w8a16), register streaming at every size:
// the pipeline role of stream_gemm.hip (gate-up reads tokens through the
// route index, SiLU-and-mul in its epilogue; down writes bf16 rows), with
// half the bf16 weight bytes.
//
//  * Weights: int8 codes with one fp32 scale per weight row, packed by
//    moe_pack_weights into 1 KiB chunks of 16 rows x 64 bytes.  A K step is
//    one chunk (64 K values): lane l holds row l % 16, K values
//    16*(l/16) .. +16 of the step, as one 16-byte load.
//  * Conversion in registers: each code becomes an exact fp32 integer (a
//    sign-extending byte conversion) whose upper half is its bf16 value (at
//    most 8 significant bits), and a byte permute packs two of them: about
//    1.5 VALU operations per weight, no offset to correct.
//  * Two bf16 MFMAs (16x16x32) per step and weight block: the lane's first
//    eight K values, then its last eight, against the token rows' bf16
//    values at the same K positions (32 contiguous bytes per lane and step).
//  * The row scale is constant along K, so it multiplies the sums once in
//    the epilogue: h = SiLU(g * s_g) * (u * s_u) on gate-up, y = sum * s on
//    down.
//  * Work item = (task tile, 16 h columns) for gate-up (a gate block and its
//    up block) or (task tile, 32 columns) for down; the K steps of an item
//    split over the W waves of a workgroup, partial sums added in LDS in
//    ascending wave order (deterministic).
#include "lds_dma.h"
#include "decode_route.h"

namespace moe {

constexpr int kW8NB = 2;   // 16-column weight blocks per item

__device__ __forceinline__ void w8_mfma(f32x4& acc, const u32x4& a, const u32x4& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 acc, 0, 0, 0);
}

// two int8 codes (bytes `at` and `at + 1` of a dword, lower K first) -> one
// dword of two bf16 values: the upper halves of their exact fp32 values
// (v_perm_b32: bytes 0-3 of the second source, 4-7 of the first)
__device__ __forceinline__ uint32_t w8_pair(uint32_t packed, int at) {
  const float f0 = (float)(int)(int8_t)((packed >> (8 * at)) & 0xffu);
  const float f1 = (float)(int)(int8_t)((packed >> (8 * at + 8)) & 0xffu);
  return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
}

// 16 codes -> the bf16 fragments of the lane's first and last eight K values
__device__ __forceinline__ void w8_expand(const u32x4& c, u32x4& first, u32x4& last) {
  first = u32x4{w8_pair(c[0], 0), w8_pair(c[0], 2), w8_pair(c[1], 0), w8_pair(c[1], 2)};
  last = u32x4{w8_pair(c[2], 0), w8_pair(c[2], 2), w8_pair(c[3], 0), w8_pair(c[3], 2)};
}

// NB weight blocks per item: 2, or 4 on tiles of 32 or more rows (gate-up:
// two gate and two up blocks, down: 64 columns), halving the re-reads of
// the tile's token rows.
// ROUTE: gate-up of a decode batch (at most 64 pairs) with the routing build
// folded in (tasks and row tokens from decode_route).
template <int MB, int W, bool GATEUP, int NB = kW8NB, bool ROUTE = false>
__global__ void __launch_bounds__(W * 64)
stream_w8_kernel(moe_host::StreamArgs g) {
  static_assert(!ROUTE || GATEUP, "the folded routing build serves the gate-up");
  constexpr int NH = GATEUP ? NB / 2 : NB;   // 16-column output blocks per item
  __shared__ f32x4 red[W][MB][NB][64];
  const int lane = threadIdx.x & 63;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  DecodeRoute rt{};
  int num_tasks;
  if constexpr (ROUTE) {
    rt = decode_route(g.route.ids, g.P, g.route.E, g.route.block_m, lane);
    if (blockIdx.x == 0) decode_route_write(rt, g.route, g.P, threadIdx.x, W * 64, lane, wave);
    num_tasks = min(rt.ntasks, g.max_tasks);
  } else {
    num_tasks = min(g.header[kHdrNumTasks], g.max_tasks);
  }
  const int n_groups = g.N_out / 16 / NH;
  const int total = num_tasks * n_groups;
  const size_t x_row_bytes = (size_t)g.K * 2;
  const int nsteps = g.K / 64;   // 64 K values per step
  const int spw = nsteps / W;
  const int w_blocks = g.w_rows / 16;
  const char* __restrict__ A = static_cast<const char*>(g.a);
  const char* __restrict__ B = static_cast<const char*>(g.b);

  const int G = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd = G / 8, extra = G % 8;
  const int vid = (xcd < extra ? xcd * (per_xcd + 1) : extra * (per_xcd + 1) + (xcd - extra) * per_xcd) + slot;

  for (int item = vid; item < total; item += G) {
    const int ti = item / n_groups;
    const int cg = item - ti * n_groups;
    moe_task_t task;
    if constexpr (ROUTE) task = decode_task(rt, ti, g.route.block_m);
    else task = load_task_scalar(g.tasks + ti);
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
    const int step0 = wave * spw;
    // token rows: past the tile, the tile's first row (valid, never stored)
    const char* ap[MB];
#pragma unroll
    for (int b = 0; b < MB; b++) {
      const int rb = b * 16 < task.rows ? b : 0;
      int arow;
      if constexpr (ROUTE) {
        arow = decode_sorted_pair(rt, task.row_begin + (rb * 16 + lrow < task.rows ? rb * 16 + lrow : 0)) / g.topk;
      } else if constexpr (GATEUP) {
        const i32x16_t sp = load16_scalar(g.sorted_pairs + task.row_begin + rb * 16);
        const int p = rb * 16 + lrow < task.rows ? spread16(sp, lane) : sp[0];
        arow = p / g.topk;
      } else {
        arow = task.row_begin + (rb * 16 + lrow < task.rows ? rb * 16 + lrow : 0);
      }
      ap[b] = A + (size_t)arow * x_row_bytes + (size_t)step0 * 128 + 32 * lgrp;
    }
    const char* bp[NB];
#pragma unroll
    for (int q = 0; q < NB; q++)
      bp[q] = B + (((size_t)task.expert * w_blocks + blk[q]) * nsteps + step0) * 1024 + 16 * lane;

    f32x4 acc[MB][NB];
#pragma unroll
    for (int m = 0; m < MB; m++)
#pragma unroll
      for (int q = 0; q < NB; q++) acc[m][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 fa0[MB][2], fb0[NB], fa1[MB][2], fb1[NB];
    auto load = [&](u32x4 (&fa)[MB][2], u32x4 (&fb)[NB], int st) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < NB; q++)
        fb[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bp[q] + (size_t)st * 1024));
#pragma unroll
      for (int b = 0; b < MB; b++)
#pragma unroll
        for (int j = 0; j < 2; j++) fa[b][j] = *reinterpret_cast<const u32x4*>(ap[b] + (size_t)st * 128 + 16 * j);
    };
    auto compute = [&](const u32x4 (&fa)[MB][2], const u32x4 (&fb)[NB]) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < NB; q++) {
        u32x4 w0, w1;
        w8_expand(fb[q], w0, w1);
#pragma unroll
        for (int b = 0; b < MB; b++) {
          w8_mfma(acc[b][q], fa[b][0], w0);
          w8_mfma(acc[b][q], fa[b][1], w1);
        }
      }
    };
    // two register stages, no load under a condition (spw >= 1)
    load(fa0, fb0, 0);
    int i = 0;
    for (; i + 2 < spw; i += 2) {
      load(fa1, fb1, i + 1);
      compute(fa0, fb0);
      load(fa0, fb0, i + 2);
      compute(fa1, fb1);
    }
    if (i + 1 < spw) {
      load(fa1, fb1, i + 1);
      compute(fa0, fb0);
      compute(fa1, fb1);
    } else {
      compute(fa0, fb0);
    }

#pragma unroll
    for (int m = 0; m < MB; m++)
#pragma unroll
      for (int q = 0; q < NB; q++) red[wave][m][q][lane] = acc[m][q];
    __syncthreads();

    // Epilogue of row block m by wave m % W: lane holds column (lane % 16)
    // and rows 4*(lane / 16) + i of each 16 x 16 block.
    for (int m = wave; m < MB; m += W) {
      f32x4 tot[NB];
      float cs[NB];   // the row scales of this lane's weight rows
#pragma unroll
      for (int q = 0; q < NB; q++) {
        tot[q] = red[0][m][q][lane];
#pragma unroll
        for (int s = 1; s < W; s++) tot[q] += red[s][m][q][lane];
        const i32x16_t v = load16_scalar(g.b_scale + (size_t)task.expert * g.w_rows + blk[q] * 16);
        cs[q] = __int_as_float(spread16(v, lane));
      }
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        const int rr = m * 16 + 4 * lgrp + r4;
        if (rr >= task.rows) continue;
        const size_t r = (size_t)(task.row_begin + rr);
        if constexpr (GATEUP) {
#pragma unroll
          for (int h = 0; h < NH; h++)
            static_cast<uint16_t*>(g.c)[r * g.N_out + blk[h] * 16 + lrow] =
                f32_to_bf16_bits(silu_f32(tot[h][r4] * cs[h]) * (tot[NH + h][r4] * cs[NH + h]));
        } else {
#pragma unroll
          for (int q = 0; q < NB; q++)
            static_cast<uint16_t*>(g.c)[r * g.N_out + blk[q] * 16 + lrow] = f32_to_bf16_bits(tot[q][r4] * cs[q]);
        }
      }
    }
    __syncthreads();   // LDS free for the next item
  }
}

template <int MB, int W>
static hipError_t launch_w8_t(const moe_host::StreamArgs& a, bool gateup, int nb, int grid, hipStream_t s) {
  if (a.route.ids) {   // the routing build folded in: gate-up on 16-row tiles, two blocks per item
    if constexpr (MB == 1) {
      if (gateup && nb == 2) {
        hipLaunchKernelGGL((stream_w8_kernel<MB, W, true, 2, true>), dim3(grid), dim3(W * 64), 0, s, a);
        return hipGetLastError();
      }
    }
    return hipErrorInvalidValue;
  }
  if (nb == 4) {
    if constexpr (MB >= 2 && MB * W <= 16) {   // partial sums within 64 KiB of LDS
      if (gateup)
        hipLaunchKernelGGL((stream_w8_kernel<MB, W, true, 4>), dim3(grid), dim3(W * 64), 0, s, a);
      else
        hipLaunchKernelGGL((stream_w8_kernel<MB, W, false, 4>), dim3(grid), dim3(W * 64), 0, s, a);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (gateup)
    hipLaunchKernelGGL((stream_w8_kernel<MB, W, true>), dim3(grid), dim3(W * 64), 0, s, a);
  else
    hipLaunchKernelGGL((stream_w8_kernel<MB, W, false>), dim3(grid), dim3(W * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe

namespace moe_host {

hipError_t launch_stream_w8(const StreamArgs& a, bool gateup, int mb, int waves, int grid, hipStream_t s,
                            int nb) {
#define MOE_W8_CASE(M, Wv) \
  if (mb == M && waves == Wv) return moe::launch_w8_t<M, Wv>(a, gateup, nb, grid, s);
  MOE_W8_CASE(1, 1) MOE_W8_CASE(1, 2) MOE_W8_CASE(1, 4) MOE_W8_CASE(1, 8)
  MOE_W8_CASE(2, 1) MOE_W8_CASE(2, 2) MOE_W8_CASE(2, 4) MOE_W8_CASE(2, 8)
  MOE_W8_CASE(4, 1) MOE_W8_CASE(4, 2) MOE_W8_CASE(4, 4) MOE_W8_CASE(4, 8)
#undef MOE_W8_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe_host
