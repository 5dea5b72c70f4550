// Grouped expert GEMM with int4 weights and bf16 activations (w4a16; SGLang
// tuning guide dtype list: int4_w4a16), register streaming for decode and
// small batches: the pipeline role of stream_gemm.hip (gate-up reads tokens
// through the route index, SiLU-and-mul in its epilogue; down writes bf16
// rows), with a quarter of the bf16 weight bytes.
//
//  * Weights: two's-complement nibbles, the lower K index in the low nibble,
//    one fp32 scale per 128 K values of a row; packed by moe_pack_weights
//    into 1 KiB chunks of 16 rows x 64 bytes (= 128 K values).  A K step is
//    one chunk: lane l holds row l % 16, K values 32*(l/16) .. +32 of the
//    step, as four dwords of eight values.
//  * Conversion in registers, about 1.5 VALU operations per value: the
//    nibbles n = q + 8 (an xor with 0x8) of a dword split into low and high
//    nibble bytes, and byte permutes place each pair next to 0x43 bytes:
//    bf16 0x4300 | n = 128 + n = 136 + q exactly.  The products then carry
//    136 * sum(x) too; one more MFMA per 32 K values of each token block
//    against a constant 136 operand gives that sum, subtracted per step.
//  * Four bf16 MFMAs (16x16x32) per step and weight block, each on eight
//    consecutive K values of the lane; the x fragments are loaded at the
//    same K positions (64 contiguous bytes per lane and step).  The step's
//    sum is one scale group: acc += scale * (sum - 136 * sum(x)), in fp32.
//  * Work item = (task tile, 16 h columns) for gate-up (a gate block and its
//    up block) or (task tile, 32 columns) for down; the K steps of an item
//    split over the W waves of a workgroup, partial sums added in LDS in
//    ascending wave order (deterministic).
#include "lds_dma.h"
#include "decode_route.h"

namespace moe {

constexpr int kW4NB = 2;   // 16-column weight blocks per item

__device__ __forceinline__ void w4_mfma(f32x4& acc, const u32x4& a, const u32x4& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 acc, 0, 0, 0);
}

// eight nibbles (K order, low nibble first) -> eight bf16 values 136 + q
__device__ __forceinline__ u32x4 w4_expand(uint32_t packed) {
  const uint32_t t = packed ^ 0x88888888u;          // q + 8 in every nibble
  const uint32_t lo = t & 0x0f0f0f0fu;              // values 0, 2, 4, 6
  const uint32_t hi = (t >> 4) & 0x0f0f0f0fu;       // values 1, 3, 5, 7
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    // bytes: lo[k], 0, hi[k], 0 (v_perm_b32: 0-3 select the second source, 4-7 the first, 12 -> 0)
    const uint32_t sel = (uint32_t)k | (0x0cu << 8) | ((uint32_t)(4 + k) << 16) | (0x0cu << 24);
    r[k] = __builtin_amdgcn_perm(hi, lo, sel) | 0x43004300u;
  }
  return r;
}

// NB weight blocks per item: 2, or 4 on tiles of 32 or more rows (gate-up:
// two gate and two up blocks, down: 64 columns), halving the re-reads of
// the tile's token rows.
// ROUTE: gate-up of a decode batch (at most 64 pairs) with the routing build
// folded in (tasks and row tokens from decode_route).
template <int MB, int W, bool GATEUP, int NB = kW4NB, bool ROUTE = false>
__global__ void __launch_bounds__(W * 64)
stream_w4_kernel(moe_host::StreamArgs g) {
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
  const int nsteps = g.K / 128;   // 128 K values per step
  const int spw = nsteps / W;
  const int w_blocks = g.w_rows / 16;
  const char* __restrict__ A = static_cast<const char*>(g.a);
  const char* __restrict__ B = static_cast<const char*>(g.b);
  const u32x4 c136 = {0x43084308u, 0x43084308u, 0x43084308u, 0x43084308u};   // bf16 136.0

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
      ap[b] = A + (size_t)arow * x_row_bytes + (size_t)step0 * 256 + 64 * lgrp;
    }
    const char* bp[NB];
    const float* sp[NB];
#pragma unroll
    for (int q = 0; q < NB; q++) {
      bp[q] = B + (((size_t)task.expert * w_blocks + blk[q]) * nsteps + step0) * 1024 + 16 * lane;
      sp[q] = g.b_scale + ((size_t)task.expert * g.w_rows + blk[q] * 16 + lrow) * nsteps + step0;
    }

    f32x4 acc[MB][NB];
#pragma unroll
    for (int m = 0; m < MB; m++)
#pragma unroll
      for (int q = 0; q < NB; q++) acc[m][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 fa0[MB][4], fb0[NB], fa1[MB][4], fb1[NB];
    float fs0[NB], fs1[NB];
    auto load = [&](u32x4 (&fa)[MB][4], u32x4 (&fb)[NB], float (&fs)[NB], int st)
        __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < NB; q++) {
        fb[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bp[q] + (size_t)st * 1024));
        fs[q] = sp[q][st];
      }
#pragma unroll
      for (int b = 0; b < MB; b++)
#pragma unroll
        for (int j = 0; j < 4; j++) fa[b][j] = *reinterpret_cast<const u32x4*>(ap[b] + (size_t)st * 256 + 16 * j);
    };
    auto compute = [&](const u32x4 (&fa)[MB][4], const u32x4 (&fb)[NB], const float (&fs)[NB])
        __attribute__((always_inline)) {
      f32x4 cb[MB];   // 136 * sum of the step's x values of each row
#pragma unroll
      for (int b = 0; b < MB; b++) {
        cb[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; j++) w4_mfma(cb[b], fa[b][j], c136);
      }
#pragma unroll
      for (int q = 0; q < NB; q++) {
        u32x4 wv[4];
#pragma unroll
        for (int j = 0; j < 4; j++) wv[j] = w4_expand(fb[q][j]);
#pragma unroll
        for (int b = 0; b < MB; b++) {
          f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; j++) w4_mfma(t, fa[b][j], wv[j]);
          acc[b][q] += fs[q] * (t - cb[b]);
        }
      }
    };
    // two register stages, no load under a condition (spw >= 1)
    load(fa0, fb0, fs0, 0);
    int i = 0;
    for (; i + 2 < spw; i += 2) {
      load(fa1, fb1, fs1, i + 1);
      compute(fa0, fb0, fs0);
      load(fa0, fb0, fs0, i + 2);
      compute(fa1, fb1, fs1);
    }
    if (i + 1 < spw) {
      load(fa1, fb1, fs1, i + 1);
      compute(fa0, fb0, fs0);
      compute(fa1, fb1, fs1);
    } else {
      compute(fa0, fb0, fs0);
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
#pragma unroll
      for (int q = 0; q < NB; q++) {
        tot[q] = red[0][m][q][lane];
#pragma unroll
        for (int s = 1; s < W; s++) tot[q] += red[s][m][q][lane];
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
                f32_to_bf16_bits(silu_f32(tot[h][r4]) * tot[NH + h][r4]);
        } else {
#pragma unroll
          for (int q = 0; q < NB; q++)
            static_cast<uint16_t*>(g.c)[r * g.N_out + blk[q] * 16 + lrow] = f32_to_bf16_bits(tot[q][r4]);
        }
      }
    }
    __syncthreads();   // LDS free for the next item
  }
}

template <int MB, int W>
static hipError_t launch_w4_t(const moe_host::StreamArgs& a, bool gateup, int nb, int grid, hipStream_t s) {
  if (a.route.ids) {   // the routing build folded in: gate-up on 16-row tiles, two blocks per item
    if constexpr (MB == 1) {
      if (gateup && nb == 2) {
        hipLaunchKernelGGL((stream_w4_kernel<MB, W, true, 2, true>), dim3(grid), dim3(W * 64), 0, s, a);
        return hipGetLastError();
      }
    }
    return hipErrorInvalidValue;
  }
  if (nb == 4) {
    if constexpr (MB >= 2 && MB * W <= 16) {   // partial sums within 64 KiB of LDS
      if (gateup)
        hipLaunchKernelGGL((stream_w4_kernel<MB, W, true, 4>), dim3(grid), dim3(W * 64), 0, s, a);
      else
        hipLaunchKernelGGL((stream_w4_kernel<MB, W, false, 4>), dim3(grid), dim3(W * 64), 0, s, a);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (gateup)
    hipLaunchKernelGGL((stream_w4_kernel<MB, W, true>), dim3(grid), dim3(W * 64), 0, s, a);
  else
    hipLaunchKernelGGL((stream_w4_kernel<MB, W, false>), dim3(grid), dim3(W * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe

namespace moe_host {

hipError_t launch_stream_w4(const StreamArgs& a, bool gateup, int mb, int waves, int grid, hipStream_t s,
                            int nb) {
#define MOE_W4_CASE(M, Wv) \
  if (mb == M && waves == Wv) return moe::launch_w4_t<M, Wv>(a, gateup, nb, grid, s);
  MOE_W4_CASE(1, 1) MOE_W4_CASE(1, 2) MOE_W4_CASE(1, 4) MOE_W4_CASE(1, 8)
  MOE_W4_CASE(2, 1) MOE_W4_CASE(2, 2) MOE_W4_CASE(2, 4) MOE_W4_CASE(2, 8)
  MOE_W4_CASE(4, 1) MOE_W4_CASE(4, 2) MOE_W4_CASE(4, 4) MOE_W4_CASE(4, 8)
#undef MOE_W4_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe_host
