// Grouped expert GEMM for few rows per expert (decode and small batches):
// weights streamed into registers, the reduction split over the waves of a
// workgroup and summed through LDS, SiLU-and-mul fused into the gate-up
// epilogue.
//
// Same pipeline role as the other grouped GEMMs (HPC-Ops x SGLang blog,
// section "MoE": gate-up reads tokens through the route index; a persistent
// grid consumes the per-tile task map; the activation follows the gate-up
// GEMM).
//
//  * Work item = (task tile of 16*MB rows, 32 output columns; 64 with four
//    weight blocks).  Gate-up: 16-column blocks of gate rows of W1 and the
//    matching blocks of up rows, so the item holds both halves of its h
//    columns; down: adjacent 16-column blocks of W2.
//  * A workgroup of W waves takes one item; wave w reduces K slice w
//    (nsteps / W 64-byte steps), streaming the item's two packed weight
//    blocks into registers (1 KiB non-temporal loads, two register stages of
//    two steps) and reading token rows through the route index (gate-up) or
//    contiguously (down).  Few rows per expert leave few items, and the split
//    keeps enough loads in flight; unlike a split over workgroups it needs no
//    partial sums in memory and no extra kernel to add them.
//  * The waves' partial sums meet in LDS and are added in ascending wave
//    order (deterministic).  Gate-up then writes h = SiLU(gate) * up: bf16,
//    or on fp8 the fp32 values for the requantisation pass, which finds
//    each row's amax from the row (folding it here with atomics cost about
//    8% of the gate-up time).
//    Down writes bf16 rows; on fp8 only the weight column scale is applied
//    there and the row scale by the top-k reduction.
//  * Per-item metadata (task record, token indices, fp8 scales) comes from
//    scalar loads.
//  * MXFP8 (MX): every 32 K values of a row carry their own e8m0 scale, in
//    both operands.  Each register stage is one 128-value K unit (two
//    64-byte steps), multiplied by the scaled gfx950 instruction, which
//    applies the lane's activation and weight block scales itself: lane
//    16g + r supplies the scale of row r's K block 4u + g, the dword of the
//    row's four block scales of unit u shifted to the lane's byte.  The
//    epilogue then applies no scale; gate-up writes fp32 h for the MX
//    requantisation pass.
//  * int8 w8a8 (I8): one integer instruction (v_mfma_i32_16x16x64_i8) per
//    64-byte step on the same fragments; the int32 sums become fp32 where
//    the waves' partial sums meet, and the per-channel epilogue of the fp8
//    path follows.
#include <type_traits>

#include "lds_dma.h"
#include "decode_route.h"

namespace moe {

constexpr int kStreamNB = 2;   // 16-column weight blocks per item

template <bool FP8>
__device__ __forceinline__ void stream_mfma(f32x4& acc, const u32x4& a, const u32x4& b) {
  if constexpr (FP8) {
    const i64x2 a2 = __builtin_bit_cast(i64x2, a);
    const i64x2 b2 = __builtin_bit_cast(i64x2, b);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[0], b2[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[1], b2[1], acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
}

// MB 16-row blocks per task tile, W waves per workgroup (K slices), U
// 64-byte K steps per register stage, NB weight blocks per item: 2, or 4
// (gate-up: two gate and two up blocks, down: 64 columns), halving the
// re-reads of the tile's token rows: MX and int8 w8a8 on 64-row tiles (one
// or two waves), bf16 on 32-row tiles (one, two or four waves).
// ROUTE: bf16 gate-up of a decode batch (at most 64 pairs) with the routing
// build folded in (tasks and row tokens from decode_route).
template <int MB, int W, int U, bool GATEUP, bool FP8, bool MX, bool I8, int NB = kStreamNB, bool ROUTE = false>
__global__ void __launch_bounds__(W * 64)
stream_gemm_kernel(moe_host::StreamArgs g) {
  constexpr int NH = GATEUP ? NB / 2 : NB;   // 16-column output blocks per item
  static_assert(!MX || (FP8 && U == 2), "MX stages are one 128-value K unit");
  static_assert(!I8 || (FP8 && !MX), "int8 uses the 1-byte per-channel path");
  static_assert(!ROUTE || (GATEUP && !MX), "the folded routing build serves the gate-up");
  __shared__ f32x4 red[W][MB][NB][64];   // the waves' partial sums of one item
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
  const int n_groups = g.N_out / 16 / NH;   // column groups per task
  const int total = num_tasks * n_groups;
  const size_t row_bytes = (size_t)g.K * (FP8 ? 1 : 2);
  const int nsteps = (int)(row_bytes / 64);
  const int spw = nsteps / W;            // K steps of each wave, a positive multiple of U
  const int ngroups = spw / U;
  const int w_blocks = g.w_rows / 16;
  const char* __restrict__ A = static_cast<const char*>(g.a);
  const char* __restrict__ B = static_cast<const char*>(g.b);

  // XCD-aware numbering: consecutive items (the column groups of one task)
  // on the workgroups of one XCD, sharing the task's token rows in L2.
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
    // weight 16-row blocks of this item
    int blk[NB];
    if constexpr (GATEUP) {
#pragma unroll
      for (int h = 0; h < NH; h++) {
        blk[h] = cg * NH + h;                        // gate rows [16 blk, 16 blk + 16)
        blk[NH + h] = g.N_out / 16 + cg * NH + h;    // the matching up rows
      }
    } else {
#pragma unroll
      for (int q = 0; q < NB; q++) blk[q] = cg * NB + q;
    }
    const int step0 = wave * spw;
    // Rows past the tile re-read the tile's first row: a valid address whose
    // products land only in rows that are never stored.  The loads stay
    // unconditional, so the compiler's vmcnt waits count exactly and the
    // next register stage stays in flight while this one is multiplied (a
    // load under a branch would make it wait for everything).
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
      ap[b] = A + (size_t)arow * row_bytes + (size_t)step0 * 64 + 16 * lgrp;
    }
    const char* bp[NB];
#pragma unroll
    for (int q = 0; q < NB; q++)
      bp[q] = B + (((size_t)task.expert * w_blocks + blk[q]) * nsteps + step0) * 1024 + 16 * lane;
    // MX: this lane's rows' block-scale codes, from the wave's first unit
    // (K / 32 codes per row, four per 128-value unit)
    const uint8_t* asp[MB];
    const uint8_t* bsp[NB];
    if constexpr (MX) {
      const size_t nblk = (size_t)g.K / 32;
#pragma unroll
      for (int b = 0; b < MB; b++) {
        const int rb = b * 16 < task.rows ? b : 0;
        int arow;
        if constexpr (GATEUP) {
          const i32x16_t sp = load16_scalar(g.sorted_pairs + task.row_begin + rb * 16);
          const int p = rb * 16 + lrow < task.rows ? spread16(sp, lane) : sp[0];
          arow = p / g.topk;
        } else {
          arow = task.row_begin + (rb * 16 + lrow < task.rows ? rb * 16 + lrow : 0);
        }
        asp[b] = g.a_mx + (size_t)arow * nblk + (size_t)step0 * 2;
      }
#pragma unroll
      for (int q = 0; q < NB; q++)
        bsp[q] = g.b_mx + ((size_t)task.expert * g.w_rows + blk[q] * 16 + lrow) * nblk + (size_t)step0 * 2;
    }

    f32x4 acc[MB][NB];
#pragma unroll
    for (int m = 0; m < MB; m++)
#pragma unroll
      for (int q = 0; q < NB; q++) acc[m][q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    u32x4 fa0[U][MB], fb0[U][NB], fa1[U][MB], fb1[U][NB];
    uint32_t sa0[MB], sb0[NB], sa1[MB], sb1[NB];   // MX: block-scale dwords of the stage's unit
    auto load_scales = [&](uint32_t (&sa)[MB], uint32_t (&sb)[NB], int grp) __attribute__((always_inline)) {
      if constexpr (MX) {
#pragma unroll
        for (int b = 0; b < MB; b++) sa[b] = *reinterpret_cast<const uint32_t*>(asp[b] + (size_t)grp * 4);
#pragma unroll
        for (int q = 0; q < NB; q++) sb[q] = *reinterpret_cast<const uint32_t*>(bsp[q] + (size_t)grp * 4);
      }
    };
    auto load = [&](u32x4 (&fa)[U][MB], u32x4 (&fb)[U][NB], int grp) {
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int step = grp * U + u;
#pragma unroll
        for (int q = 0; q < NB; q++)
          fb[u][q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bp[q] + (size_t)step * 1024));
#pragma unroll
        for (int b = 0; b < MB; b++) fa[u][b] = *reinterpret_cast<const u32x4*>(ap[b] + (size_t)step * 64);
      }
    };
    auto compute = [&](const u32x4 (&fa)[U][MB], const u32x4 (&fb)[U][NB], const uint32_t (&sa)[MB],
                       const uint32_t (&sb)[NB]) {
      if constexpr (MX) {
        const int sh = 8 * lgrp;   // the lane's block within the unit
#pragma unroll
        for (int b = 0; b < MB; b++)
#pragma unroll
          for (int q = 0; q < NB; q++)
            mfma_mx_k128(acc[b][q], fa[0][b], fa[1][b], fb[0][q], fb[1][q], (int)(sa[b] >> sh),
                         (int)(sb[q] >> sh));
      } else if constexpr (I8) {
        typedef int i32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int u = 0; u < U; u++)
#pragma unroll
          for (int b = 0; b < MB; b++)
#pragma unroll
            for (int q = 0; q < NB; q++)
              acc[b][q] = __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, fa[u][b]),
                                                              __builtin_bit_cast(i32x4, fb[u][q]),
                                                              __builtin_bit_cast(i32x4, acc[b][q]), 0, 0, 0));
      } else {
#pragma unroll
        for (int u = 0; u < U; u++)
#pragma unroll
          for (int b = 0; b < MB; b++)
#pragma unroll
            for (int q = 0; q < NB; q++) stream_mfma<FP8>(acc[b][q], fa[u][b], fb[u][q]);
      }
    };
    // Two register stages in turn.  No load sits under a condition: the
    // loop runs whole pairs and the tail (one stage or two) is chosen after
    // it, so each multiply waits for exactly its own stage while the next
    // one is in flight.
    load(fa0, fb0, 0);
    load_scales(sa0, sb0, 0);
    int grp = 0;
    for (; grp + 2 < ngroups; grp += 2) {
      load(fa1, fb1, grp + 1);
      load_scales(sa1, sb1, grp + 1);
      compute(fa0, fb0, sa0, sb0);
      load(fa0, fb0, grp + 2);
      load_scales(sa0, sb0, grp + 2);
      compute(fa1, fb1, sa1, sb1);
    }
    if (grp + 1 < ngroups) {
      load(fa1, fb1, grp + 1);
      load_scales(sa1, sb1, grp + 1);
      compute(fa0, fb0, sa0, sb0);
      compute(fa1, fb1, sa1, sb1);
    } else {
      compute(fa0, fb0, sa0, sb0);
    }

    // ---- the waves' partial sums meet in LDS (lane-contiguous 16-byte slots)
#pragma unroll
    for (int m = 0; m < MB; m++)
#pragma unroll
      for (int q = 0; q < NB; q++) {
        if constexpr (I8) {   // int32 sums (|sum| <= 127^2 K < 2^31) to fp32
          typedef int i32x4 __attribute__((ext_vector_type(4)));
          red[wave][m][q][lane] = __builtin_convertvector(__builtin_bit_cast(i32x4, acc[m][q]), f32x4);
        } else {
          red[wave][m][q][lane] = acc[m][q];
        }
      }
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
      float cs[NB];   // fp8: this lane's weight column scales
      float rs[4];    // fp8 gate-up: activation scales of this lane's four rows
#pragma unroll
      for (int q = 0; q < NB; q++) cs[q] = 1.0f;
#pragma unroll
      for (int i = 0; i < 4; i++) rs[i] = 1.0f;
      if constexpr (FP8 && !MX) {
#pragma unroll
        for (int q = 0; q < NB; q++) {
          const i32x16_t v = load16_scalar(g.b_scale + (size_t)task.expert * g.w_rows + blk[q] * 16);
          cs[q] = __int_as_float(spread16(v, lane));
        }
        if constexpr (GATEUP) {
          const int rb = m * 16 < task.rows ? m : 0;
          const i32x16_t v = load16_scalar(g.row_scale + task.row_begin + rb * 16);
          const float mine = __int_as_float(spread16(v, lane));
#pragma unroll
          for (int i = 0; i < 4; i++) rs[i] = __shfl(mine, 4 * lgrp + i, 64);
        }
      }
      if constexpr (GATEUP) {
#pragma unroll
        for (int h = 0; h < NH; h++) {
          const int col = blk[h] * 16 + lrow;
          float hv[4];
#pragma unroll
          for (int i = 0; i < 4; i++) {
            float gv = tot[h][i], uv = tot[NH + h][i];
            if constexpr (FP8 && !MX) {
              gv = (gv * rs[i]) * cs[h];
              uv = (uv * rs[i]) * cs[NH + h];
            }
            hv[i] = silu_f32(gv) * uv;
          }
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int rr = m * 16 + 4 * lgrp + i;
            if (rr < task.rows) {
              const size_t r = (size_t)(task.row_begin + rr);
              if constexpr (FP8) static_cast<float*>(g.c)[r * g.N_out + col] = hv[i];
              else static_cast<uint16_t*>(g.c)[r * g.N_out + col] = f32_to_bf16_bits(hv[i]);
            }
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int rr = m * 16 + 4 * lgrp + i;
          if (rr < task.rows) {
            const size_t r = (size_t)(task.row_begin + rr);
#pragma unroll
            for (int q = 0; q < NB; q++) {
              const int col = blk[q] * 16 + lrow;
              static_cast<uint16_t*>(g.c)[r * g.N_out + col] = f32_to_bf16_bits(tot[q][i] * cs[q]);
            }
          }
        }
      }
    }
    __syncthreads();   // LDS free for the next item
  }
}

// bf16 gate-up with half-width items (decode): item = (16-row task tile, 8
// h columns), its 16-row weight block made of 8 gate rows and the matching
// 8 up rows, so twice as many items of half the bytes spread evenly when
// the full-width count leaves CUs with one more item than others (e.g. 384
// items on 256 CUs).  Lanes of weight rows 0-7 read gate rows, 8-15 the up
// rows (half of a packed 16-row chunk each); in the epilogue lane c (c < 8)
// takes the up sum of lane c + 8 and writes h column 8 * item + c.
// ROUTE: a decode batch (at most 64 pairs) with the routing build folded in.
template <int W, bool ROUTE = false>
__global__ void __launch_bounds__(W * 64)
stream_half_gateup_kernel(moe_host::StreamArgs g) {
  constexpr int U = 2;
  __shared__ f32x4 red[W][64];
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
  const int n_groups = g.N_out / 8;
  const int total = num_tasks * n_groups;
  const size_t row_bytes = (size_t)g.K * 2;
  const int nsteps = (int)(row_bytes / 64);
  const int spw = nsteps / W;
  const int ngroups = spw / U;
  const int w_blocks = g.w_rows / 16;
  const char* __restrict__ A = static_cast<const char*>(g.a);
  const char* __restrict__ B = static_cast<const char*>(g.b);

  const int G = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd = G / 8, extra = G % 8;
  const int vid = (xcd < extra ? xcd * (per_xcd + 1) : extra * (per_xcd + 1) + (xcd - extra) * per_xcd) + slot;

  for (int item = vid; item < total; item += G) {
    const int ti = item / n_groups;
    const int c8 = item - ti * n_groups;
    moe_task_t task;
    if constexpr (ROUTE) task = decode_task(rt, ti, g.route.block_m);
    else task = load_task_scalar(g.tasks + ti);
    const int step0 = wave * spw;
    // this lane's weight row: gate row 8 c8 + lrow, or up row I + 8 c8 + (lrow - 8)
    const int wrow = lrow < 8 ? 8 * c8 + lrow : g.N_out + 8 * c8 + (lrow - 8);
    const char* bp = B + (((size_t)task.expert * w_blocks + wrow / 16) * nsteps + step0) * 1024 +
                     16 * ((wrow & 15) + 16 * lgrp);
    int arow;
    if constexpr (ROUTE) {
      arow = decode_sorted_pair(rt, task.row_begin + (lrow < task.rows ? lrow : 0)) / g.topk;
    } else {
      const i32x16_t sp = load16_scalar(g.sorted_pairs + task.row_begin);
      const int p = lrow < task.rows ? spread16(sp, lane) : sp[0];
      arow = p / g.topk;
    }
    const char* ap = A + (size_t)arow * row_bytes + (size_t)step0 * 64 + 16 * lgrp;

    f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    u32x4 fa0[U], fb0[U], fa1[U], fb1[U];
    auto load = [&](u32x4 (&fa)[U], u32x4 (&fb)[U], int grp) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int step = grp * U + u;
        fb[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bp + (size_t)step * 1024));
        fa[u] = *reinterpret_cast<const u32x4*>(ap + (size_t)step * 64);
      }
    };
    auto compute = [&](const u32x4 (&fa)[U], const u32x4 (&fb)[U]) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < U; u++) stream_mfma<false>(acc, fa[u], fb[u]);
    };
    load(fa0, fb0, 0);
    int grp = 0;
    for (; grp + 2 < ngroups; grp += 2) {
      load(fa1, fb1, grp + 1);
      compute(fa0, fb0);
      load(fa0, fb0, grp + 2);
      compute(fa1, fb1);
    }
    if (grp + 1 < ngroups) {
      load(fa1, fb1, grp + 1);
      compute(fa0, fb0);
      compute(fa1, fb1);
    } else {
      compute(fa0, fb0);
    }

    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
      f32x4 tot = red[0][lane];
#pragma unroll
      for (int s2 = 1; s2 < W; s2++) tot += red[s2][lane];
      // lane holds weight row lrow (gate for lrow < 8) and token rows 4 lgrp + i
      f32x4 up;
#pragma unroll
      for (int i = 0; i < 4; i++) up[i] = __shfl(tot[i], (lane & 48) | ((lrow + 8) & 15), 64);
      if (lrow < 8) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int rr = 4 * lgrp + i;
          if (rr < task.rows)
            static_cast<uint16_t*>(g.c)[(size_t)(task.row_begin + rr) * g.N_out + 8 * c8 + lrow] =
                f32_to_bf16_bits(silu_f32(tot[i]) * up[i]);
        }
      }
    }
    __syncthreads();   // LDS free for the next item
  }
}

// Down GEMM and top-k weighted sum of a single token in one launch (decode):
// out[c] = sum over the token's sorted rows r of w_r * (h_r . W2[e_r][:, c])
// (fp8: each product also times the row's activation scale and its
// expert's column scale).
//  * Item = 16 output columns (HALF: 8), one per workgroup.  Its reduction
//    runs over the concatenation of the token's experts (every task's K
//    steps in turn), cut into equal runs of whole register stages, one per
//    wave; the waves' sums meet in LDS, so the top-k sum needs neither a
//    second launch nor partial rows in memory.
//  * One token has at most 16 pairs, so the A tile's row r is sorted row r
//    at every step, zeroed unless r belongs to the step's task: accumulator
//    row r collects only the products of its own expert's weights, and the
//    epilogue weights each row and adds the rows of each column.
//  * HALF (at most 8 pairs): twice the items at half the bytes each.  One
//    instruction covers two K steps of the item's 8 columns: B columns 0-7
//    take the columns from step 2m, columns 8-15 the same columns from step
//    2m + 1, and A rows 0-7 / 8-15 the token's rows at those two steps; the
//    two diagonal 8 x 8 quarters of the product are the useful ones, and
//    column c of the item is the sum of accumulator columns c and c + 8.
//  * Task records go to LDS first; the per-row weights and scales are loaded
//    before the weight stream starts and used after it.
//  * I8 (int8 w8a8, with FP8 set: the same one-byte layout and scales): one
//    v_mfma_i32_16x16x64_i8 per 16-byte fragment pair, int32 sums turned to
//    fp32 where the waves' sums meet.
template <int W, int U, bool HALF, bool FP8, bool I8 = false>
__global__ void __launch_bounds__(W * 64)
stream_down_reduce_kernel(moe_host::StreamArgs g, const float* __restrict__ topk_w,
                          const float* __restrict__ h_scale, uint16_t* __restrict__ out) {
#pragma clang fp contract(off)
  static_assert(!I8 || FP8, "int8 uses the one-byte per-channel layout");
  constexpr int KS = HALF ? 2 : 1;   // 64-byte K steps per instruction step
  __shared__ f32x4 red[W][64];
  __shared__ moe_task_t tk[16];
  const int lane = threadIdx.x & 63;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (threadIdx.x < 16 && (int)threadIdx.x < g.max_tasks) tk[threadIdx.x] = g.tasks[threadIdx.x];
  const int nt = min(min(g.header[kHdrNumTasks], g.max_tasks), 16);
  const i32x16_t sp = load16_scalar(g.sorted_pairs);
  __syncthreads();

  const size_t row_bytes = (size_t)g.K * (FP8 ? 1 : 2);
  const int nsteps = (int)(row_bytes / 64);
  const int nm = nsteps / KS;                  // instruction steps per task, a multiple of U
  const int total = nt * nm;
  int spw = (total + W - 1) / W;
  spw = (spw + U - 1) / U * U;
  const int s0 = min(total, wave * spw);
  const int ngroups = (min(total, s0 + spw) - s0) / U;
  // this lane's A row (a sorted row) and K step within the instruction
  // step, and its offset in a packed 1 KiB weight chunk
  const int arow = HALF ? (lrow & 7) : lrow;
  const int ksub = HALF ? (lrow >> 3) : 0;
  const int cb = HALF ? (int)(blockIdx.x >> 1) : (int)blockIdx.x;   // 16-column weight block
  const int col0 = HALF ? 8 * (int)blockIdx.x : 16 * (int)blockIdx.x;
  const int boff = HALF ? 16 * (lgrp * 16 + (blockIdx.x & 1) * 8 + (lrow & 7)) : 16 * lane;
  const char* __restrict__ A = static_cast<const char*>(g.a);
  const char* __restrict__ B = static_cast<const char*>(g.b);
  const size_t expert_bytes = (size_t)(g.w_rows / 16) * nsteps * 1024;
  const char* bcol = B + ((size_t)cb * nsteps + ksub) * 1024 + boff;

  // Accumulator rows 4 lgrp + i of this lane's column: the sorted row each
  // holds, its weight w_r (times the row scale on fp8; 0 for rows outside
  // every task, dropped pairs and rows past the token's pairs, and for the
  // off-diagonal quarters of HALF) and its expert's scale of the lane's
  // output column.
  const int ocol = col0 + (HALF ? (lrow & 7) : lrow);
  float wr[4], cs[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int r = HALF ? ((4 * lgrp + i) & 7) : 4 * lgrp + i;
    const bool diag = !HALF || ((lrow < 8) == (lgrp < 2));
    int e = -1;
    for (int t = 0; t < nt; t++)
      if ((unsigned)(r - tk[t].row_begin) < (unsigned)tk[t].rows) e = tk[t].expert;
    // the loads stay unconditional (entry 0 when the row is unused)
    const bool use = e >= 0 && diag;
    const float w = topk_w[use ? pick16(sp, r) : 0];
    wr[i] = use ? w : 0.0f;
    cs[i] = 1.0f;
    if constexpr (FP8) {
      const float rs = h_scale[use ? r : 0];
      const float c = g.b_scale[(size_t)(use ? e : 0) * g.w_rows + ocol];
      wr[i] = wr[i] * rs;
      cs[i] = c;
    }
  }

  f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  u32x4 fa0[U], fb0[U], fa1[U], fb1[U];
  bool in0 = false, in1 = false;
  auto load = [&](u32x4 (&fa)[U], u32x4 (&fb)[U], bool& in, int grp) __attribute__((always_inline)) {
    const int s = s0 + grp * U;
    const int t = s / nm;
    const int ks = (s - t * nm) * KS;   // first 64-byte step of the stage
    const moe_task_t task = tk[t];
    in = (unsigned)(arow - task.row_begin) < (unsigned)task.rows;
    // lanes of other rows read the task's first row (one line per step) and drop it
    const char* ap = A + (size_t)(in ? arow : task.row_begin) * row_bytes + (size_t)(ks + ksub) * 64 + 16 * lgrp;
    const char* bp = bcol + (size_t)task.expert * expert_bytes + (size_t)ks * 1024;
#pragma unroll
    for (int u = 0; u < U; u++) {
      fb[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bp + (size_t)u * KS * 1024));
      fa[u] = *reinterpret_cast<const u32x4*>(ap + (size_t)u * KS * 64);
    }
  };
  auto compute = [&](const u32x4 (&fa)[U], const u32x4 (&fb)[U], bool in) __attribute__((always_inline)) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < U; u++) {
      if constexpr (I8) {
        typedef int i32x4 __attribute__((ext_vector_type(4)));
        acc = __builtin_bit_cast(f32x4, __builtin_amdgcn_mfma_i32_16x16x64_i8(
                                            __builtin_bit_cast(i32x4, in ? fa[u] : zero),
                                            __builtin_bit_cast(i32x4, fb[u]), __builtin_bit_cast(i32x4, acc), 0, 0, 0));
      } else {
        stream_mfma<FP8>(acc, in ? fa[u] : zero, fb[u]);
      }
    }
  };
  if (ngroups > 0) {
    load(fa0, fb0, in0, 0);
    int grp = 0;
    for (; grp + 2 < ngroups; grp += 2) {
      load(fa1, fb1, in1, grp + 1);
      compute(fa0, fb0, in0);
      load(fa0, fb0, in0, grp + 2);
      compute(fa1, fb1, in1);
    }
    if (grp + 1 < ngroups) {
      load(fa1, fb1, in1, grp + 1);
      compute(fa0, fb0, in0);
      compute(fa1, fb1, in1);
    } else {
      compute(fa0, fb0, in0);
    }
  }

  if constexpr (I8) {   // int32 sums (|sum| <= 127^2 K < 2^31) to fp32
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    red[wave][lane] = __builtin_convertvector(__builtin_bit_cast(i32x4, acc), f32x4);
  } else {
    red[wave][lane] = acc;
  }
  __syncthreads();
  if (wave == 0) {
    f32x4 tot = red[0][lane];
#pragma unroll
    for (int w = 1; w < W; w++) tot += red[w][lane];
    // weight the lane's rows, add the four row groups of the column (and on
    // HALF the two accumulator columns of each output column)
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) v = v + wr[i] * (tot[i] * cs[i]);
    v = v + __shfl_xor(v, 16, 64);
    v = v + __shfl_xor(v, 32, 64);
    if constexpr (HALF) {
      v = v + __shfl_xor(v, 8, 64);
      if (lane < 8) out[ocol] = f32_to_bf16_bits(v);
    } else {
      if (lgrp == 0) out[ocol] = f32_to_bf16_bits(v);
    }
  }
}

template <int MB, int W, int U, bool GATEUP, bool FP8, bool MX, bool I8 = false>
static hipError_t launch_stream_t(const moe_host::StreamArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((stream_gemm_kernel<MB, W, U, GATEUP, FP8, MX, I8>), dim3(grid), dim3(W * 64), 0, s, a);
  return hipGetLastError();
}

// Four weight blocks per item: MX or int8 w8a8 on 64-row tiles with one or
// two waves (kind 1, 2), bf16 on 32-row tiles with one, two or four waves
// (kind 3); two-step stages.
hipError_t launch_stream_nb4(const moe_host::StreamArgs& a, bool gateup, int kind, int waves, int grid,
                             hipStream_t s) {
#define MOE_NB4(Wv, GU, MXv, I8v) \
  hipLaunchKernelGGL((stream_gemm_kernel<4, Wv, 2, GU, true, MXv, I8v, 4>), dim3(grid), dim3(Wv * 64), 0, s, a)
  if (kind == 1) {
    if (waves == 1) { if (gateup) MOE_NB4(1, true, true, false); else MOE_NB4(1, false, true, false); }
    else if (waves == 2) { if (gateup) MOE_NB4(2, true, true, false); else MOE_NB4(2, false, true, false); }
    else return hipErrorInvalidValue;
  } else if (kind == 2) {
    if (waves == 1) { if (gateup) MOE_NB4(1, true, false, true); else MOE_NB4(1, false, false, true); }
    else if (waves == 2) { if (gateup) MOE_NB4(2, true, false, true); else MOE_NB4(2, false, false, true); }
    else return hipErrorInvalidValue;
  } else if (kind == 3) {   // bf16, 32-row tiles
#define MOE_NB4B(Wv, GU) \
  hipLaunchKernelGGL((stream_gemm_kernel<2, Wv, 2, GU, false, false, false, 4>), dim3(grid), dim3(Wv * 64), 0, s, a)
    if (waves == 1) { if (gateup) MOE_NB4B(1, true); else MOE_NB4B(1, false); }
    else if (waves == 2) { if (gateup) MOE_NB4B(2, true); else MOE_NB4B(2, false); }
    else if (waves == 4) { if (gateup) MOE_NB4B(4, true); else MOE_NB4B(4, false); }
    else return hipErrorInvalidValue;
#undef MOE_NB4B
  } else {
    return hipErrorInvalidValue;
  }
#undef MOE_NB4
  return hipGetLastError();
}

// kind: 0 per-channel (bf16 or fp8 by `fp8`), 1 MX, 2 int8
template <int MB, int W, int U>
static hipError_t launch_stream_w(const moe_host::StreamArgs& a, bool gateup, bool fp8, int kind,
                                  int grid, hipStream_t s) {
  if (a.route.ids) {   // the routing build folded in: bf16 gate-up on 16-row tiles
    if constexpr (MB == 1) {
      if (gateup && !fp8 && kind == 0) {
        hipLaunchKernelGGL((stream_gemm_kernel<MB, W, U, true, false, false, false, kStreamNB, true>), dim3(grid),
                           dim3(W * 64), 0, s, a);
        return hipGetLastError();
      }
    }
    return hipErrorInvalidValue;
  }
  if (kind == 1) {
    if constexpr (U == 2)
      return gateup ? launch_stream_t<MB, W, U, true, true, true>(a, grid, s)
                    : launch_stream_t<MB, W, U, false, true, true>(a, grid, s);
    return hipErrorInvalidValue;
  }
  if (kind == 2)
    return gateup ? launch_stream_t<MB, W, U, true, true, false, true>(a, grid, s)
                  : launch_stream_t<MB, W, U, false, true, false, true>(a, grid, s);
  if (gateup) return fp8 ? launch_stream_t<MB, W, U, true, true, false>(a, grid, s)
                         : launch_stream_t<MB, W, U, true, false, false>(a, grid, s);
  return fp8 ? launch_stream_t<MB, W, U, false, true, false>(a, grid, s)
             : launch_stream_t<MB, W, U, false, false, false>(a, grid, s);
}

}  // namespace moe

namespace moe_host {

// (16-row blocks per tile, waves per workgroup, K steps per register stage)
// built here: two-step stages for any split, one-step stages unsplit (odd
// numbers of K steps).
#define MOE_STREAM_CONFIGS(X) \
  X(1, 1, 2) X(1, 2, 2) X(1, 4, 2) X(1, 8, 2) \
  X(2, 1, 2) X(2, 2, 2) X(2, 4, 2) X(2, 8, 2) \
  X(4, 1, 2) X(4, 2, 2) X(4, 4, 2) X(4, 8, 2) \
  X(1, 1, 1) X(2, 1, 1) X(4, 1, 1)

hipError_t launch_stream_half_gateup(const StreamArgs& a, int waves, int grid, hipStream_t s) {
  switch (waves) {
#define MOE_HALF(Wv)                                                                                    \
  {                                                                                                     \
    if (a.route.ids)                                                                                    \
      hipLaunchKernelGGL((moe::stream_half_gateup_kernel<Wv, true>), dim3(grid), dim3(Wv * 64), 0, s, a); \
    else                                                                                                \
      hipLaunchKernelGGL((moe::stream_half_gateup_kernel<Wv, false>), dim3(grid), dim3(Wv * 64), 0, s, a); \
    break;                                                                                              \
  }
    case 1: MOE_HALF(1)
    case 2: MOE_HALF(2)
    case 4: MOE_HALF(4)
    case 8: MOE_HALF(8)
    default: return hipErrorInvalidValue;
  }
#undef MOE_HALF
  return hipGetLastError();
}

hipError_t launch_stream_down_reduce(const StreamArgs& a, bool fp8, int waves, int u, bool half,
                                     const float* topk_w, const float* h_scale, uint16_t* out, hipStream_t s,
                                     bool i8) {
  const int nsteps = a.K * (fp8 ? 1 : 2) / 64;
  if (a.P > (half ? 8 : 16) || nsteps % ((half ? 2 : 1) * u) || a.N_out % 16 || (i8 && !fp8))
    return hipErrorInvalidValue;
  const dim3 grid(a.N_out / (half ? 8 : 16));
#define MOE_DR(Wv, Uv, Hv)                                                                              \
  {                                                                                                     \
    if (i8)                                                                                             \
      hipLaunchKernelGGL((moe::stream_down_reduce_kernel<Wv, Uv, Hv, true, true>), grid, dim3(Wv * 64),  \
                         0, s, a, topk_w, h_scale, out);                                                \
    else if (fp8)                                                                                       \
      hipLaunchKernelGGL((moe::stream_down_reduce_kernel<Wv, Uv, Hv, true>), grid, dim3(Wv * 64), 0, s, \
                         a, topk_w, h_scale, out);                                                      \
    else                                                                                                \
      hipLaunchKernelGGL((moe::stream_down_reduce_kernel<Wv, Uv, Hv, false>), grid, dim3(Wv * 64), 0,   \
                         s, a, topk_w, h_scale, out);                                                   \
    return hipGetLastError();                                                                           \
  }
#define MOE_DR_CASE(Wv, Uv) \
  if (waves == Wv && u == Uv) { if (half) MOE_DR(Wv, Uv, true) else MOE_DR(Wv, Uv, false) }
  MOE_DR_CASE(4, 2) MOE_DR_CASE(8, 2) MOE_DR_CASE(16, 2) MOE_DR_CASE(8, 4) MOE_DR_CASE(16, 4)
#undef MOE_DR_CASE
#undef MOE_DR
  return hipErrorInvalidValue;
}

bool stream_config_supported(int mb, int waves, int u) {
#define MOE_STREAM_CASE(M, Wv, Uv) if (mb == M && waves == Wv && u == Uv) return true;
  MOE_STREAM_CONFIGS(MOE_STREAM_CASE)
#undef MOE_STREAM_CASE
  return false;
}

hipError_t launch_stream_gemm(const StreamArgs& a, bool gateup, bool fp8, int kind, int mb, int waves,
                              int u, int grid, hipStream_t s, int nb) {
  if (nb == 4) {
    if (a.route.ids) return hipErrorInvalidValue;
    if (u != 2) return hipErrorInvalidValue;
    if (kind == 0 && !fp8) return mb == 2 ? moe::launch_stream_nb4(a, gateup, 3, waves, grid, s)
                                          : hipErrorInvalidValue;
    if (mb != 4) return hipErrorInvalidValue;
    return moe::launch_stream_nb4(a, gateup, kind, waves, grid, s);
  }
#define MOE_STREAM_CASE(M, Wv, Uv) \
  if (mb == M && waves == Wv && u == Uv) return moe::launch_stream_w<M, Wv, Uv>(a, gateup, fp8, kind, grid, s);
  MOE_STREAM_CONFIGS(MOE_STREAM_CASE)
#undef MOE_STREAM_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe_host
