// Grouped expert GEMM on MFMA for the gate-up and down projections
// (HPC-Ops x SGLang blog, section "MoE": gate-up reads the original tokens
// through the route index with no separate gather; a persistent grid
// consumes the per-tile task map and spreads small, ragged expert tiles
// over the compute units; one group of lanes both loads and multiplies).
//
// Work item = (16*NSUB output columns, task tile, K slice), n-tile major so
// that the row tiles of one expert that share a weight block run side by
// side and meet its bytes in L2.  Each wave of the persistent grid takes
// items round-robin until the device-side task count is exhausted, so one
// launch size serves every routing.
//
// A wave computes a (16*MB) x (16*NSUB) block of C with
// v_mfma_f32_16x16x32_bf16 (bf16) or two v_mfma_f32_16x16x32_fp8_fp8 per
// 64-byte step (fp8).  Lane l holds row (l % 16) of its 16-row block and
// the 16 bytes at offset 16*(l / 16) of each 64-byte K step.
//
// Weights arrive pre-packed (moe_pack_weights): every 16-row x 64-byte
// block is one contiguous 1 KiB chunk in exactly that lane order, and the
// chunks of a 16-row block follow each other along K.  A wave's weight
// loads are therefore whole 1 KiB lines, and a work item streams one
// contiguous run of its expert's weights with non-temporal loads (read
// once, kept out of the caches' way).  Token rows are read through the
// route index (gate-up) or contiguously (down) with ordinary loads; they
// are small and shared by many items through L2.  Two register stages of
// UNROLL steps keep the next loads in flight while the previous ones are
// multiplied.
//
// The K dimension may be split into S slices (split-K) to put enough loads
// in flight when there are few tasks (decode); slice s writes its fp32
// partial sums to c[s][row][col] and the consumer kernel adds the slices in
// ascending order, so the result is deterministic.
#include "moe_common.h"

namespace moe {

template <bool FP8>
__device__ __forceinline__ void mfma_step(f32x4& acc, const u32x4& a, const u32x4& b) {
  if constexpr (FP8) {
    // bytes 0..7 and 8..15 of the fragment feed two consecutive MFMAs
    const i64x2 a2 = __builtin_bit_cast(i64x2, a);
    const i64x2 b2 = __builtin_bit_cast(i64x2, b);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[0], b2[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[1], b2[1], acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
}

template <int MB, int NSUB, int UNROLL, bool GATHER, bool FP8>
__global__ void __launch_bounds__(256)
grouped_gemm_kernel(moe_host::GemmArgs g) {
  const int lane = threadIdx.x & 63;
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  const int n_tiles = g.N / (16 * NSUB);
  const int num_tasks = min(g.header[kHdrNumTasks], g.max_tasks);
  const int S = g.split;
  const int total = num_tasks * n_tiles * S;
  const size_t row_bytes = (size_t)g.K * (FP8 ? 1 : 2);
  const int steps_per_slice = (int)(row_bytes / 64) / S;   // multiple of UNROLL
  const int ngroups = steps_per_slice / UNROLL;
  const char* __restrict__ A = static_cast<const char*>(g.a);
  const char* __restrict__ B = static_cast<const char*>(g.b);

  const int nsteps = (int)(row_bytes / 64);
  for (int item = wave; item < total; item += nwaves) {
    const int s = item % S;
    const int rest = item / S;
    const int ti = rest % num_tasks;
    const int nt = rest / num_tasks;
    const moe_task_t task = g.tasks[ti];
    const int n0 = nt * 16 * NSUB;
    const int step0 = s * steps_per_slice;
    const size_t k_off = (size_t)step0 * 64 + 16 * lgrp;

    const char* ap[MB];
    bool aok[MB];
#pragma unroll
    for (int b = 0; b < MB; b++) {
      const int rr = 16 * b + lrow;
      aok[b] = rr < task.rows;
      int arow = 0;
      if (aok[b]) arow = GATHER ? g.sorted_pairs[task.row_begin + rr] / g.topk : task.row_begin + rr;
      ap[b] = A + (size_t)arow * row_bytes + k_off;
    }
    // packed weights: chunk (expert, 16-row block, step) of 1 KiB, lane-ordered
    const char* bp[NSUB];
#pragma unroll
    for (int q = 0; q < NSUB; q++)
      bp[q] = B + (((size_t)task.expert * (g.N / 16) + n0 / 16 + q) * nsteps + step0) * 1024 +
              16 * lane;

    f32x4 acc[MB][NSUB];
#pragma unroll
    for (int b = 0; b < MB; b++)
#pragma unroll
      for (int q = 0; q < NSUB; q++) acc[b][q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    u32x4 fa0[UNROLL][MB], fb0[UNROLL][NSUB];
    u32x4 fa1[UNROLL][MB], fb1[UNROLL][NSUB];

    auto load = [&](u32x4(&fa)[UNROLL][MB], u32x4(&fb)[UNROLL][NSUB], int grp) {
#pragma unroll
      for (int u = 0; u < UNROLL; u++) {
        const int step = grp * UNROLL + u;
        const size_t off = (size_t)step * 64;
#pragma unroll
        for (int q = 0; q < NSUB; q++)
          fb[u][q] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(bp[q] + (size_t)step * 1024));
#pragma unroll
        for (int b = 0; b < MB; b++)
          fa[u][b] = aok[b] ? *reinterpret_cast<const u32x4*>(ap[b] + off) : u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto compute = [&](const u32x4(&fa)[UNROLL][MB], const u32x4(&fb)[UNROLL][NSUB]) {
#pragma unroll
      for (int u = 0; u < UNROLL; u++)
#pragma unroll
        for (int b = 0; b < MB; b++)
#pragma unroll
          for (int q = 0; q < NSUB; q++) mfma_step<FP8>(acc[b][q], fa[u][b], fb[u][q]);
    };

    load(fa0, fb0, 0);
    for (int grp = 0; grp < ngroups; grp += 2) {
      if (grp + 1 < ngroups) load(fa1, fb1, grp + 1);
      compute(fa0, fb0);
      if (grp + 1 < ngroups) {
        if (grp + 2 < ngroups) load(fa0, fb0, grp + 2);
        compute(fa1, fb1);
      }
    }

    // Epilogue: lane l holds column (l % 16) of each 16-column block and rows
    // 4*(l / 16) + i of each 16-row block.
    float* __restrict__ C = g.c + (size_t)s * g.P * g.N;
#pragma unroll
    for (int b = 0; b < MB; b++) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int rr = 16 * b + 4 * lgrp + i;
        if (rr < task.rows) {
          const int r = task.row_begin + rr;
          float as = 1.0f;
          if constexpr (FP8) as = g.a_scale[GATHER ? g.sorted_pairs[r] / g.topk : r];
#pragma unroll
          for (int q = 0; q < NSUB; q++) {
            const int col = n0 + 16 * q + lrow;
            float v = acc[b][q][i];
            if constexpr (FP8) v = (v * as) * g.b_scale[(size_t)task.expert * g.N + col];
            C[(size_t)r * g.N + col] = v;
          }
        }
      }
    }
  }
}

template <bool GATHER, bool FP8, int MB>
static hipError_t launch_mb(const moe_host::GemmArgs& a, const moe_host::GemmPlan& p,
                            hipStream_t s) {
  const dim3 grid(p.grid), block(256);
  if (p.nsub != 1) return hipErrorInvalidValue;
  switch (p.unroll) {
    case 1: hipLaunchKernelGGL((grouped_gemm_kernel<MB, 1, 1, GATHER, FP8>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((grouped_gemm_kernel<MB, 1, 2, GATHER, FP8>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((grouped_gemm_kernel<MB, 1, 4, GATHER, FP8>), grid, block, 0, s, a); break;
    case 8:
      if constexpr (MB == 1) {
        hipLaunchKernelGGL((grouped_gemm_kernel<MB, 1, 8, GATHER, FP8>), grid, block, 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool GATHER, bool FP8>
static hipError_t launch_gf(const moe_host::GemmArgs& a, const moe_host::GemmPlan& p,
                            hipStream_t s) {
  switch (p.mb) {
    case 1: return launch_mb<GATHER, FP8, 1>(a, p, s);
    case 2: return launch_mb<GATHER, FP8, 2>(a, p, s);
    case 4: return launch_mb<GATHER, FP8, 4>(a, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe

namespace moe_host {

hipError_t launch_grouped_gemm(const GemmArgs& a, bool gather, bool fp8, const GemmPlan& plan,
                               hipStream_t s) {
  if (gather) return fp8 ? moe::launch_gf<true, true>(a, plan, s) : moe::launch_gf<true, false>(a, plan, s);
  return fp8 ? moe::launch_gf<false, true>(a, plan, s) : moe::launch_gf<false, false>(a, plan, s);
}

}  // namespace moe_host
