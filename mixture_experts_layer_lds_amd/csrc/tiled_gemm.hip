// LDS-tiled grouped expert GEMM for large token counts (many rows per
// expert), where the layer turns from HBM-bound to MFMA-bound.
//
// Same pipeline role as stream_gemm.hip (HPC-Ops x SGLang blog, section
// "MoE": gate-up reads tokens through the route index, persistent grid over
// the task map), but each workgroup owns a BM x BN output tile of one task
// and stages its operands through LDS, so every A row and weight column is
// fetched once per tile and reused by several waves.
//
//  * 256 threads = 2 x 2 waves; each wave computes (BM/2) x (BN/2) with
//    v_mfma_f32_16x16x32_bf16 (or two fp8 MFMAs per 64-byte step).
//  * One K iteration covers 128 bytes of every row (two 64-byte steps).
//    LDS holds the A and B tiles of an iteration in 1 KiB chunks laid out
//    in MFMA lane order (piece l of a chunk = row l % 16, bytes 16*(l/16)),
//    the same order the weights are packed in, so weight chunks are copied
//    verbatim and every fragment read is a conflict-free, lane-contiguous
//    128-bit LDS read.  Two LDS stages: the next iteration's global loads
//    are in flight while the current one is multiplied.
//  * Gate-up mode pairs gate and up column blocks inside each wave (wave
//    column half c holds gate blocks and the matching up blocks), so
//    SiLU(gate)*up is formed in registers in the epilogue and the fp32 gate/
//    up sums never reach memory.  The bf16 path stores h in bf16; the fp8
//    path stores h in fp32 and folds each row's amax into h_scale with an
//    atomic max on the (non-negative) float bits, which is order-independent;
//    a small kernel then requantises the rows.
//  * Down mode stores the unweighted rows y in bf16 for the top-k reduction.
//  * Work items (task, n-tile) are handed out XCD-aware: consecutive items
//    go to workgroups of the same XCD, so the A rows of a task and the
//    weight block of an expert are shared through one L2.
#include "lds_dma.h"

namespace moe {

constexpr int kTileThreads = 256;
constexpr int kIterSteps = 2;   // 64-byte K steps per K iteration

template <int BM, int BN>
struct TileShape {
  static constexpr int kWM = BM / 2, kWN = BN / 2;
  static constexpr int kMB = kWM / 16, kNB = kWN / 16;
  static constexpr int kAChunks = BM / 16 * kIterSteps;
  static constexpr int kBChunks = BN / 16 * kIterSteps;
  static constexpr int kAPieces = kAChunks * 64 / kTileThreads;
  static constexpr int kBPieces = kBChunks * 64 / kTileThreads;
  static constexpr int kStageBytes = (kAChunks + kBChunks) * 1024;
};

template <bool FP8>
__device__ __forceinline__ void mfma_step_t(f32x4& acc, const u32x4& a, const u32x4& b) {
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

template <int BM, int BN, bool GATEUP, bool FP8>
__global__ void __launch_bounds__(kTileThreads, 2)
tiled_gemm_kernel(moe_host::TiledArgs g) {
  using S = TileShape<BM, BN>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int num_tasks = min(g.header[kHdrNumTasks], g.max_tasks);
  // gate-up: each tile covers BN/2 output columns of h (BN/2 gate + BN/2 up rows of W1)
  const int out_cols = GATEUP ? BN / 2 : BN;
  const int n_tiles = g.N_out / out_cols;
  const int total = num_tasks * n_tiles;
  const size_t row_bytes = (size_t)g.K * (FP8 ? 1 : 2);
  const int nsteps = (int)(row_bytes / 64);
  const int nk = (nsteps + kIterSteps - 1) / kIterSteps;
  const int w_blocks = g.w_rows / 16;   // 16-row blocks per expert in the packed weights
  const char* __restrict__ A = static_cast<const char*>(g.a);
  const char* __restrict__ B = static_cast<const char*>(g.b);

  // XCD-aware order: workgroups are dispatched round-robin over 8 XCDs, so
  // renumber them to give each XCD a contiguous run of items.
  const int G = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd = G / 8, extra = G % 8;
  const int vid = (xcd < extra ? xcd * (per_xcd + 1) : extra * (per_xcd + 1) + (xcd - extra) * per_xcd) + slot;

  for (int item = vid; item < total; item += G) {
    const int ti = item / n_tiles;
    const int nt = item - ti * n_tiles;
    const moe_task_t task = g.tasks[ti];

    // --- per-thread global sources of its A and B pieces
    const char* asrc[S::kAPieces];
    bool aok[S::kAPieces];
    int ast[S::kAPieces];
#pragma unroll
    for (int i = 0; i < S::kAPieces; i++) {
      const int p = tid + kTileThreads * i;
      const int c = p >> 6, l = p & 63;
      const int rb = c / kIterSteps;
      ast[i] = c % kIterSteps;
      const int rr = rb * 16 + (l & 15);
      aok[i] = rr < task.rows;
      int arow = 0;
      if (aok[i]) arow = GATEUP ? g.sorted_pairs[task.row_begin + rr] / g.topk : task.row_begin + rr;
      asrc[i] = A + (size_t)arow * row_bytes + ast[i] * 64 + 16 * (l >> 4);
    }
    const char* bsrc[S::kBPieces];
    int bst[S::kBPieces];
#pragma unroll
    for (int i = 0; i < S::kBPieces; i++) {
      const int p = tid + kTileThreads * i;
      const int c = p >> 6, l = p & 63;
      const int j = c / kIterSteps;   // 16-row block of the tile's weight rows
      bst[i] = c % kIterSteps;
      int wrb;
      if (GATEUP) {
        const int half = BN / 32;
        wrb = (j < half) ? (nt * half + j) : (g.N_out / 16 + nt * half + (j - half));
      } else {
        wrb = nt * (BN / 16) + j;
      }
      bsrc[i] = B + (((size_t)task.expert * w_blocks + wrb) * nsteps + bst[i]) * 1024 + 16 * l;
    }

    u32x4 ra[S::kAPieces], rb_[S::kBPieces];
    auto gload = [&](int kt) {
#pragma unroll
      for (int i = 0; i < S::kAPieces; i++) {
        const bool ok = aok[i] && (kt * kIterSteps + ast[i] < nsteps);
        ra[i] = ok ? *reinterpret_cast<const u32x4*>(asrc[i] + (size_t)kt * 128) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < S::kBPieces; i++) {
        const bool ok = kt * kIterSteps + bst[i] < nsteps;
        rb_[i] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                          bsrc[i] + (size_t)kt * kIterSteps * 1024))
                    : u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto lstore = [&](int stage) {
      char* base = lds + stage * S::kStageBytes;
#pragma unroll
      for (int i = 0; i < S::kAPieces; i++)
        *reinterpret_cast<u32x4*>(base + (size_t)(tid + kTileThreads * i) * 16) = ra[i];
#pragma unroll
      for (int i = 0; i < S::kBPieces; i++)
        *reinterpret_cast<u32x4*>(base + S::kAChunks * 1024 + (size_t)(tid + kTileThreads * i) * 16) = rb_[i];
    };

    f32x4 acc[S::kMB][S::kNB];
#pragma unroll
    for (int m = 0; m < S::kMB; m++)
#pragma unroll
      for (int q = 0; q < S::kNB; q++) acc[m][q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // LDS chunk index of this wave's q-th weight block
    auto bblock = [&](int q) {
      if (GATEUP) {
        const int half = S::kNB / 2;
        return q < half ? (wn * half + q) : (BN / 32 + wn * half + (q - half));
      }
      return wn * S::kNB + q;
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
      const int cur = kt & 1;
      if (kt + 1 < nk) gload(kt + 1);
      const char* base = lds + cur * S::kStageBytes;
      if constexpr (FP8) {
        // both K steps of the iteration in one full-rate fp8 instruction
        static_assert(kIterSteps == 2, "fp8 pairs the two steps of an iteration");
        u32x4 fa[S::kMB][2], fb[S::kNB][2];
#pragma unroll
        for (int st = 0; st < 2; st++) {
#pragma unroll
          for (int m = 0; m < S::kMB; m++)
            fa[m][st] = *reinterpret_cast<const u32x4*>(base + ((wm * S::kMB + m) * kIterSteps + st) * 1024 + 16 * lane);
#pragma unroll
          for (int q = 0; q < S::kNB; q++)
            fb[q][st] = *reinterpret_cast<const u32x4*>(base + S::kAChunks * 1024 +
                                                        (bblock(q) * kIterSteps + st) * 1024 + 16 * lane);
        }
#pragma unroll
        for (int m = 0; m < S::kMB; m++)
#pragma unroll
          for (int q = 0; q < S::kNB; q++)
            mfma_fp8_k128(acc[m][q], fa[m][0], fa[m][1], fb[q][0], fb[q][1]);
      } else {
#pragma unroll
        for (int st = 0; st < kIterSteps; st++) {
          u32x4 fa[S::kMB], fb[S::kNB];
#pragma unroll
          for (int m = 0; m < S::kMB; m++)
            fa[m] = *reinterpret_cast<const u32x4*>(base + ((wm * S::kMB + m) * kIterSteps + st) * 1024 + 16 * lane);
#pragma unroll
          for (int q = 0; q < S::kNB; q++)
            fb[q] = *reinterpret_cast<const u32x4*>(base + S::kAChunks * 1024 +
                                                    (bblock(q) * kIterSteps + st) * 1024 + 16 * lane);
#pragma unroll
          for (int m = 0; m < S::kMB; m++)
#pragma unroll
            for (int q = 0; q < S::kNB; q++) mfma_step_t<FP8>(acc[m][q], fa[m], fb[q]);
        }
      }
      if (kt + 1 < nk) lstore(cur ^ 1);
      __syncthreads();
    }

    // --- epilogue: lane holds column (lane % 16) and rows 4*(lane/16)+i of each block
    const int lrow = lane & 15, lgrp = lane >> 4;
#pragma unroll
    for (int m = 0; m < S::kMB; m++) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int rr = wm * S::kWM + m * 16 + 4 * lgrp + i;
        const bool ok = rr < task.rows;
        const int r = task.row_begin + (ok ? rr : 0);
        if constexpr (GATEUP) {
          constexpr int half = S::kNB / 2;
          float sx = 1.0f;
          if constexpr (FP8) sx = ok ? g.a_scale[g.sorted_pairs[r] / g.topk] : 0.0f;
          float rmax = 0.0f;
#pragma unroll
          for (int q = 0; q < half; q++) {
            const int col = nt * (BN / 2) + wn * half * 16 + q * 16 + lrow;
            float gv = acc[m][q][i], uv = acc[m][q + half][i];
            if constexpr (FP8) {
              gv = (gv * sx) * g.b_scale[(size_t)task.expert * g.w_rows + col];
              uv = (uv * sx) * g.b_scale[(size_t)task.expert * g.w_rows + g.N_out + col];
            }
            const float hv = silu_f32(gv) * uv;
            if (ok) {
              if constexpr (FP8) {
                static_cast<float*>(g.c)[(size_t)r * g.N_out + col] = hv;
              } else {
                static_cast<uint16_t*>(g.c)[(size_t)r * g.N_out + col] = f32_to_bf16_bits(hv);
              }
            }
            rmax = __builtin_fmaxf(rmax, __builtin_fabsf(hv));
          }
          if constexpr (FP8) {
            rmax = max16(rmax);
            if (ok && lrow == 0)
              atomicMax(reinterpret_cast<unsigned int*>(g.row_amax) + r, __float_as_uint(rmax));
          }
        } else {
          float sa = 1.0f;
          if constexpr (FP8) sa = ok ? g.a_scale[r] : 0.0f;
#pragma unroll
          for (int q = 0; q < S::kNB; q++) {
            const int col = nt * BN + wn * S::kWN + q * 16 + lrow;
            float v = acc[m][q][i];
            if constexpr (FP8) v = (v * sa) * g.b_scale[(size_t)task.expert * g.w_rows + col];
            if (ok) static_cast<uint16_t*>(g.c)[(size_t)r * g.N_out + col] = f32_to_bf16_bits(v);
          }
        }
      }
    }
  }
}

template <int BM, int BN, bool GATEUP, bool FP8>
static hipError_t launch_tiled_t(const moe_host::TiledArgs& a, int grid, hipStream_t s) {
  constexpr int lds_bytes = 2 * TileShape<BM, BN>::kStageBytes;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&tiled_gemm_kernel<BM, BN, GATEUP, FP8>),
        hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((tiled_gemm_kernel<BM, BN, GATEUP, FP8>), dim3(grid), dim3(kTileThreads),
                     lds_bytes, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Direct-to-LDS variant: BM x BN tiles computed by 8 waves (two per SIMD, so
// one wave's MFMAs cover the other's waits), one workgroup per CU.
// Operand chunks go from global memory straight into LDS with
// global_load_lds_dwordx4 (each wave instruction fills one 1 KiB chunk,
// lane l writing bytes 16*l..16*l+15), through a ring of NST stages of KS
// 64-byte K steps each.  Weight chunks arrive in MFMA lane order as packed;
// A chunks in the token-chunk layout of lds_dma.h (a row's 64 bytes per quad
// of lanes), whose fragment offsets the MFMA reads apply.  Stage f+NST-1 is issued while stage f is being
// multiplied, so NST-1 compute phases cover the load latency; the ring runs
// straight across work-item boundaries (the next tile's first stages load
// while the current tile finishes), which matters for the short-K down
// GEMM.  Waits are explicit vmcnt counts plus a plain s_barrier (a fenced
// __syncthreads() would drain the whole ring).
//
// Shapes used: 128 x 256, two steps per stage, three stages (48 KiB
// stages), and 256 x 256, one step per stage, five stages (32 KiB stages;
// two thirds of the operand bytes per flop of the former).  Requires
// row_bytes % (64*KS) == 0, at least KS*(NST-1) K steps and N_out a multiple
// of the tile's output columns.
template <int BM_, int BN_, int KS_, int NST_, int WM_, int WN_>
struct DmaShape {
  static constexpr int BM = BM_, BN = BN_, KS = KS_, NST = NST_, WM = WM_, WN = WN_;
  static constexpr int kWaves = WM * WN, kThreads = kWaves * 64;
  static constexpr int MB = BM / WM / 16, NB = BN / WN / 16;   // 16x16 blocks per wave
  static constexpr int kAChunks = BM / 16 * KS, kBChunks = BN / 16 * KS;
  static constexpr int kAPerWave = kAChunks / kWaves, kBPerWave = kBChunks / kWaves;
  static constexpr int kPerWave = kAPerWave + kBPerWave;   // DMA ops per wave per stage
  static constexpr int kStageBytes = (kAChunks + kBChunks) * 1024;
  static constexpr int kLdsBytes = NST * kStageBytes;
  static constexpr int kAhead = NST - 1;                      // stages in flight ahead
  static_assert(kAChunks % kWaves == 0 && kBChunks % kWaves == 0, "chunk split");
  static_assert(kWaves % KS == 0, "a wave's chunks share one K step");
};
using DmaWide = DmaShape<128, 256, 2, 3, 2, 4>;   // 48 KiB stages x 3
using DmaBig = DmaShape<256, 256, 1, 5, 4, 2>;    // 32 KiB stages x 5 (all of LDS)

template <class Sh>
struct DmaItem {
  int expert, row_begin, rows, nt;
  const char* a[Sh::kAPerWave];   // this lane's A sources (step and lane offsets applied)
  const char* b;                  // this lane's packed-B source for weight block 0
};

template <class Sh, bool GATEUP>
__device__ __forceinline__ DmaItem<Sh> dma_item(const moe_host::TiledArgs& g, int item, int n_tiles,
                                                size_t row_bytes, int nsteps, int w_blocks,
                                                int wave, int lane) {
  DmaItem<Sh> it;
  const int ti = item / n_tiles;
  it.nt = item - ti * n_tiles;
  const moe_task_t task = load_task_scalar(g.tasks + ti);
  it.expert = task.expert;
  it.row_begin = task.row_begin;
  it.rows = task.rows;
  // wave w loads chunks w + kWaves*i: 16-row block (w + kWaves*i) / KS, step w % KS
  const int st = wave % Sh::KS;
#pragma unroll
  for (int i = 0; i < Sh::kAPerWave; i++) {
    int rr = ((wave + Sh::kWaves * i) / Sh::KS) * 16 + tok_copy_row(lane);
    if (rr >= task.rows) rr = 0;    // a valid row; its products are never stored
    const int arow = GATEUP ? g.sorted_pairs[task.row_begin + rr] / g.topk : task.row_begin + rr;
    it.a[i] = static_cast<const char*>(g.a) + (size_t)arow * row_bytes + st * 64 + 16 * tok_copy_piece(lane);
  }
  it.b = static_cast<const char*>(g.b) + ((size_t)task.expert * w_blocks * nsteps + st) * 1024 + 16 * lane;
  return it;
}

template <class Sh, bool GATEUP, bool FP8>
__global__ void __launch_bounds__(Sh::kThreads, 1)
tiled_dma_kernel(moe_host::TiledArgs g) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  constexpr int MB = Sh::MB, NB = Sh::NB, KS = Sh::KS, NST = Sh::NST, AHEAD = Sh::kAhead;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / Sh::WN, wn = wave % Sh::WN;

  const int num_tasks = min(g.header[kHdrNumTasks], g.max_tasks);
  const int out_cols = GATEUP ? Sh::BN / 2 : Sh::BN;
  const int n_tiles = g.N_out / out_cols;
  const int total = num_tasks * n_tiles;
  const size_t row_bytes = (size_t)g.K * (FP8 ? 1 : 2);
  const int nsteps = (int)(row_bytes / 64);
  const int nk = nsteps / KS;
  const int w_blocks = g.w_rows / 16;

  const int G = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd = G / 8, extra = G % 8;
  const int vid = (xcd < extra ? xcd * (per_xcd + 1) : extra * (per_xcd + 1) + (xcd - extra) * per_xcd) + slot;
  if (vid >= total) return;
  const int n_items = (total - vid + G - 1) / G;
  const int F = n_items * nk;

  // weight 16-row block of the tile's j-th B block
  auto wrb = [&](int nt, int j) {
    if (GATEUP) {
      constexpr int half = Sh::BN / 32;   // gate blocks, then the matching up blocks
      return j < half ? nt * half + j : g.N_out / 16 + nt * half + (j - half);
    }
    return nt * (Sh::BN / 16) + j;
  };

  // Sources of the current and the next item, kept in registers.
  DmaItem<Sh> cur = dma_item<Sh, GATEUP>(g, vid, n_tiles, row_bytes, nsteps, w_blocks, wave, lane);
  DmaItem<Sh> nxt = cur;
  if (n_items > 1)
    nxt = dma_item<Sh, GATEUP>(g, vid + G, n_tiles, row_bytes, nsteps, w_blocks, wave, lane);

  auto issue = [&](const DmaItem<Sh>& it, int kt, int slot_) {
    char* sb = lds + slot_ * Sh::kStageBytes;
#pragma unroll
    for (int i = 0; i < Sh::kAPerWave; i++)
      dma16(it.a[i] + (size_t)kt * KS * 64, sb + (wave + Sh::kWaves * i) * 1024);
#pragma unroll
    for (int i = 0; i < Sh::kBPerWave; i++) {
      const int c = wave + Sh::kWaves * i;
      dma16(it.b + ((size_t)wrb(it.nt, c / KS) * nsteps + (size_t)kt * KS) * 1024,
            sb + (Sh::kAChunks + c) * 1024);
    }
  };
  // flat stage index fi -> (item relative to the current one, K iteration)
  auto issue_flat = [&](int fi, int ii) {
    const int item_rel = fi / nk - ii;
    const int kt = fi % nk;
    if (item_rel == 0) issue(cur, kt, fi % NST);
    else issue(nxt, kt, fi % NST);
  };

#pragma unroll
  for (int d = 0; d < AHEAD; d++)
    if (d < F) issue_flat(d, 0);   // nk >= AHEAD: all in item 0

  const int aoff = tok_frag_off(lane);   // this lane's fragment in an A chunk
  int f = 0;   // flat stage index over all items of this workgroup
  for (int ii = 0; ii < n_items; ii++) {
    f32x4 acc[MB][NB];
#pragma unroll
    for (int m = 0; m < MB; m++)
#pragma unroll
      for (int q = 0; q < NB; q++) acc[m][q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int kt = 0; kt < nk; kt++, f++) {
      // stage f landed (only the stages issued after it may still be in
      // flight), in every wave
      const int later = min(AHEAD - 1, F - 1 - f);
      if (later >= 4) wait_vm<4 * Sh::kPerWave>();
      else if (later == 3) wait_vm<3 * Sh::kPerWave>();
      else if (later == 2) wait_vm<2 * Sh::kPerWave>();
      else if (later == 1) wait_vm<Sh::kPerWave>();
      else wait_vm<0>();
      barrier_nofence();
      const char* base = lds + (f % NST) * Sh::kStageBytes;
      auto bchunk = [&](int q) {
        if (GATEUP) return q < NB / 2 ? wn * (NB / 2) + q : Sh::BN / 32 + wn * (NB / 2) + (q - NB / 2);
        return wn * NB + q;
      };
      if constexpr (FP8 && KS % 2 == 0) {
        // two K steps per full-rate fp8 instruction
#pragma unroll
        for (int st = 0; st < KS; st += 2) {
          u32x4 fa[MB][2], fb[NB][2];
#pragma unroll
          for (int h = 0; h < 2; h++) {
#pragma unroll
            for (int m = 0; m < MB; m++)
              fa[m][h] = *reinterpret_cast<const u32x4*>(base + ((wm * MB + m) * KS + st + h) * 1024 + aoff);
#pragma unroll
            for (int q = 0; q < NB; q++)
              fb[q][h] = *reinterpret_cast<const u32x4*>(base + (Sh::kAChunks + bchunk(q) * KS + st + h) * 1024 + 16 * lane);
          }
#pragma unroll
          for (int m = 0; m < MB; m++)
#pragma unroll
            for (int q = 0; q < NB; q++) mfma_fp8_k128(acc[m][q], fa[m][0], fa[m][1], fb[q][0], fb[q][1]);
        }
      } else {
#pragma unroll
        for (int st = 0; st < KS; st++) {
          u32x4 fa[MB], fb[NB];
#pragma unroll
          for (int m = 0; m < MB; m++)
            fa[m] = *reinterpret_cast<const u32x4*>(base + ((wm * MB + m) * KS + st) * 1024 + aoff);
#pragma unroll
          for (int q = 0; q < NB; q++)
            fb[q] = *reinterpret_cast<const u32x4*>(base + (Sh::kAChunks + bchunk(q) * KS + st) * 1024 + 16 * lane);
#pragma unroll
          for (int m = 0; m < MB; m++)
#pragma unroll
            for (int q = 0; q < NB; q++) mfma_step_t<FP8>(acc[m][q], fa[m], fb[q]);
        }
      }
      // Stage f+AHEAD goes into the slot of stage f-1, which every wave
      // finished reading before the barrier above.  Issued after this
      // stage's MFMAs (which run on asynchronously) so the two overlap.
      if (f + AHEAD < F) issue_flat(f + AHEAD, ii);
    }

    // ---- epilogue of this item
    const int lrow = lane & 15, lgrp = lane >> 4;
    constexpr int WROWS = Sh::BM / Sh::WM;
#pragma unroll
    for (int m = 0; m < MB; m++) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int rr = wm * WROWS + m * 16 + 4 * lgrp + i;
        const bool ok = rr < cur.rows;
        const int r = cur.row_begin + (ok ? rr : 0);
        if constexpr (GATEUP) {
          float sx = 1.0f;
          if constexpr (FP8) sx = g.a_scale[g.sorted_pairs[r] / g.topk];
          float rmax = 0.0f;
#pragma unroll
          for (int q = 0; q < NB / 2; q++) {
            const int col = cur.nt * (Sh::BN / 2) + wn * (NB / 2) * 16 + q * 16 + lrow;
            float gv = acc[m][q][i], uv = acc[m][q + NB / 2][i];
            if constexpr (FP8) {
              gv = (gv * sx) * g.b_scale[(size_t)cur.expert * g.w_rows + col];
              uv = (uv * sx) * g.b_scale[(size_t)cur.expert * g.w_rows + g.N_out + col];
            }
            const float hv = silu_f32(gv) * uv;
            if (ok) {
              if constexpr (FP8) static_cast<float*>(g.c)[(size_t)r * g.N_out + col] = hv;
              else static_cast<uint16_t*>(g.c)[(size_t)r * g.N_out + col] = f32_to_bf16_bits(hv);
              rmax = __builtin_fmaxf(rmax, __builtin_fabsf(hv));
            }
          }
          if constexpr (FP8) {
            rmax = max16(rmax);
            if (ok && lrow == 0)
              atomicMax(reinterpret_cast<unsigned int*>(g.row_amax) + r, __float_as_uint(rmax));
          }
        } else {
          float sa = 1.0f;
          if constexpr (FP8) sa = g.a_scale[r];
#pragma unroll
          for (int q = 0; q < NB; q++) {
            const int col = cur.nt * Sh::BN + wn * (NB * 16) + q * 16 + lrow;
            float v = acc[m][q][i];
            if constexpr (FP8) v = (v * sa) * g.b_scale[(size_t)cur.expert * g.w_rows + col];
            if (ok) static_cast<uint16_t*>(g.c)[(size_t)r * g.N_out + col] = f32_to_bf16_bits(v);
          }
        }
      }
    }
    cur = nxt;
    if (ii + 2 < n_items)
      nxt = dma_item<Sh, GATEUP>(g, vid + (ii + 2) * G, n_tiles, row_bytes, nsteps, w_blocks, wave, lane);
  }
}

template <class Sh, bool GATEUP, bool FP8>
static hipError_t launch_dma_t(const moe_host::TiledArgs& a, int grid, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&tiled_dma_kernel<Sh, GATEUP, FP8>),
        hipFuncAttributeMaxDynamicSharedMemorySize, Sh::kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((tiled_dma_kernel<Sh, GATEUP, FP8>), dim3(grid), dim3(Sh::kThreads),
                     Sh::kLdsBytes, s, a);
  return hipGetLastError();
}

template <class Sh>
static hipError_t launch_dma_shape(const moe_host::TiledArgs& a, bool gateup, bool fp8, int grid,
                                   hipStream_t s) {
  if (gateup) return fp8 ? launch_dma_t<Sh, true, true>(a, grid, s) : launch_dma_t<Sh, true, false>(a, grid, s);
  return fp8 ? launch_dma_t<Sh, false, true>(a, grid, s) : launch_dma_t<Sh, false, false>(a, grid, s);
}

// requantise fp32 rows h32[r][0..I) of the valid sorted rows with the
// row amax accumulated in h_scale[r] by the GEMM epilogue, or, with
// find_amax, found here from the row itself; h_scale[r] then holds the row
// scale.
// NV > 0: the row is read once into registers (I <= NV * 4 * 256), its amax
// found (find_amax) and the codes written from there; NV == 0: read twice.
template <int NV>
__global__ void __launch_bounds__(256)
requant_rows_kernel(const float* __restrict__ h32, int I, const int32_t* __restrict__ expert_offsets,
                    int E, uint8_t* __restrict__ hq, float* __restrict__ h_scale, int find_amax) {
  const int r = blockIdx.x;
  if (r >= expert_offsets[E]) return;
  const f32x4* row = reinterpret_cast<const f32x4*>(h32 + (size_t)r * I);
  uint32_t* q = reinterpret_cast<uint32_t*>(hq + (size_t)r * I);
  const int nv = I / 4;
  f32x4 v[NV > 0 ? NV : 1];
  float amax;
  if constexpr (NV > 0) {
#pragma unroll
    for (int j = 0; j < NV; j++) {
      const int i = threadIdx.x + j * 256;
      v[j] = i < nv ? row[i] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
  if (find_amax) {
    if constexpr (NV > 0) {
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < NV; j++)
        m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[j][0]), __builtin_fabsf(v[j][1])),
                                               __builtin_fmaxf(__builtin_fabsf(v[j][2]), __builtin_fabsf(v[j][3]))));
      amax = block_max_f32<256>(m);
    } else {
      amax = row_amax_f32<256>(h32 + (size_t)r * I, I);
    }
  } else {
    amax = h_scale[r];
    __syncthreads();   // every thread has read the amax before it is replaced
  }
  float sc, inv;
  e4m3_row_scales(amax, &sc, &inv);
  if constexpr (NV > 0) {
#pragma unroll
    for (int j = 0; j < NV; j++) {
      const int i = threadIdx.x + j * 256;
      if (i < nv)
        q[i] = f32x4_to_e4m3x4_sat(__fmul_rn(v[j][0], inv), __fmul_rn(v[j][1], inv), __fmul_rn(v[j][2], inv),
                                   __fmul_rn(v[j][3], inv));
    }
  } else {
    for (int i = threadIdx.x; i < nv; i += 256) {
      const f32x4 w = row[i];
      q[i] = f32x4_to_e4m3x4_sat(__fmul_rn(w[0], inv), __fmul_rn(w[1], inv), __fmul_rn(w[2], inv),
                                 __fmul_rn(w[3], inv));
    }
  }
  if (threadIdx.x == 0) h_scale[r] = sc;
}

}  // namespace moe

namespace moe_host {

hipError_t launch_tiled_gemm(const TiledArgs& a, bool gateup, bool fp8, int bm, int bn, int grid,
                             hipStream_t s) {
  if (bm == 256 && bn == 256) return moe::launch_dma_shape<moe::DmaBig>(a, gateup, fp8, grid, s);
  if (bm != 128) return hipErrorInvalidValue;
  if (bn == 256) return moe::launch_dma_shape<moe::DmaWide>(a, gateup, fp8, grid, s);
  if (bn == 128) {
    if (gateup) return fp8 ? moe::launch_tiled_t<128, 128, true, true>(a, grid, s)
                           : moe::launch_tiled_t<128, 128, true, false>(a, grid, s);
    return fp8 ? moe::launch_tiled_t<128, 128, false, true>(a, grid, s)
               : moe::launch_tiled_t<128, 128, false, false>(a, grid, s);
  }
  if (bn == 64) {
    if (gateup) return fp8 ? moe::launch_tiled_t<128, 64, true, true>(a, grid, s)
                           : moe::launch_tiled_t<128, 64, true, false>(a, grid, s);
    return fp8 ? moe::launch_tiled_t<128, 64, false, true>(a, grid, s)
               : moe::launch_tiled_t<128, 64, false, false>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_requant_rows(const float* h32, int P, int I, const int32_t* expert_offsets,
                               int E, uint8_t* hq, float* h_scale, bool find_amax, hipStream_t s) {
  const int per = (I / 4 + 255) / 256;   // 16-byte vectors per thread
#define MOE_REQUANT_NV(NVv)                                                                             \
  hipLaunchKernelGGL(moe::requant_rows_kernel<NVv>, dim3(P), dim3(256), 0, s, h32, I, expert_offsets, E, \
                     hq, h_scale, find_amax ? 1 : 0)
  if (per <= 1) MOE_REQUANT_NV(1);
  else if (per <= 2) MOE_REQUANT_NV(2);
  else if (per <= 4) MOE_REQUANT_NV(4);
  else if (per <= 8) MOE_REQUANT_NV(8);
  else MOE_REQUANT_NV(0);
#undef MOE_REQUANT_NV
  return hipGetLastError();
}

}  // namespace moe_host
