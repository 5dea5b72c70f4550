// Grouped expert GEMM for a few dozen to a few hundred rows per expert:
// the layer is still bound by streaming the expert weights from HBM, but a
// task tile holds too many token rows for register streaming, which would
// re-read every row of the tile from L2 once per 16 weight columns.
//
// Same pipeline role as stream_gemm.hip (HPC-Ops x SGLang blog, section
// "MoE": gate-up reads tokens through the route index with no separate
// gather; a persistent grid consumes the per-tile task map).
//
//  * One workgroup of 8 waves per CU.  Work item = (task tile of 16*MB
//    rows, strip of 256 output columns, K slice).
//  * The tile's token rows go through LDS: a ring of NBUF+1 stages, each
//    holding KS 64-byte K steps of all 16*MB rows as 1 KiB chunks (16 rows
//    of one step, each row's 64 bytes copied by one quad of lanes; the
//    token-chunk layout of lds_dma.h), filled by direct global->LDS copies
//    spread over the waves.
//  * Each wave owns 32 columns of the strip and streams their packed
//    weights (1 KiB chunks) straight into registers NBUF
//    stages ahead, so a CU keeps 8 x NBUF x KS x 2 KiB of weights in flight
//    without passing them through LDS.  A weight fragment in registers
//    meets all 16*MB rows of the tile; a token fragment read from LDS meets
//    both of the wave's 16-column blocks.
//  * The ring runs straight across work items: the next item's first stages
//    are in flight while the current one finishes and stores its results.
//  * Optionally (rotate) the strips of one tile start their K loops at
//    different stages, so that the 16 workgroups sharing its token rows do not
//    ask L2 for the same lines at the same moment; every stage is still summed
//    once, in an order fixed by the strip's position.
//  * Per-item metadata (the task record, the tile's token indices, fp8
//    column scales) comes from scalar loads, whose waits are on lgkmcnt, so
//    the vector-memory queue holds only the ring's loads and the epilogue's
//    stores, and the explicit vmcnt waits below count exactly those.
//
// int8 w8a8 (I8, with FP8 set: the same one-byte layout and per-channel
// scales): one v_mfma_i32_16x16x64_i8 per 64-byte step; the int32 sums
// (|sum| <= 127^2 K < 2^31) become fp32 at the start of the epilogue, which
// then applies the scales as on fp8.
//
// Output: fp32 partial sums c[s][P][N], bf16 rows c[P][N] (one slice,
// out_bf16), or on gate-up with one slice h = SiLU(gate) * up (act: the
// wave's two blocks are a gate block and its up block; fp8 writes fp32 h for
// the requantisation).  On fp8 the per-column weight scale is applied here,
// and the per-row activation scale by the consumer (SiLU-and-mul, the top-k
// reduction) or, with act, here.
#include <type_traits>

#include "lds_dma.h"

namespace moe {

// A strip is 256 output columns: 16 * NSUB columns per wave, 16 / NSUB
// waves per workgroup (8 waves of two column blocks).
template <int NSUB>
constexpr int strip_waves() {
  return 16 / NSUB;
}

// Token chunks a wave copies per stage: the tile's MB * KS chunks spread
// over the waves, rounded up; the copies past the tile's chunks (160-row
// tiles: 20 chunks over 8 waves) re-read one line of its first row, so that
// every wave issues the same number of operations per stage.
template <int MB, int KS, int NSUB>
struct StripItem {
  static constexpr int NA = (MB * KS + strip_waves<NSUB>() - 1) / strip_waves<NSUB>();
  int row_begin, rows, s;
  int rot;                     // K stages the item's loop is rotated by
  int col;                     // first output column of this wave (of h when fusing SiLU-and-mul)
  const char* a[NA];           // this lane's token sources (K step and lane offsets applied)
  const char* b;               // this lane's packed-weight source of column block 0
  float bs[NSUB];              // fp8: weight scale of this lane's column in each block
  // block fp8: this lane's row scale in the stage's copy (float offset at
  // the item's first stage), and per block q the index of its first unit in
  // the weight-scale array
  int sc_off;
  int wq0[NSUB];
  // MXFP8: this lane's weight row scale dword in the stage's copy (byte
  // offset from wmx, the expert's e8m0 codes)
  int sc_woff;
  const uint8_t* wmx;
};

// Block fp8 row scales per stage: KS / 2 units of 16 * MB rows, copied in
// parts of 64 rows (one 4-byte copy instruction each); wave w copies part
// w % parts, so every wave issues one instruction per stage.
template <int MB, int KS>
constexpr int blk_row_parts() {
  return MB * KS / 8;
}

// Distance between a wave's column blocks in the packed weights: adjacent
// blocks, or with SiLU-and-mul fused the gate block and its up block N/2
// columns further.
__device__ __forceinline__ size_t strip_block_stride(const moe_host::StripArgs& g, int nsteps) {
  return (size_t)(g.act ? g.N / 32 : 1) * nsteps * 1024;
}

template <int MB, int KS, int NSUB, bool GATHER, bool FP8, int SC = 0>
__device__ __forceinline__ StripItem<MB, KS, NSUB> strip_item(const moe_host::StripArgs& g, int item,
                                                              int n_strips, int nk, size_t row_bytes,
                                                              int nsteps, int wave, int lane) {
  constexpr int W = strip_waves<NSUB>();
  constexpr int kCols = W * NSUB * 16;
  StripItem<MB, KS, NSUB> it;
  const int s = item % g.split;
  const int rest = item / g.split;
  // the strips of one tile side by side: they meet its token rows in L2
  const int nt = rest % n_strips;
  const int ti = rest / n_strips;
  const moe_task_t task = load_task_scalar(g.tasks + ti);
  it.row_begin = task.row_begin;
  it.rows = task.rows;
  it.s = s;
  it.rot = g.rotate ? (nt % 16) * (nk / 16) : 0;
  it.col = g.act ? (nt * W + wave) * 16 : nt * kCols + wave * (NSUB * 16);
  const int step0 = s * nk * KS;
  const int crow = tok_copy_row(lane);   // this lane's row of each token chunk it copies
#pragma unroll
  for (int i = 0; i < StripItem<MB, KS, NSUB>::NA; i++) {
    // chunk c = 16-row block c / KS, K step c % KS of every stage
    const int c0 = wave + W * i;
    const bool pad = c0 >= MB * KS;   // a copy past the tile's chunks
    const int c = pad ? 0 : c0;
    const int rb = c / KS, st = c % KS;
    // Row blocks past the tile, and rows past it inside the last block,
    // re-read the tile's first row: always a valid address, never stored.
    // A whole block past the tile thus reads one 64-byte line per step
    // (every lane the same row), not 16 rows.
    const bool blk_in = !pad && rb * 16 < task.rows;
    const bool in_tile = blk_in && rb * 16 + crow < task.rows;
    int arow;
    if constexpr (GATHER) {
      const i32x16_t sp = load16_scalar(g.sorted_pairs + task.row_begin + (blk_in ? rb * 16 : 0));
      const int p = in_tile ? pick16(sp, crow) : sp[0];
      arow = p / g.topk;
    } else {
      arow = task.row_begin + (in_tile ? rb * 16 + crow : 0);
    }
    // rows past the tile read the first row's pieces in the same order
    it.a[i] = static_cast<const char*>(g.a) + (size_t)arow * row_bytes + (size_t)(step0 + st) * 64 +
              16 * tok_copy_piece(lane);
  }
  it.b = static_cast<const char*>(g.b) +
         (((size_t)task.expert * (g.N / 16) + it.col / 16) * nsteps + step0) * 1024 + 16 * lane;
#pragma unroll
  for (int q = 0; q < NSUB; q++) {
    it.bs[q] = 1.0f;
    if constexpr (FP8 && SC == 0) {
      const int wcol = g.act ? it.col + q * (g.N / 2) : it.col + 16 * q;   // weight row of block q
      const i32x16_t v = load16_scalar(g.b_scale + (size_t)task.expert * g.N + wcol);
      it.bs[q] = __int_as_float(spread16(v, lane));
    }
  }
  it.sc_off = 0;
  it.sc_woff = 0;
  it.wmx = nullptr;
  if constexpr (SC == 2) {
    // MXFP8: e8m0 codes, K / 32 bytes per row, one dword per row and
    // 128-value unit; the K slice starts at unit step0 / 2
    const int kb = g.K / 32, unit0 = step0 / 2;
    // row scales: the lane's row of the part this wave copies (64 rows of
    // one unit); rows past the tile take the tile's first row
    const int lin = (wave % blk_row_parts<MB, KS>()) * 64;
    const int uis = lin / (16 * MB), rb0 = lin % (16 * MB);
    const int r = rb0 + lane;
    int srow;
    if constexpr (GATHER) {   // the token of the row (scalar loads of 16 indices)
      const i32x16_t s0 = load16_scalar(g.sorted_pairs + task.row_begin);
      int tk = s0[0];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if (rb0 + 16 * j < task.rows) {
          const i32x16_t sj = load16_scalar(g.sorted_pairs + task.row_begin + rb0 + 16 * j);
          const int v = spread16(sj, lane);
          tk = (lane >> 4) == j ? v : tk;
        }
      }
      srow = (r < task.rows ? tk : s0[0]) / g.topk;
    } else {
      srow = task.row_begin + (r < task.rows ? r : 0);
    }
    it.sc_off = srow * kb + (unit0 + uis) * 4;
    // weight scales: the rows of the wave's blocks, KS / 2 units (lanes
    // past them repeat the first ones)
    const int jw = lane % (KS / 2 * NSUB * 16);
    const int wu = jw / (NSUB * 16), wq = (jw / 16) % NSUB, wc = jw % 16;
    const int wrow = (g.act ? it.col + wq * (g.N / 2) : it.col + 16 * wq) + wc;
    it.wmx = g.b_mx + (size_t)task.expert * g.N * kb;
    it.sc_woff = wrow * kb + (unit0 + wu) * 4;
  }
  if constexpr (SC == 1) {
    // unit-major scales: activations [K/128][P] per sorted row, weights
    // [E][N/128][K/128] per 128 x 128 block; the K slice starts at unit
    // step0 / 2
    const int units = g.K / 128, unit0 = step0 / 2;
#pragma unroll
    for (int q = 0; q < NSUB; q++) {
      const int wrow = g.act ? it.col + q * (g.N / 2) : it.col + 16 * q;
      it.wq0[q] = (task.expert * (g.N / 128) + wrow / 128) * units + unit0;
    }
    const int row = (wave % blk_row_parts<MB, KS>()) * 64 + lane;   // of the stage's KS / 2 units
    const int uis = row / (16 * MB), r = row % (16 * MB);
    // rows past the tile re-read its first row
    it.sc_off = (unit0 + uis) * g.P + task.row_begin + (r < task.rows ? r : 0);
  }
  return it;
}

template <bool FP8, bool I8 = false>
__device__ __forceinline__ void strip_mfma(f32x4& acc, const u32x4& a, const u32x4& b) {
  if constexpr (I8) {
    acc = __builtin_bit_cast(f32x4, __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, a),
                                                                         __builtin_bit_cast(i32x4_t, b),
                                                                         __builtin_bit_cast(i32x4_t, acc),
                                                                         0, 0, 0));
  } else if constexpr (FP8) {
    const i64x2 a2 = __builtin_bit_cast(i64x2, a);
    const i64x2 b2 = __builtin_bit_cast(i64x2, b);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[0], b2[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[1], b2[1], acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
}

// One register stage of a wave's weights: KS 64-byte K steps of NSUB column
// blocks.  On fp8 with whole 128-value units (PAIRS) two consecutive steps
// of a block share one 8-dword tuple, the operand of the 128-value MFMA, so
// each load lands in its half of the operand and nothing is copied to
// assemble it.
template <int KS, int NSUB, bool PAIRS>
struct WeightStage {
  u32x4 r[KS][NSUB];
  __device__ __forceinline__ void set(int u, int q, const u32x4& v) { r[u][q] = v; }
  __device__ __forceinline__ const u32x4& step(int u, int q) const { return r[u][q]; }
};

template <int KS, int NSUB>
struct WeightStage<KS, NSUB, true> {
  i32x8 r[KS / 2][NSUB];
  __device__ __forceinline__ void set(int u, int q, const u32x4& v) {
    if (u & 1) r[u >> 1][q].hi = __builtin_bit_cast(i32x4_t, v);
    else r[u >> 1][q].lo = __builtin_bit_cast(i32x4_t, v);
  }
  __device__ __forceinline__ const i32x8& unit(int u2, int q) const { return r[u2][q]; }
};

template <int MB, int KS, int NBUF, int NSUB, bool GATHER, bool FP8, bool I8 = false, int SC = 0>
__global__ void __launch_bounds__(strip_waves<NSUB>() * 64, 1)
strip_gemm_kernel(moe_host::StripArgs g) {
  constexpr bool BLK = SC == 1, MXS = SC == 2;
  static_assert(!I8 || (FP8 && SC == 0), "int8 uses the one-byte per-channel path");
  static_assert(SC == 0 || (FP8 && KS % 2 == 0), "block scales: whole 128-value units per stage");
  using It = StripItem<MB, KS, NSUB>;
  constexpr int NA = It::NA;
  // vector-memory operations per wave per stage: token chunks, weights, and
  // the scale copies (block fp8: row scales; MXFP8: row and weight scales)
  constexpr int PER = NA + KS * NSUB + (BLK ? 1 : (MXS ? 2 : 0));
  constexpr int NST = NBUF + 1;         // LDS ring slots
  constexpr int W = strip_waves<NSUB>();
  constexpr int TOK = NA * W * 1024;    // a slot's token chunks (and padding copies)
  constexpr int RSB = KS / 2 * MB * 64;   // then the row scales (4 bytes per row and unit)
  // then (MXFP8) 256 bytes of weight scales per wave
  constexpr int SLOT = TOK + (BLK ? 1024 : (MXS ? RSB + W * 256 : 0));
  static_assert(SC == 0 || (blk_row_parts<MB, KS>() >= 1 && blk_row_parts<MB, KS>() * 64 == KS / 2 * MB * 16 &&
                            blk_row_parts<MB, KS>() <= W && RSB <= 1024),
                "row-scale copy parts");
  static_assert(!MXS || KS / 2 * NSUB * 16 <= 64, "one weight-scale copy per wave");
  static_assert(NA >= 1 && (SC == 0 || NA * W == MB * KS), "token chunks split evenly over waves");
  static_assert(NBUF >= 2, "ring depth");
  static_assert((NBUF - 1) * PER < 64, "vmcnt range");
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int lane = threadIdx.x & 63;
  // wave-uniform, and known to be so: the scalar loads address with it
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int num_tasks = min(g.header[kHdrNumTasks], g.max_tasks);
  const int n_strips = g.N / (W * NSUB * 16);
  const int total = num_tasks * n_strips * g.split;
  const size_t row_bytes = (size_t)g.K * (FP8 ? 1 : 2);
  const int nsteps = (int)(row_bytes / 64);
  const int nk = nsteps / (KS * g.split);   // stages per item: a multiple of NBUF, >= NBUF
  const size_t bq = strip_block_stride(g, nsteps);

  // XCD-aware numbering: workgroups are dispatched round-robin over the 8
  // XCDs; give each XCD a contiguous run of items, so the strips of one task
  // tile share its token rows through one L2.
  const int G = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd = G / 8, extra = G % 8;
  const int vid = (xcd < extra ? xcd * (per_xcd + 1) : extra * (per_xcd + 1) + (xcd - extra) * per_xcd) + slot;
  if (vid >= total) return;
  const int n_items = (total - vid + G - 1) / G;

  // Weight strips read by one tile each stream past the caches (non-temporal
  // loads).  When some expert has several tiles (a skewed or dense routing),
  // its tiles' work items run side by side and read the same strip, so the
  // strips are read with ordinary loads and the later tiles find them in L2
  // (measured: DeepSeek-V3 fp8 T=4096 gate-up at 128-row tiles 2277 -> 1830
  // us; ordinary loads cost 3-7% where nothing is shared).  The choice is
  // made once per launch from the routing header: the cache hint is part of
  // the load instruction, and the two bodies below never rejoin, which keeps
  // the compiler's waits on the weight registers exact.
  auto body = [&](auto nt_tag) {
    constexpr bool NT_B = decltype(nt_tag)::value;
    It cur = strip_item<MB, KS, NSUB, GATHER, FP8, SC>(g, vid, n_strips, nk, row_bytes, nsteps, wave,
                                                       lane);
    It nxt = cur;
    if (n_items > 1)
      nxt = strip_item<MB, KS, NSUB, GATHER, FP8, SC>(g, vid + G, n_strips, nk, row_bytes, nsteps, wave,
                                                      lane);

    // Every stage issues exactly PER vector-memory operations per wave: the
    // NBUF stages past the last one re-load the last item's first stages
    // (valid addresses, never used), so the wait before each stage is the
    // same count and the compiler's own waits for the weight registers see
    // the same queue on every path.
    constexpr bool PAIRS = FP8 && !I8 && KS % 2 == 0;
    WeightStage<KS, NSUB, PAIRS> bb[NBUF];
    // block fp8: each stage's weight block scales (wave-uniform), loaded
    // NBUF stages ahead through the scalar cache
    float swb[NBUF][NSUB][KS / 2 > 0 ? KS / 2 : 1];
    const __attribute__((address_space(4))) float* bsc =
        (const __attribute__((address_space(4))) float*)(g.b_scale);
    auto issue = [&](bool in_cur, int kt, int fslot, WeightStage<KS, NSUB, PAIRS>& b,
                     float (&sw)[NSUB][KS / 2 > 0 ? KS / 2 : 1]) {
      char* sb = lds + fslot * SLOT;
      // the item's stage kt in its rotated order (every stage exactly once)
      kt += in_cur ? cur.rot : nxt.rot;
      if (kt >= nk) kt -= nk;
  #pragma unroll
      for (int i = 0; i < NA; i++)
        dma16((in_cur ? cur.a[i] : nxt.a[i]) + (size_t)kt * KS * 64,
              sb + (wave + W * i) * 1024);
      if constexpr (BLK) {
        // the stage's row scales, one part per wave (parts copied by several
        // waves get the same bytes twice; one instruction per wave keeps the
        // per-stage counts equal)
        dma4(g.rs_u + ((in_cur ? cur.sc_off : nxt.sc_off) + kt * (KS / 2) * g.P),
             sb + TOK + (wave % blk_row_parts<MB, KS>()) * 256);
#pragma unroll
        for (int q = 0; q < NSUB; q++)
#pragma unroll
          for (int v = 0; v < KS / 2; v++)
            sw[q][v] = bsc[(in_cur ? cur.wq0[q] : nxt.wq0[q]) + kt * (KS / 2) + v];
      }
      if constexpr (MXS) {
        // the stage's row scale dwords (one part of 64 rows per wave, as on
        // block fp8) and the wave's own weight scale dwords
        dma4(g.a_mx + ((in_cur ? cur.sc_off : nxt.sc_off) + kt * (KS / 2) * 4),
             sb + TOK + (wave % blk_row_parts<MB, KS>()) * 256);
        dma4((in_cur ? cur.wmx : nxt.wmx) + ((in_cur ? cur.sc_woff : nxt.sc_woff) + kt * (KS / 2) * 4),
             sb + TOK + RSB + wave * 256);
      }
      const char* bsrc = in_cur ? cur.b : nxt.b;
  #pragma unroll
      for (int u = 0; u < KS; u++)
  #pragma unroll
        for (int q = 0; q < NSUB; q++)
          if constexpr (NT_B)
            b.set(u, q, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                            bsrc + q * bq + ((size_t)kt * KS + u) * 1024)));
          else
            b.set(u, q, *reinterpret_cast<const u32x4*>(bsrc + q * bq + ((size_t)kt * KS + u) * 1024));
    };

    // The empty asm statements keep each stage's operations together in
    // issue order (the barriers do so inside the loop), which the vmcnt
    // counts rely on.
  #pragma unroll
    for (int d = 0; d < NBUF; d++) {
      issue(true, d, d, bb[d], swb[d]);
      __asm__ volatile("" ::: "memory");
    }

    const int lrow = lane & 15, lgrp = lane >> 4;
    const int aoff = tok_frag_off(lane);   // this lane's token fragment in a chunk
    int f = 0;   // flat stage index over all items of this workgroup
    for (int ii = 0; ii < n_items; ii++) {
      f32x4 acc[MB][NSUB];
  #pragma unroll
      for (int m = 0; m < MB; m++)
  #pragma unroll
        for (int q = 0; q < NSUB; q++) acc[m][q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

      for (int kt0 = 0; kt0 < nk; kt0 += NBUF, f += NBUF) {
  #pragma unroll
        for (int u = 0; u < NBUF; u++) {
          const int fc = f + u;
          // stage fc has landed in this wave (NBUF-1 later stages, and any
          // epilogue stores, may still be in flight), then in every wave
          wait_vm<(NBUF - 1) * PER>();
          barrier_nofence();
          const char* sb = lds + (fc % NST) * SLOT;
          if constexpr (MXS) {
            // MXFP8: the scaled instruction applies the lane's e8m0 codes,
            // lane 16 g + r those of K block g of row / column r
            const uint32_t* rsc = reinterpret_cast<const uint32_t*>(sb + TOK);
            const uint32_t* wsc = reinterpret_cast<const uint32_t*>(sb + TOK + RSB + wave * 256);
  #pragma unroll
            for (int st = 0; st < KS; st += 2) {
              const int uis = st >> 1;
              int sbq[NSUB];
  #pragma unroll
              for (int q = 0; q < NSUB; q++) sbq[q] = (int)(wsc[(uis * NSUB + q) * 16 + lrow] >> (8 * lgrp));
  #pragma unroll
              for (int m = 0; m < MB; m++) {
                i32x8 a;
                a.lo = *reinterpret_cast<const i32x4_t*>(sb + (m * KS + st) * 1024 + aoff);
                a.hi = *reinterpret_cast<const i32x4_t*>(sb + (m * KS + st + 1) * 1024 + aoff);
                const int sa = (int)(rsc[uis * 16 * MB + 16 * m + lrow] >> (8 * lgrp));
  #pragma unroll
                for (int q = 0; q < NSUB; q++)
                  acc[m][q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb[u].unit(uis, q), acc[m][q], 0,
                                                                              0, 0, sa, 0, sbq[q]);
              }
            }
          } else if constexpr (BLK) {
            // block fp8: each 128-value unit into a fresh sum, then added
            // times (row group scale x weight block scale)
            const float* scs = reinterpret_cast<const float*>(sb + TOK);
  #pragma unroll
            for (int st = 0; st < KS; st += 2) {
              const int uis = st >> 1;
              float sw[NSUB];
  #pragma unroll
              for (int q = 0; q < NSUB; q++) sw[q] = swb[u][q][uis];
  #pragma unroll
              for (int m = 0; m < MB; m++) {
                i32x8 a;
                a.lo = *reinterpret_cast<const i32x4_t*>(sb + (m * KS + st) * 1024 + aoff);
                a.hi = *reinterpret_cast<const i32x4_t*>(sb + (m * KS + st + 1) * 1024 + aoff);
                const f32x4 sx = *reinterpret_cast<const f32x4*>(scs + uis * MB * 16 + 16 * m + 4 * lgrp);
  #pragma unroll
                for (int q = 0; q < NSUB; q++) {
                  f32x4 t = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                  mfma_fp8_unit(t, a, bb[u].unit(st >> 1, q));
  #pragma unroll
                  for (int i = 0; i < 4; i++) acc[m][q][i] += t[i] * (sx[i] * sw[q]);
                }
              }
            }
          } else if constexpr (PAIRS) {
            // two K steps per full-rate fp8 instruction, both operands read
            // into their 8-dword tuples as they are
  #pragma unroll
            for (int st = 0; st < KS; st += 2) {
  #pragma unroll
              for (int m = 0; m < MB; m++) {
                i32x8 a;
                a.lo = *reinterpret_cast<const i32x4_t*>(sb + (m * KS + st) * 1024 + aoff);
                a.hi = *reinterpret_cast<const i32x4_t*>(sb + (m * KS + st + 1) * 1024 + aoff);
  #pragma unroll
                for (int q = 0; q < NSUB; q++) mfma_fp8_unit(acc[m][q], a, bb[u].unit(st >> 1, q));
              }
            }
          } else {
  #pragma unroll
            for (int st = 0; st < KS; st++) {
  #pragma unroll
              for (int m = 0; m < MB; m++) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(sb + (m * KS + st) * 1024 + aoff);
  #pragma unroll
                for (int q = 0; q < NSUB; q++) strip_mfma<FP8, I8>(acc[m][q], a, bb[u].step(st, q));
              }
            }
          }
          // Stage fc+NBUF reuses this stage's registers and the ring slot of
          // stage fc-1, which every wave finished reading before the barrier.
          const int ktn = kt0 + u + NBUF;
          const bool in_cur = ktn < nk;
          issue(in_cur, in_cur ? ktn : ktn - nk, (fc + NBUF) % NST, bb[u], swb[u]);
        }
      }

      // Epilogue: lane holds column (lane % 16) and rows 4*(lane / 16) + i of
      // each 16 x 16 block.
      if constexpr (I8) {   // int32 sums to fp32
  #pragma unroll
        for (int m = 0; m < MB; m++)
  #pragma unroll
          for (int q = 0; q < NSUB; q++)
            acc[m][q] = __builtin_convertvector(__builtin_bit_cast(i32x4_t, acc[m][q]), f32x4);
      }
      // SiLU-and-mul in this epilogue (gate-up, one K slice): bf16 h, or on
      // fp8 the fp32 h that the requantisation pass turns into codes (it
      // finds each row's amax from the row: folding it here would take one
      // atomic per row and 16 columns).  The fp8 row scales come through
      // scalar loads, 16 rows at a time, so the epilogue issues no vector
      // load whose wait would drain the ring.
      bool fused = false;
      if constexpr (GATHER && NSUB == 2) fused = g.act != 0;
      if (fused) {
        // h = SiLU(gate) * up: the wave's gate block and its up block
        const int hn = g.N / 2;
  #pragma unroll
        for (int m = 0; m < MB; m++) {
          float xs[4] = {1.0f, 1.0f, 1.0f, 1.0f};
          if constexpr (FP8 && SC == 0) {
            // the block's 16 row scales (rows inside the tile only: the array
            // has 16 entries past its last row, not MB * 16)
            if (16 * m < cur.rows) {
              const i32x16_t sv = load16_scalar(g.x_scale_rows + cur.row_begin + 16 * m);
  #pragma unroll
              for (int i = 0; i < 4; i++) xs[i] = __int_as_float(pick16(sv, 4 * lgrp + i));
            }
          }
  #pragma unroll
          for (int i = 0; i < 4; i++) {
            const int rr = 16 * m + 4 * lgrp + i;
            const bool ok = rr < cur.rows;
            const size_t r = (size_t)(cur.row_begin + (ok ? rr : 0));
            float gv = acc[m][0][i], uv = acc[m][1][i];
            if constexpr (FP8 && SC == 0) {
              gv = (gv * cur.bs[0]) * xs[i];
              uv = (uv * cur.bs[1]) * xs[i];
            }
            const float hv = silu_f32(gv) * uv;
            const int col = cur.col + lrow;
            if (ok) {
              if constexpr (FP8) static_cast<float*>(g.c)[r * hn + col] = hv;
              else static_cast<uint16_t*>(g.c)[r * hn + col] = f32_to_bf16_bits(hv);
            }
          }
        }
      } else {
  #pragma unroll
        for (int m = 0; m < MB; m++) {
  #pragma unroll
          for (int i = 0; i < 4; i++) {
            const int rr = 16 * m + 4 * lgrp + i;
            if (rr < cur.rows) {
              const size_t r = (size_t)(cur.row_begin + rr);
  #pragma unroll
              for (int q = 0; q < NSUB; q++) {
                const int col = cur.col + 16 * q + lrow;
                float v = acc[m][q][i];
                if constexpr (FP8 && SC == 0) v = v * cur.bs[q];
                if (g.out_bf16)
                  static_cast<uint16_t*>(g.c)[r * g.N + col] = f32_to_bf16_bits(v);
                else
                  static_cast<float*>(g.c)[((size_t)cur.s * g.P + r) * g.N + col] = v;
              }
            }
          }
        }
      }
      cur = nxt;
      if (ii + 2 < n_items)
        nxt = strip_item<MB, KS, NSUB, GATHER, FP8, SC>(g, vid + (ii + 2) * G, n_strips, nk, row_bytes,
                                                        nsteps, wave, lane);
    }
    // the trailing re-loads still write this workgroup's LDS: let them land
    wait_vm<0>();
  };
  if (g.header[kHdrMaxExpertTiles] > 1) body(std::false_type{});
  else body(std::true_type{});
}

template <int MB, int KS, int NBUF, int NSUB, bool GATHER, bool FP8, bool I8, int SC = 0>
static hipError_t launch_strip_t(const moe_host::StripArgs& a, int grid, hipStream_t s) {
  constexpr int lds_bytes =
      (NBUF + 1) * (StripItem<MB, KS, NSUB>::NA * strip_waves<NSUB>() * 1024 + (SC == 1 ? 1024 : (SC == 2 ? KS / 2 * MB * 64 + strip_waves<NSUB>() * 256 : 0)));
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&strip_gemm_kernel<MB, KS, NBUF, NSUB, GATHER, FP8, I8, SC>),
        hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((strip_gemm_kernel<MB, KS, NBUF, NSUB, GATHER, FP8, I8, SC>), dim3(grid),
                     dim3(strip_waves<NSUB>() * 64), lds_bytes, s, a);
  return hipGetLastError();
}

// kind: 0 bf16, 1 fp8, 2 int8 (one-byte per-channel path with the integer
// MFMA), 3 block fp8 (128 x 128 weight blocks, 128-value activation groups),
// 4 MXFP8 (e8m0 codes per 32 values of both operands)
template <int MB, int KS, int NBUF, int NSUB>
static hipError_t launch_strip_cfg(const moe_host::StripArgs& a, bool gather, int kind, int grid,
                                   hipStream_t s) {
  if constexpr (MB * KS % strip_waves<NSUB>() != 0) {
    // tiles whose chunks do not split evenly over the waves: the one-byte
    // per-channel paths (fp8, int8) only
    if (kind == 2) return gather ? launch_strip_t<MB, KS, NBUF, NSUB, true, true, true>(a, grid, s)
                                 : launch_strip_t<MB, KS, NBUF, NSUB, false, true, true>(a, grid, s);
    if (kind != 1) return hipErrorInvalidValue;
    return gather ? launch_strip_t<MB, KS, NBUF, NSUB, true, true, false>(a, grid, s)
                  : launch_strip_t<MB, KS, NBUF, NSUB, false, true, false>(a, grid, s);
  } else {
    if (kind == 3 || kind == 4) {
      if constexpr (KS % 2 == 0) {
        if (kind == 3)
          return gather ? launch_strip_t<MB, KS, NBUF, NSUB, true, true, false, 1>(a, grid, s)
                        : launch_strip_t<MB, KS, NBUF, NSUB, false, true, false, 1>(a, grid, s);
        return gather ? launch_strip_t<MB, KS, NBUF, NSUB, true, true, false, 2>(a, grid, s)
                      : launch_strip_t<MB, KS, NBUF, NSUB, false, true, false, 2>(a, grid, s);
      }
      return hipErrorInvalidValue;
    }
    if (kind == 2) return gather ? launch_strip_t<MB, KS, NBUF, NSUB, true, true, true>(a, grid, s)
                                 : launch_strip_t<MB, KS, NBUF, NSUB, false, true, true>(a, grid, s);
    if (gather) return kind == 1 ? launch_strip_t<MB, KS, NBUF, NSUB, true, true, false>(a, grid, s)
                                 : launch_strip_t<MB, KS, NBUF, NSUB, true, false, false>(a, grid, s);
    return kind == 1 ? launch_strip_t<MB, KS, NBUF, NSUB, false, true, false>(a, grid, s)
                     : launch_strip_t<MB, KS, NBUF, NSUB, false, false, false>(a, grid, s);
  }
}

}  // namespace moe

namespace moe_host {

// (16-row blocks per tile, K steps per stage, stages in flight) built here.
#define MOE_STRIP_CONFIGS(X) \
  X(4, 2, 4) X(4, 4, 3) X(4, 4, 4) X(4, 2, 3) X(4, 4, 2) X(4, 2, 2) \
  X(8, 2, 4) X(8, 2, 3) X(8, 1, 4) X(8, 2, 2)             \
  X(12, 2, 4) X(12, 2, 3) X(12, 2, 2) X(10, 2, 4) X(10, 2, 3) X(10, 2, 2)

bool strip_config_supported(int mb, int ks, int nbuf, bool fp8) {
  // 160- and 192-row tiles serve the one-byte paths only (the bf16 ones
  // would spill registers); the 160-row ones per-channel fp8 and int8 only
  if ((mb == 12 || mb == 10) && !fp8) return false;
#define MOE_STRIP_CASE(M, K, N) if (mb == M && ks == K && nbuf == N) return true;
  MOE_STRIP_CONFIGS(MOE_STRIP_CASE)
#undef MOE_STRIP_CASE
  return false;
}

hipError_t launch_strip_gemm(const StripArgs& a, bool gather, bool fp8, int mb, int ks, int nbuf,
                             int grid, hipStream_t s, int variant) {
  if (variant && !fp8) return hipErrorInvalidValue;
  if (variant >= 2 && (ks % 2 || a.K % 128 || (a.act && a.split != 1))) return hipErrorInvalidValue;
  const int kind = variant == 1 ? 2 : (variant == 2 ? 3 : (variant == 3 ? 4 : (fp8 ? 1 : 0)));
#define MOE_STRIP_CASE(M, K, N) \
  if (mb == M && ks == K && nbuf == N) return moe::launch_strip_cfg<M, K, N, 2>(a, gather, kind, grid, s);
  MOE_STRIP_CONFIGS(MOE_STRIP_CASE)
#undef MOE_STRIP_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe_host
