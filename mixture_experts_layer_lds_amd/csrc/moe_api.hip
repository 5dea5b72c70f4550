// C ABI of the fused MoE layer: argument checks, buffer layouts, the tile
// plan and the launch sequence.  See include/moe.h for the contract.
//
// The launch path is plain C++ over the HIP runtime with native-type
// arguments and a per-device cache of the compute-unit count, so no Python
// sits between the caller and the kernels (the FlagOS C++ launch wrapper
// article makes the same point about interpreter overhead on the launch
// path).
#include <algorithm>
#include <cmath>
#include <mutex>

#include "moe_common.h"
#include "decode_route.h"

// Workspace of moe_forward_fp8_noalloc: one array per GPU, held until the
// process ends.  In host code its name is only a stand-in for the device
// symbol; the device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_WORKSPACE_BYTES];

namespace {


constexpr size_t kNone = ~(size_t)0;
constexpr long kStreamWaves = 2048;   // waves that fill 256 CUs x 8
// The plan is a fixed function of the sizes (the layout queries run without
// a device), so it balances work for MI355X's compute-unit count; launches
// use the device's actual count.
constexpr long kPlanCUs = 256;
// One-byte per-channel layers (fp8, int8 w8a8): strips from this many mean
// rows per expert on, register streaming below.  Same-box A/B (graph replay,
// DeepSeek-V3 shape): T=128 (4 rows) fp8 1759 us strips against 1700
// streaming, int8 1750 / 1703; T=256 (8) fp8 1816 / 1765, int8 1807 / 1778;
// T=512 (16) fp8 1891 / 2099, int8 1877 / 2099.
constexpr long kOneByteStripMin = 12;
constexpr int kStripCols = 256;       // output columns per strip work item

enum Tiling { kStreaming = 0, kLdsTiles = 1, kStrips = 2 };

struct Plan {
  int block_m = 16;
  int mb = 1;
  int max_tasks = 0;
  int tiling = kStreaming;
  int bm_t = 128;                // LDS tiles: rows per tile (128 or 256)
  int bn1 = 128, bn2 = 128;      // LDS tiles: N tile of gate-up / down
  int split1 = 1, split2 = 1;    // strips: K slices of gate-up (K = H) / down (K = I)
  int sw1 = 1, su1 = 2;          // streaming gate-up: waves per workgroup, K steps per stage
  int sw2 = 1, su2 = 2;          // streaming down
  int ks1 = 4, nbuf1 = 4;        // strips: K steps per stage, stages in flight (gate-up)
  int ks2 = 4, nbuf2 = 4;        // (down)
  bool fp8_units = false;        // fp8 streaming on 128-value units (fp8b_gemm.hip, per-channel mode)
  bool half1 = false;            // bf16 streaming gate-up on half-width (8-column) items
  int nb = 2;                    // streaming: weight blocks per item, 2 or 4 (bf16 on 32-row
                                 // tiles; MX, int8, block fp8 on 64-row tiles; int4 and
                                 // int8 w8a16 on 32- or 64-row tiles)
  int dr_waves = 0;              // streaming, one token: down GEMM and top-k sum in one launch
  int dr_u = 2;                  // with this many waves per workgroup (0: two launches), K steps
  bool dr_half = false;          // per register stage and 8-column items
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool known_dtype(int dtype) {
  return dtype == MOE_DTYPE_BF16 || dtype == MOE_DTYPE_FP8_W8A8 || dtype == MOE_DTYPE_MXFP8 ||
         dtype == MOE_DTYPE_INT8_W8A8 || dtype == MOE_DTYPE_INT4_W4A16 ||
         dtype == MOE_DTYPE_FP8_BLOCK || dtype == MOE_DTYPE_INT8_W8A16;
}

int check_shape(int T, int k, int E, int H, int I, int dtype = MOE_DTYPE_BF16) {
  if (T < 0 || k < 1 || k > moe::kMaxTopK || E < 1 || E > moe::kMaxExperts || H <= 0 || I <= 0)
    return MOE_ERR_INVALID_ARG;
  if (H % 64 || I % 64 || H > 65536 || I > 65536) return MOE_ERR_UNSUPPORTED_SHAPE;
  // MX: both reductions in whole 128-value units of the scaled instruction
  if ((dtype == MOE_DTYPE_MXFP8 || dtype == MOE_DTYPE_INT4_W4A16 || dtype == MOE_DTYPE_FP8_BLOCK) &&
      (H % 128 || I % 128))
    return MOE_ERR_UNSUPPORTED_SHAPE;   // whole 128-value units / scale groups
  if ((long)T * k > moe::kMaxPairs) return MOE_ERR_UNSUPPORTED_SHAPE;
  return MOE_OK;
}

// Register-streaming split of a reduction of nsteps 64-byte steps over the
// waves of a workgroup for `items` work items, each wave taking a whole
// number of two-step stages; one-step stages, unsplit, when the steps are
// odd.
void choose_stream(int nsteps, int mb, long items, int* waves, int* u) {
  // Each wave of a launch (kStreamWaves of them) runs whole items in turn, so
  // a launch lasts (items per workgroup, rounded up) x (K steps per wave +
  // the latency of an item's first loads, about kItemSteps steps).  The
  // split that minimises this is taken, the smallest on a tie.
  constexpr long kItemSteps = 4;
  int best = 0;
  long best_cost = 0;
  for (int w = 1; w <= 8; w *= 2) {
    if (nsteps % (2 * w) || !moe_host::stream_config_supported(mb, w, 2)) continue;
    long grid = kStreamWaves / w;
    if (items < grid) grid = items;
    if (grid < 1) grid = 1;
    const long rounds = (items + grid - 1) / grid;
    const long cost = rounds * (nsteps / w + kItemSteps);
    if (!best || cost < best_cost) {
      best = w;
      best_cost = cost;
    }
  }
  if (best) {
    *waves = best;
    *u = 2;
  } else {
    *waves = 1;
    *u = 1;
  }
}

// Strip GEMM configuration for a reduction of nsteps 64-byte steps and
// `items` work items per K slice: the (K steps per stage, stages in flight)
// pairs the kernel is built for, in order of preference, and the smallest
// power-of-two K split whose items spread evenly (>= 80%) over the CUs, else
// the best-spread one.  Returns false if no configuration divides the
// reduction.
bool choose_strip(int nsteps, int mb, bool fp8, long items, int* split, int* ks, int* nbuf,
                  bool even_ks = false, bool down = false) {
  // about 12-24 KiB of weights in flight per wave first.  The down GEMM
  // starts from a two-stage ring: its K is the short intermediate width, so
  // a deep ring's fill is a large part of each item (measured 1-2% faster
  // on the whole layer at 128-4096 tokens, up to 7% on its down kernel).  So
  // do the 160- and 192-row tiles: there the four-stage ring spills
  // registers on int8, MXFP8 and block fp8 (same-box A/B at DeepSeek-V3
  // T=4096, us per layer: int8 2877 -> 2866, MXFP8 3500 -> 3481, block fp8
  // 3453 -> 3417; per-channel fp8, which does not spill, 2736 against 2739).
  static const int kCfgUp[8][2] = {{2, 4}, {4, 3}, {4, 4}, {2, 3}, {4, 2}, {1, 4}, {2, 2}, {1, 2}};
  static const int kCfgDown[8][2] = {{2, 2}, {2, 4}, {4, 3}, {4, 4}, {2, 3}, {4, 2}, {1, 4}, {1, 2}};
  const auto& kCfg = down || mb >= 10 ? kCfgDown : kCfgUp;
  double best_eff = -1.0;
  for (int S = 1; S <= 8; S *= 2) {
    for (const auto& c : kCfg) {
      if (!moe_host::strip_config_supported(mb, c[0], c[1], fp8) || (even_ks && c[0] % 2)) continue;
      if (nsteps % (c[0] * S)) continue;
      const int nk = nsteps / (c[0] * S);
      if (nk < c[1] || nk % c[1]) continue;
      const long n = items * S;
      const long rounds = (n + kPlanCUs - 1) / kPlanCUs;
      const double eff = (double)n / (double)(rounds * kPlanCUs);
      if (eff > best_eff + 1e-9) {
        best_eff = eff;
        *split = S;
        *ks = c[0];
        *nbuf = c[1];
      }
      break;   // first supported configuration for this split
    }
    if (best_eff >= 0.8) break;
  }
  return best_eff >= 0.0;
}

// Strips of 160-row tiles run with the K loops of a tile's strips rotated
// against each other (StripArgs::rotate).
int rotate_strips(const Plan& p, bool down) {
  (void)down;
  return p.mb == 10 ? 1 : 0;
}

// Tile plan: a fixed function of the shape and dtype, shared by the routing
// build, the workspace layout and the forward pass.
// Waves per workgroup for the 128-value-unit streaming kernels (int4,
// block fp8, per-channel fp8 on units): the wave count w dividing the units
// that minimises (items per workgroup slot) x (units per wave + 2), the
// number of register stages on the critical path plus the ramp.
int pick_unit_waves(int units, long items) {
  int best = 1;
  long best_cost = -1;
  for (int w = 1; w <= 8; w *= 2) {
    if (units % w) continue;
    long grid = kStreamWaves / w;
    if (items < grid) grid = items;
    if (grid < 1) grid = 1;
    const long cost = (items + grid - 1) / grid * (units / w + 2);
    if (best_cost < 0 || cost < best_cost) best = w, best_cost = cost;
  }
  return best;
}

// Expected number of distinct experts among T tokens that each pick k
// distinct experts uniformly: E (1 - (1 - k/E)^T), at least 1.
long expected_active(int T, int k, int E) {
  if (k >= E) return E;
  const double miss = std::pow(1.0 - (double)k / E, (double)T);
  const long ex = (long)std::ceil(E * (1.0 - miss) - 1e-9);
  return ex < 1 ? 1 : ex;
}

Plan make_plan(int dtype, int T, int k, int E, int H, int I) {
  Plan p;
  const long P = (long)T * k;
  const long active = P < E ? P : E;
  // The down GEMM's wave split is chosen for the expected number of active
  // experts, the gate-up's for the bound min(P, E).  Same-box A/B (graph
  // replay) of the expected count in the down choice: Mixtral-8x7B T=4 355
  // -> 338 us, int4 153 -> 143, int8 w8a16 197 -> 192, Qwen2-57B T=4 71.1
  // -> 66.7, T=8 110.4 -> 106.6; in the gate-up choice as well it helped
  // Qwen3-30B-A3B T=8 (56.8 -> 53.5) but cost DeepSeek-V3 T=16 (714 -> 734)
  // and Qwen2-57B T=8 (110 -> 112).
  const long active_d = std::min(active, expected_active(T, k, E));
  const long avg = active > 0 ? (P + active - 1) / active : 1;
  const int esz_t = dtype == MOE_DTYPE_BF16 ? 2 : 1;
  const int nsteps1 = H * esz_t / 64, nsteps2 = I * esz_t / 64;
  if (dtype == MOE_DTYPE_FP8_BLOCK && avg >= kOneByteStripMin && avg <= 160 && (2 * I) % kStripCols == 0 &&
      H % kStripCols == 0) {
    // [128,128] block fp8 with many rows per expert: the strips, each
    // 128-value unit rescaled by its row group and weight block scales, with
    // the fp8 tile heights (192-row tiles spill ten registers here and are
    // still ahead: DeepSeek-V3 T=4096 3653 us on 128-row tiles, 3463 us on
    // 192), an unsplit gate-up (its epilogue forms the fp32 h of the group
    // requantisation)
    const int first = avg <= 40 ? 4 : (avg <= 96 ? 8 : 12);
    for (int mb = first; mb <= 12; mb = mb == 8 ? 12 : mb * 2) {
      long tasks = (P + 16 * mb - 1) / (16 * mb);
      if (tasks < active) tasks = active;
      Plan q = p;
      if (choose_strip(nsteps1, mb, true, tasks * (2L * I / kStripCols), &q.split1, &q.ks1, &q.nbuf1, true) &&
          q.split1 == 1 &&
          choose_strip(nsteps2, mb, true, tasks * ((long)H / kStripCols), &q.split2, &q.ks2, &q.nbuf2, true, true)) {
        q.tiling = kStrips;
        q.mb = mb;
        q.block_m = 16 * mb;
        q.max_tasks = (int)(P / q.block_m + (P < E ? P : E));
        return q;
      }
    }
  }
  if (dtype == MOE_DTYPE_INT4_W4A16 || dtype == MOE_DTYPE_FP8_BLOCK || dtype == MOE_DTYPE_INT8_W8A16) {
    // int4 and int8 weights, block-scaled fp8: register streaming (128-value K steps;
    // int8: 64-value steps) at every size; waves per workgroup by the streaming cost
    // model on whole steps
    p.tiling = kStreaming;
    p.block_m = avg <= 8 ? 16 : (avg <= 16 ? 32 : 64);
    p.mb = p.block_m / 16;
    p.max_tasks = (int)(P / p.block_m + (P < E ? P : E));
    long est = (P + p.block_m - 1) / p.block_m;
    if (est < active) est = active;
    const int per = dtype == MOE_DTYPE_INT8_W8A16 ? 64 : 128;   // K values per step
    p.sw1 = pick_unit_waves(H / per, est * ((long)I / 16));
    long est_d = (P + p.block_m - 1) / p.block_m;
    if (est_d < active_d) est_d = active_d;
    p.sw2 = pick_unit_waves(I / per, est_d * ((long)H / 32));
    if ((dtype == MOE_DTYPE_INT4_W4A16 || dtype == MOE_DTYPE_INT8_W8A16) && p.mb >= 2 && I % 32 == 0 &&
        H % 64 == 0) {
      // tiles of 32 or 64 rows: four weight blocks per item halve the token-row re-reads
      p.nb = 4;
      const int wmax = 16 / p.mb;   // the waves' partial sums within 64 KiB of LDS
      p.sw1 = std::min(pick_unit_waves(H / per, est * ((long)I / 32)), wmax);
      p.sw2 = std::min(pick_unit_waves(I / per, est_d * ((long)H / 64)), wmax);
    }
    if (dtype == MOE_DTYPE_FP8_BLOCK && p.mb == 4 && I % 32 == 0 && H % 64 == 0) {
      // 64-row tiles: four weight blocks per item halve the token-row
      // re-reads (the register tile allows at most two waves)
      p.nb = 4;
      p.sw1 = std::min(pick_unit_waves(H / per, est * ((long)I / 32)), 2);
      p.sw2 = std::min(pick_unit_waves(I / per, est_d * ((long)H / 64)), 2);
    }
    p.su1 = p.su2 = 1;
    return p;
  }
  if ((dtype == MOE_DTYPE_INT8_W8A8 || dtype == MOE_DTYPE_MXFP8) && avg >= kOneByteStripMin && avg <= 160 &&
      (2 * I) % kStripCols == 0 && H % kStripCols == 0) {
    // int8 w8a8 and MXFP8 with many rows per expert: the fp8 strips (the
    // same one-byte layout) on the integer MFMA (int8, per-channel scales)
    // or the scaled one (MX: e8m0 codes of rows and weights copied per
    // stage, whole 128-value units), with the fp8 tile heights; only an
    // unsplit gate-up, whose epilogue forms the fp32 h that the
    // requantisation reads.
    const bool mx = dtype == MOE_DTYPE_MXFP8;
    // int8 takes 160-row tiles up to 128 mean rows, as per-channel fp8 does
    // (DeepSeek-V3 int8 T=4096: 2866 -> 2733 us against 192-row tiles); the
    // MX copies of row scales need whole 64-row parts
    const bool i8 = dtype == MOE_DTYPE_INT8_W8A8;
    const int first = avg <= 40 ? 4 : (avg <= 96 ? 8 : (avg <= 128 && i8 ? 10 : 12));
    for (int mb = first; mb <= 12; mb = mb == 8 ? (i8 ? 10 : 12) : (mb == 10 ? 12 : mb * 2)) {
      long tasks = (P + 16 * mb - 1) / (16 * mb);
      if (tasks < active) tasks = active;
      Plan q = p;
      if (choose_strip(nsteps1, mb, true, tasks * (2L * I / kStripCols), &q.split1, &q.ks1, &q.nbuf1, mx) &&
          q.split1 == 1 &&
          choose_strip(nsteps2, mb, true, tasks * ((long)H / kStripCols), &q.split2, &q.ks2, &q.nbuf2, mx, true)) {
        q.tiling = kStrips;
        q.mb = mb;
        q.block_m = 16 * mb;
        q.max_tasks = (int)(P / q.block_m + (P < E ? P : E));
        return q;
      }
    }
  }
  if (dtype == MOE_DTYPE_MXFP8 || dtype == MOE_DTYPE_INT8_W8A8) {
    // MXFP8 and int8: register streaming (MXFP8 at every size: its activation
    // block scales ride with the register stages; the strips' and tiles' LDS
    // rings count their loads exactly and carry no scale stream).  Two-step
    // stages: one 128-value unit of the scaled instruction each.
    p.tiling = kStreaming;
    p.block_m = avg <= 8 ? 16 : (avg <= 16 ? 32 : 64);
    p.mb = p.block_m / 16;
    p.max_tasks = (int)(P / p.block_m + (P < E ? P : E));
    long est = (P + p.block_m - 1) / p.block_m;
    if (est < active) est = active;
    choose_stream(nsteps1, p.mb, est * ((long)I / 16), &p.sw1, &p.su1);
    long est_d = (P + p.block_m - 1) / p.block_m;
    if (est_d < active_d) est_d = active_d;
    choose_stream(nsteps2, p.mb, est_d * ((long)H / 32), &p.sw2, &p.su2);
    if (p.mb == 4 && I % 32 == 0 && H % 64 == 0 && nsteps1 % 2 == 0 && nsteps2 % 2 == 0) {
      // 64-row tiles: four weight blocks per item halve the token-row
      // re-reads (the register tile allows at most two waves)
      p.nb = 4;
      p.su1 = p.su2 = 2;
      p.sw1 = nsteps1 % 4 == 0 ? std::min(p.sw1, 2) : 1;
      p.sw2 = nsteps2 % 4 == 0 ? std::min(p.sw2, 2) : 1;
    }
    if (dtype == MOE_DTYPE_INT8_W8A8 && T == 1 && nsteps2 % 2 == 0) {
      // one token: the down GEMM adds the top-k rows itself, as on bf16 and
      // per-channel fp8 (below)
      p.dr_waves = 8;
      p.dr_half = k <= 8 && nsteps2 % 4 == 0 && H / 16 < kPlanCUs * 3 / 4;
      p.dr_u = nsteps2 % (p.dr_half ? 8 : 4) == 0 ? 4 : 2;
    }
    return p;
  }
  // Few rows per expert (decode): register streaming, tiles of 16 rows.
  // 9 to ~80 rows (fp8: 12 to ~160): strips (token rows in LDS, weights streamed),
  // tiles of about twice the mean rows per active expert so that the usual
  // spread of a uniform routing still fits one tile per expert.  More rows:
  // LDS tiles of both operands.
  // Measured crossover to LDS tiles: ~80 rows per expert for bf16 (Qwen2-57B
  // T=1024: 287 us tiles, 332 us strips) and above 128 for fp8 (DeepSeek-V3
  // T=4096: 3285 us strips, 3484 us tiles).
  // The low end likewise: strips from 12 rows on fp8 (kOneByteStripMin), from
  // 9 on bf16 (Mixtral-8x7B T=16: 464 us streaming, 508 us strips).
  const long strip_max = dtype == MOE_DTYPE_FP8_W8A8 ? 160 : 80;
  const long strip_min = dtype == MOE_DTYPE_FP8_W8A8 ? kOneByteStripMin : 9;
  if (dtype == MOE_DTYPE_BF16 && avg >= 9 && avg <= 16 && H >= 3072 && I % 32 == 0 && H % 64 == 0) {
    // 32-row tiles on register streaming with four weight blocks per item,
    // for long reductions (same-box A/B against the strips: Mixtral-8x7B T=64
    // 463 -> 453 us, Qwen2-57B T=128 194 -> 180 us; with H = 2048, Qwen3-30B-A3B
    // T=256, the strips stay ahead, 159 against 194 us)
    p.tiling = kStreaming;
    p.block_m = 32;
    p.mb = 2;
    p.nb = 4;
    p.max_tasks = (int)(P / p.block_m + (P < E ? P : E));
    long est = (P + p.block_m - 1) / p.block_m;
    if (est < active) est = active;
    choose_stream(nsteps1, p.mb, est * ((long)I / 32), &p.sw1, &p.su1);
    long est_d = (P + p.block_m - 1) / p.block_m;
    if (est_d < active_d) est_d = active_d;
    choose_stream(nsteps2, p.mb, est_d * ((long)H / 64), &p.sw2, &p.su2);
    p.sw1 = std::min(p.sw1, 4);
    p.sw2 = std::min(p.sw2, 4);
    if (p.su1 == 2 && p.su2 == 2) return p;
    p = Plan();
  }
  if (avg >= strip_min && avg <= strip_max && (2 * I) % kStripCols == 0 && H % kStripCols == 0) {
    // Tile height about twice the mean rows per expert, and at least 64
    // rows: a skewed routing puts several times the mean on its hottest
    // experts, whose weights a shorter tile would stream once per tile, and
    // emptier tiles cost MFMA time, which this weight-bound range has spare.
    // Same-box A/B of 64- against 32-row tiles (graph replay): Qwen3-30B-A3B
    // T=256 skewed 158 -> 146 us, uniform 222 -> 216 us; DeepSeek-V3 fp8
    // T=128 1767 -> 1759 us.  When no strip configuration divides the
    // reductions at that height, a taller one.
    const bool fp8 = dtype == MOE_DTYPE_FP8_W8A8;
    // heights 4, 8, 10 and 12 row blocks (10 and 12 only for fp8, whose
    // strips run to 160 mean rows: 160- and 192-row tiles keep an expert's
    // rows in one tile).  160 rows up to 128 mean rows, where they still hold
    // a uniform routing's fullest expert (same-box A/B, DeepSeek-V3 fp8:
    // T=4096, 128 mean rows, 2768 -> 2708 us against 192-row tiles; T=3072,
    // 96 mean rows, 2516 us against 2447 on 128-row tiles).
    const int first = avg <= 40 ? 4 : (avg <= 96 || !fp8 ? 8 : (avg <= 128 ? 10 : 12));
    for (int mb = first; mb <= 12; mb = mb == 8 ? (fp8 ? 10 : 12) : (mb == 10 ? 12 : mb * 2)) {
      long tasks = (P + 16 * mb - 1) / (16 * mb);
      if (tasks < active) tasks = active;
      Plan q = p;
      if (choose_strip(nsteps1, mb, fp8, tasks * (2L * I / kStripCols), &q.split1, &q.ks1, &q.nbuf1) &&
          choose_strip(nsteps2, mb, fp8, tasks * ((long)H / kStripCols), &q.split2, &q.ks2, &q.nbuf2, false, true)) {
        q.tiling = kStrips;
        q.mb = mb;
        q.block_m = 16 * mb;
        q.max_tasks = (int)(P / q.block_m + (P < E ? P : E));
        return q;
      }
    }
  }
  const bool tiled = avg > 48;
  p.tiling = tiled ? kLdsTiles : kStreaming;
  const int rb1 = H * esz_t, rb2 = I * esz_t;   // row bytes of the two reductions
  // 256 x 256 direct-to-LDS tiles (4-stage ring, 64-byte K steps) when the
  // experts hold enough rows to fill them; else 128-row tiles: the 128 x 256
  // direct-to-LDS ring (128-byte K steps) where the shape allows it, or the
  // register-staged 128 x 128 / 128 x 64 tiles.
  const bool big = avg >= 192 && I % 128 == 0 && H % 256 == 0 && rb1 >= 192 && rb2 >= 192;
  p.bm_t = big ? 256 : 128;
  const bool dma1 = rb1 % 128 == 0 && rb1 >= 256 && I % 128 == 0;
  const bool dma2 = rb2 % 128 == 0 && rb2 >= 256 && H % 256 == 0;
  p.bn1 = big || dma1 ? 256 : 128;       // 128 (or 64) output columns of h per tile
  p.bn2 = big || dma2 ? 256 : ((H % 128 == 0) ? 128 : 64);
  p.block_m = tiled ? p.bm_t : (avg <= 8 ? 16 : (avg <= 16 ? 32 : 64));
  p.mb = p.block_m / 16;
  p.max_tasks = (int)(P / p.block_m + (P < E ? P : E));
  long est_tasks = (P + p.block_m - 1) / p.block_m;
  if (est_tasks < active) est_tasks = active;
  long est_tasks_d = (P + p.block_m - 1) / p.block_m;
  if (est_tasks_d < active_d) est_tasks_d = active_d;
  if (!tiled) {
    choose_stream(nsteps1, p.mb, est_tasks * ((long)I / 16), &p.sw1, &p.su1);
    choose_stream(nsteps2, p.mb, est_tasks_d * ((long)H / 32), &p.sw2, &p.su2);
    if (dtype == MOE_DTYPE_BF16 && p.mb == 1 && I % 8 == 0) {
      // Half-width gate-up items when the full-width count leaves some CUs
      // one item more than others: the busiest CU streams ceil(n / CUs)
      // items' bytes (Qwen3-30B-A3B T=1: 384 items, 2 on some of 256 CUs;
      // as 768 half items, 1.5).
      // Only where every workgroup still runs a single item with at least
      // half the full-width split (more rounds of first-load latency, or
      // twice the K steps per wave, cost more than the balance gains:
      // Qwen2-57B T=1 with three half items per workgroup, 33.1 -> 34.0 us).
      const long full = est_tasks * ((long)I / 16), cus = kStreamWaves / 8;
      if ((2 * full + cus - 1) / cus < 2 * ((full + cus - 1) / cus)) {
        for (int w = 8; w >= 1 && w * 2 >= p.sw1; w /= 2) {
          if (nsteps1 % (2 * w) || 2 * full > kStreamWaves / w) continue;
          p.half1 = true;
          p.sw1 = w;
          p.su1 = 2;
          break;
        }
      }
    }
    if (dtype == MOE_DTYPE_FP8_W8A8 && H % 128 == 0 && I % 128 == 0) {
      // whole 128-value units: one 16x16x128 MFMA per unit instead of four 16x16x32
      p.fp8_units = true;
      p.sw1 = pick_unit_waves(H / 128, est_tasks * ((long)I / 16));
      p.sw2 = pick_unit_waves(I / 128, est_tasks_d * ((long)H / 32));
      p.su1 = p.su2 = 2;
    }
    if (T == 1 && nsteps2 % 2 == 0) {
      // One token: the down GEMM runs over the concatenation of the token's
      // experts per 16 output columns and adds the top-k rows itself, one
      // launch fewer.  8-column items where 16-column ones would leave a
      // quarter of the CUs idle.  Same-box A/B against down + reduction
      // (graph replay): DeepSeek-V3 fp8 74.4-75.0 -> 71.5-71.8 us,
      // Mixtral-8x7B 118.8 -> 117.3-117.6, Qwen2-57B 31.5 -> 30.9-31.0,
      // Qwen3-30B-A3B 25.4-25.5 -> 24.7-25.0 (8-column items; 16-column
      // ones, 128 workgroups, 26.7-26.9).
      p.dr_waves = 8;
      p.dr_half = k <= 8 && nsteps2 % 4 == 0 && H / 16 < kPlanCUs * 3 / 4;
      p.dr_u = nsteps2 % (p.dr_half ? 8 : 4) == 0 ? 4 : 2;
    }
  }
  return p;
}

void routing_layout(int T, int k, int E, const Plan& p, moe_routing_layout_t* L) {
  const size_t P = (size_t)T * k;
  size_t off = 0;
  L->header = off;
  off += 64;
  L->expert_offsets = off;
  off = align_up(off + 4 * ((size_t)E + 1), 16);
  L->sorted_pairs = off;
  off = align_up(off + 4 * P, 16);
  L->pair_pos = off;
  off = align_up(off + 4 * P, 16);
  L->tasks = off;
  off = align_up(off + sizeof(moe_task_t) * (size_t)p.max_tasks, 16);
  L->scratch = off;
  off = align_up(off + moe_host::route_scratch_bytes((int)P), 16);
  // tail: the strip GEMM reads the token indices of a row tile as one
  // 64-byte scalar load, which may run up to 60 bytes past the last row
  L->total_bytes = off + 64;
  L->block_m = p.block_m;
  L->max_tasks = p.max_tasks;
}

void workspace_layout(int dtype, int T, int k, int H, int I, const Plan& p,
                      moe_workspace_layout_t* W) {
  const size_t P = (size_t)T * k;
  const bool fp8 = dtype == MOE_DTYPE_FP8_W8A8;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  if (dtype == MOE_DTYPE_FP8_BLOCK) {   // e4m3 codes, group scales per token and per sorted row
    const int s2 = p.tiling == kStrips ? p.split2 : 1;
    W->xq = take((size_t)T * H);
    W->x_scale = take(4 * (size_t)T * (H / 128));
    W->x_scale_rows = take(4 * P * (H / 128));
    W->g = take(4 * P * I);
    W->h = take(P * I);
    W->h_scale = take(4 * P * (I / 128));
    W->y = s2 == 1 ? take(2 * P * H) : take(4 * (size_t)s2 * P * H);
    W->total_bytes = off;
    W->split_k1 = 1;
    W->split_k2 = s2;
    W->tiling = p.tiling;
    return;
  }
  if (dtype == MOE_DTYPE_INT4_W4A16 || dtype == MOE_DTYPE_INT8_W8A16) {   // bf16 activations: bf16 h, y
    W->xq = W->x_scale = W->x_scale_rows = W->g = W->h_scale = kNone;
    W->h = take(2 * P * I);
    W->y = take(2 * P * H);
    W->total_bytes = off;
    W->split_k1 = W->split_k2 = 1;
    W->tiling = p.tiling;
    return;
  }
  if (dtype == MOE_DTYPE_INT8_W8A8) {   // the fp8 streaming / unsplit-strip layout, int8 codes
    const int s2 = p.tiling == kStrips ? p.split2 : 1;
    W->xq = take((size_t)T * H);
    W->x_scale = take(4 * (size_t)T);
    W->x_scale_rows = take(4 * (P + 16));
    W->g = take(4 * P * I);
    W->h = take(P * I);
    W->h_scale = take(4 * P);
    // one token on streaming: the down launch adds the top-k rows itself
    W->y = p.tiling == kStreaming && p.dr_waves ? kNone : (s2 == 1 ? take(2 * P * H) : take(4 * (size_t)s2 * P * H));
    W->total_bytes = off;
    W->split_k1 = 1;
    W->split_k2 = s2;
    W->tiling = p.tiling;
    return;
  }
  if (dtype == MOE_DTYPE_MXFP8) {   // e4m3 codes + e8m0 codes per 32 values
    const int s2 = p.tiling == kStrips ? p.split2 : 1;
    W->xq = take((size_t)T * H);
    W->x_scale = take((size_t)T * H / 32);
    W->x_scale_rows = kNone;
    W->g = take(4 * P * I);          // fp32 SiLU(gate)*up before requantisation
    W->h = take(P * I);
    W->h_scale = take(P * I / 32);
    W->y = s2 == 1 ? take(2 * P * H) : take(4 * (size_t)s2 * P * H);
    W->total_bytes = off;
    W->split_k1 = 1;
    W->split_k2 = s2;
    W->tiling = p.tiling;
    return;
  }
  W->xq = fp8 ? take((size_t)T * H) : kNone;
  W->x_scale = fp8 ? take(4 * (size_t)T) : kNone;
  // per-sorted-row x scales, read 16 at a time by the streaming epilogue
  // and the strips' fused one
  const bool strip_act = p.tiling == kStrips && p.split1 == 1;
  W->x_scale_rows = fp8 && (p.tiling == kStreaming || strip_act) ? take(4 * (P + 16)) : kNone;
  if (p.tiling == kStrips && !strip_act)   // fp32 gate-up partial sums
    W->g = take(4 * (size_t)p.split1 * P * 2 * I);
  else
    W->g = fp8 ? take(4 * P * I) : kNone;               // fp32 SiLU(gate)*up before requant
  W->h = take(P * I * (fp8 ? 1 : 2));
  W->h_scale = fp8 ? take(4 * P) : kNone;
  const bool y_bf16 = p.tiling != kStrips || p.split2 == 1;
  if (p.dr_waves)   // one token: the down launch adds the top-k rows itself
    W->y = kNone;
  else
    W->y = y_bf16 ? take(2 * P * H) : take(4 * (size_t)p.split2 * P * H);
  W->total_bytes = off;
  W->split_k1 = p.tiling == kStrips ? p.split1 : 1;
  W->split_k2 = p.tiling == kStrips ? p.split2 : 1;
  W->tiling = p.tiling;
}

// Compute-unit count per device, queried once.
int cu_count(int* out) {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return MOE_ERR_HIP;
    cache[dev] = n;
  }
  *out = cache[dev];
  return MOE_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_address(void** out) {
  static std::mutex mu;
  static void* cache[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    cache[dev] = p;
  }
  *out = cache[dev];
  return MOE_OK;
}

// Workgroups of a streaming launch: 8 waves per CU, no more than the items.
int stream_grid(long max_items, int waves, int cus) {
  long groups = (long)cus * 8 / waves;
  if (max_items < groups) groups = max_items;
  return (int)(groups < 1 ? 1 : groups);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Check value of a packed-weight descriptor: a 64-bit mix of its other
// fields (the splitmix64 finaliser applied after each, from a fixed seed).
// It tells a descriptor from moe_pack_weights apart from raw weight
// pointers and hand-made descriptors; it is not a secret.
uint64_t mix64(uint64_t h, uint64_t v) {
  h ^= v + 0x9e3779b97f4a7c15ull + (h << 6) + (h >> 2);
  h ^= h >> 30;
  h *= 0xbf58476d1ce4e5b9ull;
  h ^= h >> 27;
  h *= 0x94d049bb133111ebull;
  h ^= h >> 31;
  return h;
}

uint64_t packed_check(const moe_packed_weights_t& d) {
  uint64_t h = 0x4d6f4550616b6564ull;
  h = mix64(h, reinterpret_cast<uintptr_t>(d.data));
  h = mix64(h, (uint32_t)d.dtype);
  h = mix64(h, (uint32_t)d.experts);
  h = mix64(h, (uint32_t)d.rows);
  h = mix64(h, (uint32_t)d.cols);
  return h;
}

// The W1 and W2 descriptors of a forward call, after the sizes: made by
// moe_pack_weights for this dtype, E experts and the matrices [2I][H] and
// [H][I].  T == 0 passes with any descriptors (nothing is read).
int check_packed(int dtype, const moe_packed_weights_t* w1, const moe_packed_weights_t* w2, int T,
                 int k, int E, int H, int I) {
  const int rc = check_shape(T, k, E, H, I, dtype);
  if (rc != MOE_OK || T == 0) return rc;
  auto ok = [&](const moe_packed_weights_t* d, int rows, int cols) {
    return d && d->data && d->dtype == dtype && d->experts == E && d->rows == rows && d->cols == cols &&
           d->check == packed_check(*d);
  };
  return ok(w1, 2 * I, H) && ok(w2, H, I) ? MOE_OK : MOE_ERR_INVALID_ARG;
}

const void* packed_data(const moe_packed_weights_t* d) { return d ? d->data : nullptr; }

// Stage-event hook (measurement only).
void* g_events[10];
bool g_events_on = false;

struct StageScope {
  hipStream_t s;
  int stage;
  StageScope(hipStream_t s_, int st) : s(s_), stage(st) {
    if (g_events_on && g_events[2 * stage])
      (void)hipEventRecord(static_cast<hipEvent_t>(g_events[2 * stage]), s);
  }
  ~StageScope() {
    if (g_events_on && g_events[2 * stage + 1])
      (void)hipEventRecord(static_cast<hipEvent_t>(g_events[2 * stage + 1]), s);
  }
};

int build_routing(int dtype, const int32_t* ids, int T, int k, int E, int H, int I,
                  void* routing, size_t routing_bytes, void* stream) {
  int rc = check_shape(T, k, E, H, I, dtype);
  if (rc != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (!ids || !routing) return MOE_ERR_INVALID_ARG;
  if (!aligned(ids, 4) || !aligned(routing, 16)) return MOE_ERR_INVALID_ARG;
  const Plan p = make_plan(dtype, T, k, E, H, I);
  moe_routing_layout_t L;
  routing_layout(T, k, E, p, &L);
  if (routing_bytes < L.total_bytes) return MOE_ERR_BUFFER_TOO_SMALL;
  const hipError_t e = moe_host::launch_route(ids, T * k, E, p.block_m, p.max_tasks, routing, L,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

struct RoutingView {
  const int32_t* header;
  const int32_t* expert_offsets;
  const int32_t* sorted_pairs;
  const int32_t* pair_pos;
  const moe_task_t* tasks;
};

RoutingView view_routing(const void* routing, const moe_routing_layout_t& L) {
  const char* b = static_cast<const char*>(routing);
  return RoutingView{reinterpret_cast<const int32_t*>(b + L.header),
                     reinterpret_cast<const int32_t*>(b + L.expert_offsets),
                     reinterpret_cast<const int32_t*>(b + L.sorted_pairs),
                     reinterpret_cast<const int32_t*>(b + L.pair_pos),
                     reinterpret_cast<const moe_task_t*>(b + L.tasks)};
}

// MXFP8 forward: x to MX blocks, register-streaming gate-up on the scaled
// instruction (fp32 SiLU(gate)*up), MX requantisation of h, register-
// streaming down (bf16 rows), top-k reduction.
int forward_mx(const void* x, const float* topk_w, const void* routing, const void* w1,
               const uint8_t* w1_scale, const void* w2, const uint8_t* w2_scale, int T, int k, int E,
               int H, int I, void* workspace, size_t workspace_bytes, void* out, void* stream,
               const moe_host::DecodeRouteOut* fold = nullptr) {
  int rc = check_shape(T, k, E, H, I, MOE_DTYPE_MXFP8);
  if (rc != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !topk_w || !routing || !w1 || !w2 || !w1_scale || !w2_scale || !workspace || !out)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(out, 16) ||
      !aligned(topk_w, 4) || !aligned(routing, 16) || !aligned(workspace, 256) ||
      !aligned(w1_scale, 4) || !aligned(w2_scale, 4))
    return MOE_ERR_INVALID_ARG;
  const Plan p = make_plan(MOE_DTYPE_MXFP8, T, k, E, H, I);
  if (p.tiling == kStreaming && (p.su1 != 2 || p.su2 != 2)) return MOE_ERR_UNSUPPORTED_SHAPE;
  moe_routing_layout_t L;
  routing_layout(T, k, E, p, &L);
  moe_workspace_layout_t W;
  workspace_layout(MOE_DTYPE_MXFP8, T, k, H, I, p, &W);
  if (workspace_bytes < W.total_bytes) return MOE_ERR_BUFFER_TOO_SMALL;
  int cus = 0;
  if ((rc = cu_count(&cus)) != MOE_OK) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const RoutingView R = view_routing(routing, L);
  char* ws = static_cast<char*>(workspace);
  const int P = T * k;
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + W.xq);
  uint8_t* sx = reinterpret_cast<uint8_t*>(ws + W.x_scale);
  float* h32 = reinterpret_cast<float*>(ws + W.g);
  uint8_t* hq = reinterpret_cast<uint8_t*>(ws + W.h);
  uint8_t* sh = reinterpret_cast<uint8_t*>(ws + W.h_scale);
  hipError_t e;
  {
    StageScope st(s, 0);
    e = moe_host::launch_mx_quant_bf16(static_cast<const uint16_t*>(x), T, H, xq, sx, s, fold, P);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (p.tiling == kStrips) {
    // strips: gate-up with SiLU(gate)*up in its epilogue (fp32 h), MX
    // requantisation, down (bf16 rows, or fp32 partial sums of split_k2
    // slices), reduction; the scaled instruction applies every e8m0 code
    const bool y_bf16 = p.split2 == 1;
    {
      StageScope st(s, 1);
      moe_host::StripArgs a{};
      a.a = xq;
      a.a_mx = sx;
      a.b = w1;
      a.b_mx = w1_scale;
      a.sorted_pairs = R.sorted_pairs;
      a.header = R.header;
      a.tasks = R.tasks;
      a.c = h32;
      a.K = H;
      a.N = 2 * I;
      a.P = P;
      a.topk = k;
      a.max_tasks = p.max_tasks;
      a.split = 1;
      a.out_bf16 = 0;
      a.act = 1;
      e = moe_host::launch_strip_gemm(a, true, true, p.mb, p.ks1, p.nbuf1, cus, s, 3);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    {
      StageScope st(s, 2);
      e = moe_host::launch_mx_requant(h32, P, I, R.expert_offsets, E, hq, sh, s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    {
      StageScope st(s, 3);
      moe_host::StripArgs a{};
      a.a = hq;
      a.a_mx = sh;
      a.b = w2;
      a.b_mx = w2_scale;
      a.sorted_pairs = R.sorted_pairs;
      a.header = R.header;
      a.tasks = R.tasks;
      a.c = ws + W.y;
      a.K = I;
      a.N = H;
      a.P = P;
      a.topk = k;
      a.max_tasks = p.max_tasks;
      a.split = p.split2;
      a.out_bf16 = y_bf16 ? 1 : 0;
      e = moe_host::launch_strip_gemm(a, false, true, p.mb, p.ks2, p.nbuf2, cus, s, 3);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    {
      StageScope st(s, 4);
      e = moe_host::launch_reduce(ws + W.y, y_bf16, p.split2, P, topk_w, R.pair_pos, R.expert_offsets,
                                  nullptr, E, T, k, H, static_cast<uint16_t*>(out), s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    return MOE_OK;
  }
  {
    StageScope st(s, 1);
    moe_host::StreamArgs a{};
    a.a = xq;
    a.b = w1;
    a.a_mx = sx;
    a.b_mx = w1_scale;
    a.sorted_pairs = R.sorted_pairs;
    a.header = R.header;
    a.tasks = R.tasks;
    a.c = h32;
    a.K = H;
    a.N_out = I;
    a.w_rows = 2 * I;
    a.topk = k;
    a.max_tasks = p.max_tasks;
    e = moe_host::launch_stream_gemm(a, true, true, 1, p.mb, p.sw1, p.su1,
                                     stream_grid((long)p.max_tasks * (I / 16) / (p.nb / 2), p.sw1, cus), s,
                                     p.nb);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  {
    StageScope st(s, 2);
    e = moe_host::launch_mx_requant(h32, P, I, R.expert_offsets, E, hq, sh, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  {
    StageScope st(s, 3);
    moe_host::StreamArgs a{};
    a.a = hq;
    a.b = w2;
    a.a_mx = sh;
    a.b_mx = w2_scale;
    a.sorted_pairs = R.sorted_pairs;
    a.header = R.header;
    a.tasks = R.tasks;
    a.c = ws + W.y;
    a.K = I;
    a.N_out = H;
    a.w_rows = H;
    a.topk = k;
    a.max_tasks = p.max_tasks;
    e = moe_host::launch_stream_gemm(a, false, true, 1, p.mb, p.sw2, p.su2,
                                     stream_grid((long)p.max_tasks * (H / 16) / p.nb, p.sw2, cus), s, p.nb);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  {
    StageScope st(s, 4);
    e = moe_host::launch_reduce(ws + W.y, true, 1, P, topk_w, R.pair_pos, R.expert_offsets, nullptr,
                                E, T, k, H, static_cast<uint16_t*>(out), s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

// Block-scaled fp8 forward: group quantisation of x, register-streaming
// gate-up (fp32 SiLU(gate)*up), group requantisation of h, down (bf16
// rows), top-k reduction.
int forward_fp8b(const void* x, const float* topk_w, const void* routing, const void* w1,
                 const float* w1_scale, const void* w2, const float* w2_scale, int T, int k, int E,
                 int H, int I, void* workspace, size_t workspace_bytes, void* out, void* stream,
                 const moe_host::DecodeRouteOut* fold = nullptr) {
  int rc = check_shape(T, k, E, H, I, MOE_DTYPE_FP8_BLOCK);
  if (rc != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !topk_w || !routing || !w1 || !w2 || !w1_scale || !w2_scale || !workspace || !out)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(out, 16) ||
      !aligned(topk_w, 4) || !aligned(routing, 16) || !aligned(workspace, 256) ||
      !aligned(w1_scale, 4) || !aligned(w2_scale, 4))
    return MOE_ERR_INVALID_ARG;
  const Plan p = make_plan(MOE_DTYPE_FP8_BLOCK, T, k, E, H, I);
  moe_routing_layout_t L;
  routing_layout(T, k, E, p, &L);
  moe_workspace_layout_t W;
  workspace_layout(MOE_DTYPE_FP8_BLOCK, T, k, H, I, p, &W);
  if (workspace_bytes < W.total_bytes) return MOE_ERR_BUFFER_TOO_SMALL;
  int cus = 0;
  if ((rc = cu_count(&cus)) != MOE_OK) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const RoutingView R = view_routing(routing, L);
  char* ws = static_cast<char*>(workspace);
  const int P = T * k;
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + W.xq);
  float* x_rows = reinterpret_cast<float*>(ws + W.x_scale_rows);
  float* h32 = reinterpret_cast<float*>(ws + W.g);
  uint8_t* hq = reinterpret_cast<uint8_t*>(ws + W.h);
  float* h_rows = reinterpret_cast<float*>(ws + W.h_scale);
  hipError_t e;
  {
    StageScope st(s, 0);
    e = moe_host::launch_quant_groups_bf16(static_cast<const uint16_t*>(x), T, H, xq,
                                           reinterpret_cast<float*>(ws + W.x_scale), x_rows, P, k,
                                           R.pair_pos, s, fold);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (p.tiling == kStrips) {
    // strips: gate-up with SiLU(gate)*up in its epilogue (fp32 h), group
    // requantisation, down (bf16 rows, or fp32 partial sums of split_k2
    // slices), reduction; every product already carries both scales
    const bool y_bf16 = p.split2 == 1;
    {
      StageScope st(s, 1);
      moe_host::StripArgs a{};
      a.a = xq;
      a.b = w1;
      a.b_scale = w1_scale;
      a.rs_u = x_rows;
      a.sorted_pairs = R.sorted_pairs;
      a.header = R.header;
      a.tasks = R.tasks;
      a.c = h32;
      a.K = H;
      a.N = 2 * I;
      a.P = P;
      a.topk = k;
      a.max_tasks = p.max_tasks;
      a.split = 1;
      a.out_bf16 = 0;
      a.act = 1;
      e = moe_host::launch_strip_gemm(a, true, true, p.mb, p.ks1, p.nbuf1, cus, s, 2);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    {
      StageScope st(s, 2);
      e = moe_host::launch_requant_groups(h32, P, I, R.expert_offsets, E, hq, h_rows, s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    {
      StageScope st(s, 3);
      moe_host::StripArgs a{};
      a.a = hq;
      a.b = w2;
      a.b_scale = w2_scale;
      a.rs_u = h_rows;
      a.sorted_pairs = R.sorted_pairs;
      a.header = R.header;
      a.tasks = R.tasks;
      a.c = ws + W.y;
      a.K = I;
      a.N = H;
      a.P = P;
      a.topk = k;
      a.max_tasks = p.max_tasks;
      a.split = p.split2;
      a.out_bf16 = y_bf16 ? 1 : 0;
      e = moe_host::launch_strip_gemm(a, false, true, p.mb, p.ks2, p.nbuf2, cus, s, 2);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    {
      StageScope st(s, 4);
      e = moe_host::launch_reduce(ws + W.y, y_bf16, p.split2, P, topk_w, R.pair_pos, R.expert_offsets,
                                  nullptr, E, T, k, H, static_cast<uint16_t*>(out), s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    return MOE_OK;
  }
  {
    StageScope st(s, 1);
    moe_host::StreamArgs a{};
    a.a = xq;
    a.b = w1;
    a.b_scale = w1_scale;
    a.row_scale = x_rows;
    a.sorted_pairs = R.sorted_pairs;
    a.header = R.header;
    a.tasks = R.tasks;
    a.c = h32;
    a.P = P;
    a.K = H;
    a.N_out = I;
    a.w_rows = 2 * I;
    a.topk = k;
    a.max_tasks = p.max_tasks;
    e = moe_host::launch_stream_fp8b(a, true, true, p.mb, p.sw1,
                                     stream_grid((long)p.max_tasks * (I / 16) / (p.nb / 2), p.sw1, cus), s,
                                     p.nb);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  {
    StageScope st(s, 2);
    e = moe_host::launch_requant_groups(h32, P, I, R.expert_offsets, E, hq, h_rows, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  {
    StageScope st(s, 3);
    moe_host::StreamArgs a{};
    a.a = hq;
    a.b = w2;
    a.b_scale = w2_scale;
    a.row_scale = h_rows;
    a.sorted_pairs = R.sorted_pairs;
    a.header = R.header;
    a.tasks = R.tasks;
    a.c = ws + W.y;
    a.P = P;
    a.K = I;
    a.N_out = H;
    a.w_rows = H;
    a.topk = k;
    a.max_tasks = p.max_tasks;
    e = moe_host::launch_stream_fp8b(a, false, true, p.mb, p.sw2,
                                     stream_grid((long)p.max_tasks * (H / 16) / p.nb, p.sw2, cus), s, p.nb);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  {
    StageScope st(s, 4);
    e = moe_host::launch_reduce(ws + W.y, true, 1, P, topk_w, R.pair_pos, R.expert_offsets, nullptr,
                                E, T, k, H, static_cast<uint16_t*>(out), s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

// Weight-only forward (int4 w4a16, int8 w8a16): register-streaming gate-up
// (weights converted in registers, SiLU-and-mul in the epilogue, bf16 h),
// down (bf16 rows), the top-k reduction.
int forward_w4(int dtype, const void* x, const float* topk_w, const void* routing, const void* w1,
               const float* w1_scale, const void* w2, const float* w2_scale, int T, int k, int E,
               int H, int I, void* workspace, size_t workspace_bytes, void* out, void* stream,
               const moe_host::DecodeRouteOut* fold = nullptr) {
  int rc = check_shape(T, k, E, H, I, dtype);
  if (rc != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !topk_w || !routing || !w1 || !w2 || !w1_scale || !w2_scale || !workspace || !out)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(out, 16) ||
      !aligned(topk_w, 4) || !aligned(routing, 16) || !aligned(workspace, 256) ||
      !aligned(w1_scale, 4) || !aligned(w2_scale, 4))
    return MOE_ERR_INVALID_ARG;
  const Plan p = make_plan(dtype, T, k, E, H, I);
  moe_routing_layout_t L;
  routing_layout(T, k, E, p, &L);
  moe_workspace_layout_t W;
  workspace_layout(dtype, T, k, H, I, p, &W);
  const bool w8 = dtype == MOE_DTYPE_INT8_W8A16;
  if (workspace_bytes < W.total_bytes) return MOE_ERR_BUFFER_TOO_SMALL;
  int cus = 0;
  if ((rc = cu_count(&cus)) != MOE_OK) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const RoutingView R = view_routing(routing, L);
  char* ws = static_cast<char*>(workspace);
  const int P = T * k;
  hipError_t e;
  {
    StageScope st(s, 1);
    moe_host::StreamArgs a{};
    a.a = x;
    a.b = w1;
    a.b_scale = w1_scale;
    a.sorted_pairs = R.sorted_pairs;
    a.header = R.header;
    a.tasks = R.tasks;
    a.c = ws + W.h;
    a.K = H;
    a.N_out = I;
    a.w_rows = 2 * I;
    a.topk = k;
    a.max_tasks = p.max_tasks;
    a.P = P;
    if (fold) a.route = *fold;
    const int grid = stream_grid((long)p.max_tasks * (I / 16) / (p.nb / 2), p.sw1, cus);
    e = w8 ? moe_host::launch_stream_w8(a, true, p.mb, p.sw1, grid, s, p.nb)
           : moe_host::launch_stream_w4(a, true, p.mb, p.sw1, grid, s, p.nb);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  {
    StageScope st(s, 3);
    moe_host::StreamArgs a{};
    a.a = ws + W.h;
    a.b = w2;
    a.b_scale = w2_scale;
    a.sorted_pairs = R.sorted_pairs;
    a.header = R.header;
    a.tasks = R.tasks;
    a.c = ws + W.y;
    a.K = I;
    a.N_out = H;
    a.w_rows = H;
    a.topk = k;
    a.max_tasks = p.max_tasks;
    const int grid = stream_grid((long)p.max_tasks * (H / 16) / p.nb, p.sw2, cus);
    e = w8 ? moe_host::launch_stream_w8(a, false, p.mb, p.sw2, grid, s, p.nb)
           : moe_host::launch_stream_w4(a, false, p.mb, p.sw2, grid, s, p.nb);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  {
    StageScope st(s, 4);
    e = moe_host::launch_reduce(ws + W.y, true, 1, P, topk_w, R.pair_pos, R.expert_offsets, nullptr,
                                E, T, k, H, static_cast<uint16_t*>(out), s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

// int8 w8a8 forward (per-channel weight scales), register streaming: the
// fp8 streaming sequence with int8 quantisation and the integer MFMA.
int forward_i8(const void* x, const float* topk_w, const void* routing, const void* w1,
               const float* w1_scale, const void* w2, const float* w2_scale, int T, int k, int E,
               int H, int I, void* workspace, size_t workspace_bytes, void* out, void* stream,
               const moe_host::DecodeRouteOut* fold = nullptr) {
  int rc = check_shape(T, k, E, H, I, MOE_DTYPE_INT8_W8A8);
  if (rc != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !topk_w || !routing || !w1 || !w2 || !w1_scale || !w2_scale || !workspace || !out)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(out, 16) ||
      !aligned(topk_w, 4) || !aligned(routing, 16) || !aligned(workspace, 256) ||
      !aligned(w1_scale, 4) || !aligned(w2_scale, 4))
    return MOE_ERR_INVALID_ARG;
  const Plan p = make_plan(MOE_DTYPE_INT8_W8A8, T, k, E, H, I);
  moe_routing_layout_t L;
  routing_layout(T, k, E, p, &L);
  moe_workspace_layout_t W;
  workspace_layout(MOE_DTYPE_INT8_W8A8, T, k, H, I, p, &W);
  if (workspace_bytes < W.total_bytes) return MOE_ERR_BUFFER_TOO_SMALL;
  int cus = 0;
  if ((rc = cu_count(&cus)) != MOE_OK) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const RoutingView R = view_routing(routing, L);
  char* ws = static_cast<char*>(workspace);
  const int P = T * k;
  int8_t* xq = reinterpret_cast<int8_t*>(ws + W.xq);
  float* x_scale = reinterpret_cast<float*>(ws + W.x_scale);
  float* x_rows = reinterpret_cast<float*>(ws + W.x_scale_rows);
  float* h32 = reinterpret_cast<float*>(ws + W.g);
  int8_t* hq = reinterpret_cast<int8_t*>(ws + W.h);
  float* h_scale = reinterpret_cast<float*>(ws + W.h_scale);
  hipError_t e;
  {
    StageScope st(s, 0);
    e = moe_host::launch_quant_rows_i8(static_cast<const uint16_t*>(x), T, H, xq, x_scale, nullptr, k,
                                       R.pair_pos, x_rows, s, fold);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (p.tiling == kStrips) {
    // strips (the fp8 sequence on the integer MFMA): gate-up with SiLU(gate)*up
    // in its epilogue (fp32 h), int8 requantisation, down (bf16 rows, or fp32
    // partial sums of split_k2 slices), reduction
    const bool y_bf16 = p.split2 == 1;
    {
      StageScope st(s, 1);
      moe_host::StripArgs a{};
      a.a = xq;
      a.b = w1;
      a.b_scale = w1_scale;
      a.sorted_pairs = R.sorted_pairs;
      a.header = R.header;
      a.tasks = R.tasks;
      a.c = h32;
      a.K = H;
      a.N = 2 * I;
      a.P = P;
      a.topk = k;
      a.max_tasks = p.max_tasks;
      a.split = 1;
      a.out_bf16 = 0;
      a.act = 1;
      a.x_scale_rows = x_rows;
      a.rotate = rotate_strips(p, false);
      e = moe_host::launch_strip_gemm(a, true, true, p.mb, p.ks1, p.nbuf1, cus, s, 1);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    {
      StageScope st(s, 2);
      e = moe_host::launch_requant_rows_i8(h32, P, I, R.expert_offsets, E, hq, h_scale, s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    {
      StageScope st(s, 3);
      moe_host::StripArgs a{};
      a.a = hq;
      a.b = w2;
      a.b_scale = w2_scale;
      a.sorted_pairs = R.sorted_pairs;
      a.header = R.header;
      a.tasks = R.tasks;
      a.c = ws + W.y;
      a.K = I;
      a.N = H;
      a.P = P;
      a.topk = k;
      a.max_tasks = p.max_tasks;
      a.split = p.split2;
      a.out_bf16 = y_bf16 ? 1 : 0;
      a.rotate = rotate_strips(p, true);
      e = moe_host::launch_strip_gemm(a, false, true, p.mb, p.ks2, p.nbuf2, cus, s, 1);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    {
      StageScope st(s, 4);
      e = moe_host::launch_reduce(ws + W.y, y_bf16, p.split2, P, topk_w, R.pair_pos, R.expert_offsets,
                                  h_scale, E, T, k, H, static_cast<uint16_t*>(out), s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    return MOE_OK;
  }
  {
    StageScope st(s, 1);
    moe_host::StreamArgs a{};
    a.a = xq;
    a.b = w1;
    a.b_scale = w1_scale;
    a.row_scale = x_rows;
    a.sorted_pairs = R.sorted_pairs;
    a.header = R.header;
    a.tasks = R.tasks;
    a.c = h32;
    a.K = H;
    a.N_out = I;
    a.w_rows = 2 * I;
    a.topk = k;
    a.max_tasks = p.max_tasks;
    e = moe_host::launch_stream_gemm(a, true, true, 2, p.mb, p.sw1, p.su1,
                                     stream_grid((long)p.max_tasks * (I / 16) / (p.nb / 2), p.sw1, cus), s,
                                     p.nb);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  {
    StageScope st(s, 2);
    e = moe_host::launch_requant_rows_i8(h32, P, I, R.expert_offsets, E, hq, h_scale, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  {
    StageScope st(s, 3);
    moe_host::StreamArgs a{};
    a.a = hq;
    a.b = w2;
    a.b_scale = w2_scale;
    a.sorted_pairs = R.sorted_pairs;
    a.header = R.header;
    a.tasks = R.tasks;
    a.c = p.dr_waves ? nullptr : ws + W.y;
    a.K = I;
    a.N_out = H;
    a.w_rows = H;
    a.topk = k;
    a.max_tasks = p.max_tasks;
    a.P = P;
    if (p.dr_waves)   // one token: the down launch adds the top-k rows itself
      e = moe_host::launch_stream_down_reduce(a, true, p.dr_waves, p.dr_u, p.dr_half, topk_w, h_scale,
                                              static_cast<uint16_t*>(out), s, true);
    else
      e = moe_host::launch_stream_gemm(a, false, true, 2, p.mb, p.sw2, p.su2,
                                       stream_grid((long)p.max_tasks * (H / 16) / p.nb, p.sw2, cus), s, p.nb);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (!p.dr_waves) {
    StageScope st(s, 4);
    e = moe_host::launch_reduce(ws + W.y, true, 1, P, topk_w, R.pair_pos, R.expert_offsets, h_scale,
                                E, T, k, H, static_cast<uint16_t*>(out), s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

// Pointer, alignment and workspace-size rules of a forward pass of any dtype
// (checked before anything is launched).
int check_forward_args(int dtype, const void* x, const float* topk_w, const void* routing, const void* w1,
                       const void* w1_scale, const void* w2, const void* w2_scale, int T, int k, int E,
                       int H, int I, const void* workspace, size_t workspace_bytes, const void* out) {
  const bool generic = dtype == MOE_DTYPE_BF16 || dtype == MOE_DTYPE_FP8_W8A8;
  const int rc = generic ? check_shape(T, k, E, H, I) : check_shape(T, k, E, H, I, dtype);
  if (rc != MOE_OK || T == 0) return rc;
  const bool scaled = dtype != MOE_DTYPE_BF16;   // per-channel, block or MX scales
  if (!x || !topk_w || !routing || !w1 || !w2 || !workspace || !out) return MOE_ERR_INVALID_ARG;
  if (scaled && (!w1_scale || !w2_scale)) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(out, 16) ||
      !aligned(topk_w, 4) || !aligned(routing, 16) || !aligned(workspace, 256))
    return MOE_ERR_INVALID_ARG;
  if (scaled && (!aligned(w1_scale, 4) || !aligned(w2_scale, 4))) return MOE_ERR_INVALID_ARG;
  const Plan p = make_plan(dtype, T, k, E, H, I);
  if (dtype == MOE_DTYPE_MXFP8 && p.tiling == kStreaming && (p.su1 != 2 || p.su2 != 2))
    return MOE_ERR_UNSUPPORTED_SHAPE;
  moe_workspace_layout_t W;
  workspace_layout(dtype, T, k, H, I, p, &W);
  return workspace_bytes < W.total_bytes ? MOE_ERR_BUFFER_TOO_SMALL : MOE_OK;
}

// fold: the routing build of a decode token done by the forward's first
// kernel (fp8: the x quantisation, bf16: the gate-up), which writes the
// routing buffer for the kernels after it.
int forward(int dtype, const void* x, const float* topk_w, const void* routing, const void* w1,
            const float* w1_scale, const void* w2, const float* w2_scale, int T, int k, int E,
            int H, int I, void* workspace, size_t workspace_bytes, void* out, void* stream,
            const moe_host::DecodeRouteOut* fold = nullptr) {
  int rc = check_forward_args(dtype, x, topk_w, routing, w1, w1_scale, w2, w2_scale, T, k, E, H, I,
                              workspace, workspace_bytes, out);
  if (rc != MOE_OK || T == 0) return rc;
  const bool fp8 = dtype == MOE_DTYPE_FP8_W8A8;

  const Plan p = make_plan(dtype, T, k, E, H, I);
  moe_routing_layout_t L;
  routing_layout(T, k, E, p, &L);
  moe_workspace_layout_t W;
  workspace_layout(dtype, T, k, H, I, p, &W);
  if (fold && ((long)T * k > moe::kDecodeRoutePairs || p.tiling != kStreaming)) return MOE_ERR_INVALID_ARG;
  int cus = 0;
  if ((rc = cu_count(&cus)) != MOE_OK) return rc;

  const hipStream_t s = static_cast<hipStream_t>(stream);
  const RoutingView R = view_routing(routing, L);
  char* ws = static_cast<char*>(workspace);
  const int P = T * k;
  void* h = ws + W.h;
  float* h_scale = fp8 ? reinterpret_cast<float*>(ws + W.h_scale) : nullptr;
  uint8_t* xq = fp8 ? reinterpret_cast<uint8_t*>(ws + W.xq) : nullptr;
  float* x_scale = fp8 ? reinterpret_cast<float*>(ws + W.x_scale) : nullptr;
  hipError_t e = hipSuccess;

  if (fp8) {
    StageScope st(s, 0);
    // the row amax slots are cleared here for the epilogue that folds into
    // them (LDS tiles; the streaming and strip requantisation finds the amax
    // itself); the per-sorted-row x scales serve the epilogues that apply them
    e = moe_host::launch_quant_rows_bf16(
        static_cast<const uint16_t*>(x), T, H, xq, x_scale,
        p.tiling == kLdsTiles ? h_scale : nullptr,
        k, R.pair_pos, W.x_scale_rows != kNone ? reinterpret_cast<float*>(ws + W.x_scale_rows) : nullptr,
        s, fold);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (p.tiling == kStrips) {
    float* g = W.g == kNone ? nullptr : reinterpret_cast<float*>(ws + W.g);
    const bool y_bf16 = p.split2 == 1;
    // One gate-up slice: SiLU-and-mul in the GEMM's epilogue (fp8: fp32 h,
    // then the requantisation pass); else fp32 partial sums that the
    // activation kernel adds (and, on fp8, requantises).
    const bool fuse_act = p.split1 == 1;
    {
      StageScope st(s, 1);
      moe_host::StripArgs a{};
      a.a = fp8 ? static_cast<const void*>(xq) : x;
      a.b = w1;
      a.b_scale = w1_scale;
      a.sorted_pairs = R.sorted_pairs;
      a.header = R.header;
      a.tasks = R.tasks;
      a.c = fuse_act && !fp8 ? h : static_cast<void*>(g);
      a.K = H;
      a.N = 2 * I;
      a.P = P;
      a.topk = k;
      a.max_tasks = p.max_tasks;
      a.split = p.split1;
      a.out_bf16 = 0;
      a.act = fuse_act ? 1 : 0;
      a.x_scale_rows = fuse_act && fp8 ? reinterpret_cast<const float*>(ws + W.x_scale_rows) : nullptr;
      a.rotate = rotate_strips(p, false);
      e = moe_host::launch_strip_gemm(a, true, fp8, p.mb, p.ks1, p.nbuf1, cus, s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    if (!fuse_act) {
      StageScope st(s, 2);
      e = moe_host::launch_act(g, p.split1, P, I, R.expert_offsets, E, fp8, x_scale,
                               R.sorted_pairs, k, h, h_scale, s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    } else if (fp8) {
      StageScope st(s, 2);
      e = moe_host::launch_requant_rows(g, P, I, R.expert_offsets, E, static_cast<uint8_t*>(h), h_scale,
                                        true, s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    {
      StageScope st(s, 3);
      moe_host::StripArgs a{};
      a.a = h;
      a.b = w2;
      a.b_scale = w2_scale;
      a.sorted_pairs = R.sorted_pairs;
      a.header = R.header;
      a.tasks = R.tasks;
      a.c = ws + W.y;
      a.K = I;
      a.N = H;
      a.P = P;
      a.topk = k;
      a.max_tasks = p.max_tasks;
      a.split = p.split2;
      a.out_bf16 = y_bf16 ? 1 : 0;
      a.rotate = rotate_strips(p, true);
      e = moe_host::launch_strip_gemm(a, false, fp8, p.mb, p.ks2, p.nbuf2, cus, s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    {
      StageScope st(s, 4);
      e = moe_host::launch_reduce(ws + W.y, y_bf16, p.split2, P, topk_w, R.pair_pos,
                                  R.expert_offsets, h_scale, E, T, k, H,
                                  static_cast<uint16_t*>(out), s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    return MOE_OK;
  }
  if (p.tiling == kLdsTiles) {
    const int grid1 = p.bn1 == 256 ? cus : cus * 2;   // a direct-to-LDS ring fits once per CU
    const int grid2 = p.bn2 == 256 ? cus : cus * 2;
    float* h32 = fp8 ? reinterpret_cast<float*>(ws + W.g) : nullptr;
    {
      StageScope st(s, 1);
      moe_host::TiledArgs a{};
      a.a = fp8 ? static_cast<const void*>(xq) : x;
      a.a_scale = x_scale;
      a.b = w1;
      a.b_scale = w1_scale;
      a.sorted_pairs = R.sorted_pairs;
      a.header = R.header;
      a.tasks = R.tasks;
      a.c = fp8 ? static_cast<void*>(h32) : h;
      a.row_amax = h_scale;
      a.K = H;
      a.N_out = I;
      a.w_rows = 2 * I;
      a.topk = k;
      a.max_tasks = p.max_tasks;
      e = moe_host::launch_tiled_gemm(a, true, fp8, p.bm_t, p.bn1, grid1, s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    {
      StageScope st(s, 2);
      if (fp8) {
        e = moe_host::launch_requant_rows(h32, P, I, R.expert_offsets, E,
                                          static_cast<uint8_t*>(h), h_scale, false, s);
        if (e != hipSuccess) return MOE_ERR_HIP;
      }
    }
    {
      StageScope st(s, 3);
      moe_host::TiledArgs a{};
      a.a = h;
      a.a_scale = h_scale;
      a.b = w2;
      a.b_scale = w2_scale;
      a.sorted_pairs = R.sorted_pairs;
      a.header = R.header;
      a.tasks = R.tasks;
      a.c = ws + W.y;
      a.K = I;
      a.N_out = H;
      a.w_rows = H;
      a.topk = k;
      a.max_tasks = p.max_tasks;
      e = moe_host::launch_tiled_gemm(a, false, fp8, p.bm_t, p.bn2, grid2, s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    {
      StageScope st(s, 4);
      e = moe_host::launch_reduce(ws + W.y, true, 1, P, topk_w, R.pair_pos, R.expert_offsets,
                                  nullptr, E, T, k, H, static_cast<uint16_t*>(out), s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    return MOE_OK;
  }

  // Register streaming: the gate-up epilogue forms SiLU(gate)*up (bf16 h, or
  // fp32 h + row amax then requantised on fp8); down writes bf16 rows.
  float* h32 = fp8 ? reinterpret_cast<float*>(ws + W.g) : nullptr;
  {
    StageScope st(s, 1);
    moe_host::StreamArgs a{};
    a.a = fp8 ? static_cast<const void*>(xq) : x;
    a.b = w1;
    a.b_scale = w1_scale;
    a.row_scale = fp8 ? reinterpret_cast<const float*>(ws + W.x_scale_rows) : nullptr;
    a.sorted_pairs = R.sorted_pairs;
    a.header = R.header;
    a.tasks = R.tasks;
    a.c = fp8 ? static_cast<void*>(h32) : h;
    a.K = H;
    a.N_out = I;
    a.w_rows = 2 * I;
    a.topk = k;
    a.max_tasks = p.max_tasks;
    a.P = P;
    if (fold && !fp8) a.route = *fold;
    if (p.half1)
      e = moe_host::launch_stream_half_gateup(a, p.sw1, stream_grid((long)p.max_tasks * (I / 8), p.sw1, cus), s);
    else if (p.fp8_units)
      e = moe_host::launch_stream_fp8b(a, true, false, p.mb, p.sw1,
                                       stream_grid((long)p.max_tasks * (I / 16), p.sw1, cus), s);
    else
      e = moe_host::launch_stream_gemm(a, true, fp8, 0, p.mb, p.sw1, p.su1,
                                       stream_grid((long)p.max_tasks * (I / 16) / (p.nb / 2), p.sw1, cus), s,
                                       p.nb);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (fp8) {
    StageScope st(s, 2);
    e = moe_host::launch_requant_rows(h32, P, I, R.expert_offsets, E, static_cast<uint8_t*>(h),
                                      h_scale, true, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  {
    StageScope st(s, 3);
    moe_host::StreamArgs a{};
    a.a = h;
    a.b = w2;
    a.b_scale = w2_scale;
    a.sorted_pairs = R.sorted_pairs;
    a.header = R.header;
    a.tasks = R.tasks;
    a.c = p.dr_waves ? nullptr : ws + W.y;
    a.K = I;
    a.N_out = H;
    a.w_rows = H;
    a.topk = k;
    a.max_tasks = p.max_tasks;
    a.P = P;
    if (p.dr_waves)
      e = moe_host::launch_stream_down_reduce(a, fp8, p.dr_waves, p.dr_u, p.dr_half, topk_w,
                                              fp8 ? h_scale : nullptr, static_cast<uint16_t*>(out), s);
    else if (p.fp8_units)
      e = moe_host::launch_stream_fp8b(a, false, false, p.mb, p.sw2,
                                       stream_grid((long)p.max_tasks * (H / 32), p.sw2, cus), s);
    else
      e = moe_host::launch_stream_gemm(a, false, fp8, 0, p.mb, p.sw2, p.su2,
                                       stream_grid((long)p.max_tasks * (H / 16) / p.nb, p.sw2, cus), s, p.nb);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  {
    StageScope st(s, 4);   // empty when the down launch added the top-k rows
    if (!p.dr_waves) {
      e = moe_host::launch_reduce(ws + W.y, true, 1, P, topk_w, R.pair_pos, R.expert_offsets,
                                  fp8 ? h_scale : nullptr, E, T, k, H, static_cast<uint16_t*>(out), s);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
  }
  return MOE_OK;
}

// Routing build and forward pass in one call.  A decode batch of at most 64
// pairs on the register-streaming plan is routed inside the forward's first
// kernel (the x quantisation on the dtypes with quantised activations, the
// gate-up GEMM on bf16); otherwise the routing build runs as its own launch
// first.  Every dtype of the forward calls.
int route_forward(int dtype, const int32_t* ids, const void* x, const float* topk_w, void* routing,
                  size_t routing_bytes, const void* w1, const void* w1_scale, const void* w2,
                  const void* w2_scale, int T, int k, int E, int H, int I, void* workspace,
                  size_t workspace_bytes, void* out, void* stream) {
  int rc = check_forward_args(dtype, x, topk_w, routing, w1, w1_scale, w2, w2_scale, T, k, E, H, I,
                              workspace, workspace_bytes, out);
  if (rc != MOE_OK || T == 0) return rc;
  if (!ids || !aligned(ids, 4)) return MOE_ERR_INVALID_ARG;
  const Plan p = make_plan(dtype, T, k, E, H, I);
  moe_routing_layout_t L;
  routing_layout(T, k, E, p, &L);
  if (routing_bytes < L.total_bytes) return MOE_ERR_BUFFER_TOO_SMALL;
  auto run = [&](const moe_host::DecodeRouteOut* f) {
    const float* s1 = static_cast<const float*>(w1_scale);
    const float* s2 = static_cast<const float*>(w2_scale);
    switch (dtype) {
      case MOE_DTYPE_INT8_W8A8:
        return forward_i8(x, topk_w, routing, w1, s1, w2, s2, T, k, E, H, I, workspace, workspace_bytes, out,
                          stream, f);
      case MOE_DTYPE_FP8_BLOCK:
        return forward_fp8b(x, topk_w, routing, w1, s1, w2, s2, T, k, E, H, I, workspace, workspace_bytes,
                            out, stream, f);
      case MOE_DTYPE_MXFP8:
        return forward_mx(x, topk_w, routing, w1, static_cast<const uint8_t*>(w1_scale), w2,
                          static_cast<const uint8_t*>(w2_scale), T, k, E, H, I, workspace, workspace_bytes,
                          out, stream, f);
      case MOE_DTYPE_INT4_W4A16:
      case MOE_DTYPE_INT8_W8A16:
        return forward_w4(dtype, x, topk_w, routing, w1, s1, w2, s2, T, k, E, H, I, workspace, workspace_bytes,
                          out, stream, f);
      default:
        return forward(dtype, x, topk_w, routing, w1, s1, w2, s2, T, k, E, H, I, workspace,
                       workspace_bytes, out, stream, f);
    }
  };
  // the x quantisation comes first and takes any plan; bf16 activations
  // (bf16, int4 and int8 weights): the gate-up kernels on 16-row tiles with
  // two weight blocks per item (bf16 also the half-width items)
  const bool bf16_act = dtype == MOE_DTYPE_BF16 || dtype == MOE_DTYPE_INT4_W4A16 || dtype == MOE_DTYPE_INT8_W8A16;
  const bool first_takes_it = !bf16_act || (p.mb == 1 && (p.nb == 2 || (dtype == MOE_DTYPE_BF16 && p.half1)));
  if ((long)T * k <= moe::kDecodeRoutePairs && p.tiling == kStreaming && first_takes_it) {
    char* b = static_cast<char*>(routing);
    moe_host::DecodeRouteOut f;
    f.ids = ids;
    f.header = reinterpret_cast<int32_t*>(b + L.header);
    f.expert_offsets = reinterpret_cast<int32_t*>(b + L.expert_offsets);
    f.sorted_pairs = reinterpret_cast<int32_t*>(b + L.sorted_pairs);
    f.pair_pos = reinterpret_cast<int32_t*>(b + L.pair_pos);
    f.tasks = reinterpret_cast<moe_task_t*>(b + L.tasks);
    f.E = E;
    f.block_m = p.block_m;
    f.max_tasks = p.max_tasks;
    return run(&f);
  }
  rc = build_routing(dtype, ids, T, k, E, H, I, routing, routing_bytes, stream);
  if (rc != MOE_OK) return rc;
  return run(nullptr);
}

// Shape and pointer rules of a packed weight tensor; its row length in bytes.
int packed_shape(const void* packed, int E, int rows, int cols, int dtype, long* row_bytes) {
  if (!known_dtype(dtype)) return MOE_ERR_INVALID_ARG;
  if (E < 1 || rows < 1 || cols < 1) return MOE_ERR_INVALID_ARG;
  const long rb = dtype == MOE_DTYPE_INT4_W4A16 ? (long)cols / 2
                                                : (long)cols * (dtype == MOE_DTYPE_BF16 ? 2 : 1);
  if (dtype == MOE_DTYPE_INT4_W4A16 && cols % 2) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (rows % 16 || rb % 64 || rows > 2 * 65536 || cols > 65536) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (!packed || !aligned(packed, 16)) return MOE_ERR_INVALID_ARG;
  *row_bytes = rb;
  return MOE_OK;
}

void describe(const void* packed, int E, int rows, int cols, int dtype, moe_packed_weights_t* desc) {
  moe_packed_weights_t d{};
  d.data = packed;
  d.dtype = dtype;
  d.experts = E;
  d.rows = rows;
  d.cols = cols;
  d.check = packed_check(d);
  *desc = d;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case MOE_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int moe_routing_layout(int T, int k, int E, int H, int I, int dtype, moe_routing_layout_t* out) {
  if (!out || !known_dtype(dtype)) return MOE_ERR_INVALID_ARG;
  const int rc = check_shape(T, k, E, H, I, dtype);
  if (rc != MOE_OK) return rc;
  routing_layout(T, k, E, make_plan(dtype, T, k, E, H, I), out);
  return MOE_OK;
}

int moe_workspace_layout(int T, int k, int E, int H, int I, int dtype, moe_workspace_layout_t* out) {
  if (!out || !known_dtype(dtype)) return MOE_ERR_INVALID_ARG;
  const int rc = check_shape(T, k, E, H, I, dtype);
  if (rc != MOE_OK) return rc;
  workspace_layout(dtype, T, k, H, I, make_plan(dtype, T, k, E, H, I), out);
  return MOE_OK;
}

int moe_pack_weights(const void* w, int E, int rows, int cols, int dtype, void* packed,
                     moe_packed_weights_t* desc, void* stream) {
  if (!desc) return MOE_ERR_INVALID_ARG;
  long row_bytes = 0;
  const int rc = packed_shape(packed, E, rows, cols, dtype, &row_bytes);
  if (rc != MOE_OK) return rc;
  if (!w || !aligned(w, 16)) return MOE_ERR_INVALID_ARG;
  const size_t total = (size_t)E * rows * row_bytes;
  const char* a = static_cast<const char*>(w);
  const char* b = static_cast<const char*>(packed);
  if (a < b + total && b < a + total) return MOE_ERR_INVALID_ARG;   // overlap
  const hipError_t e = moe_host::launch_pack(w, E, rows, (int)row_bytes, packed,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return MOE_ERR_HIP;
  describe(packed, E, rows, cols, dtype, desc);
  return MOE_OK;
}

int moe_describe_packed_weights(const void* packed, int E, int rows, int cols, int dtype,
                                moe_packed_weights_t* desc) {
  if (!desc) return MOE_ERR_INVALID_ARG;
  long row_bytes = 0;
  const int rc = packed_shape(packed, E, rows, cols, dtype, &row_bytes);
  if (rc != MOE_OK) return rc;
  describe(packed, E, rows, cols, dtype, desc);
  return MOE_OK;
}

int moe_build_routing_bf16(const int32_t* topk_ids, int T, int k, int E, int H, int I,
                           void* routing, size_t routing_bytes, void* stream) {
  return build_routing(MOE_DTYPE_BF16, topk_ids, T, k, E, H, I, routing, routing_bytes, stream);
}

int moe_build_routing_fp8(const int32_t* topk_ids, int T, int k, int E, int H, int I,
                          void* routing, size_t routing_bytes, void* stream) {
  return build_routing(MOE_DTYPE_FP8_W8A8, topk_ids, T, k, E, H, I, routing, routing_bytes,
                       stream);
}

int moe_router_topk(const float* logits, int T, int E, int k, int renormalize, int n_shared,
                    int32_t* topk_ids, float* topk_w, void* stream) {
  if (T < 0 || E < 1 || k < 1 || k > E || n_shared < 0 || (renormalize != 0 && renormalize != 1))
    return MOE_ERR_INVALID_ARG;
  if (E > moe_host::router_max_experts() || k + n_shared > moe::kMaxTopK ||
      E + n_shared > moe::kMaxExperts)
    return MOE_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4)) return MOE_ERR_INVALID_ARG;
  const hipError_t e = moe_host::launch_router_topk(logits, 1, nullptr, T, E, k, renormalize, n_shared,
                                                    topk_ids, topk_w, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_router_pair_bytes(int N, int K, size_t* bytes) {
  if (!bytes || N < 1 || K < 1) return MOE_ERR_INVALID_ARG;
  if (K % 64 || K > 65536 || N > 65536) return MOE_ERR_UNSUPPORTED_SHAPE;
  *bytes = (size_t)4 * ((N + 15) / 16 * 16) * K;
  return MOE_OK;
}

int moe_router_split_weights(const float* w, int N, int K, void* w_pair, size_t w_pair_bytes,
                             void* stream) {
  size_t need = 0;
  const int rc = moe_router_pair_bytes(N, K, &need);
  if (rc != MOE_OK) return rc;
  if (!w || !w_pair || !aligned(w, 4) || !aligned(w_pair, 16)) return MOE_ERR_INVALID_ARG;
  if (w_pair_bytes < need) return MOE_ERR_BUFFER_TOO_SMALL;
  const hipError_t e = moe_host::launch_router_split(w, N, K, w_pair, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_router_workspace_bytes(int T, int N, int K, size_t* bytes) {
  if (!bytes || T < 0 || N < 1 || K < 1) return MOE_ERR_INVALID_ARG;
  if (K % 64 || K > 65536 || N > 65536) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) {
    *bytes = 0;
    return MOE_OK;
  }
  const moe_host::RouterGemmPlan p = moe_host::plan_router_gemm(T, N, K, kPlanCUs);
  *bytes = (size_t)std::max(p.S, 1) * T * N * 4;
  return MOE_OK;
}

int router_gemm_common(const void* x, const void* w_pair, int T, int N, int K, void* workspace,
                       size_t workspace_bytes, moe_host::RouterGemmPlan* plan) {
  size_t need = 0;
  const int rc = moe_router_workspace_bytes(T, N, K, &need);
  if (rc != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !w_pair || !aligned(x, 16) || !aligned(w_pair, 16)) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < need) return MOE_ERR_BUFFER_TOO_SMALL;
  if (need && (!workspace || !aligned(workspace, 16))) return MOE_ERR_INVALID_ARG;
  *plan = moe_host::plan_router_gemm(T, N, K, kPlanCUs);
  return MOE_OK;
}

int moe_router_gemm(const void* x, const void* w_pair, int T, int N, int K, void* workspace,
                    size_t workspace_bytes, float* scores, void* stream) {
  moe_host::RouterGemmPlan p;
  const int rc = router_gemm_common(x, w_pair, T, N, K, workspace, workspace_bytes, &p);
  if (rc != MOE_OK || T == 0) return rc;
  if (!scores || !aligned(scores, 4)) return MOE_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  float* planes = static_cast<float*>(workspace);
  hipError_t e = moe_host::launch_router_gemm(x, w_pair, T, N, K, p, p.S > 1 ? planes : scores, s);
  if (e == hipSuccess && p.S > 1) e = moe_host::launch_router_reduce(planes, p.S, T, N, scores, s);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_router_gemm_topk(const void* x, const void* w_pair, int T, int E, int K, int k,
                         int renormalize, int n_shared, void* workspace, size_t workspace_bytes,
                         float* scores, int32_t* topk_ids, float* topk_w, void* stream) {
  if (T < 0 || E < 1 || k < 1 || k > E || n_shared < 0 || (renormalize != 0 && renormalize != 1))
    return MOE_ERR_INVALID_ARG;
  if (E > moe_host::router_max_experts() || k + n_shared > moe::kMaxTopK ||
      E + n_shared > moe::kMaxExperts)
    return MOE_ERR_UNSUPPORTED_SHAPE;
  moe_host::RouterGemmPlan p;
  const int rc = router_gemm_common(x, w_pair, T, E, K, workspace, workspace_bytes, &p);
  if (rc != MOE_OK || T == 0) return rc;
  if (!topk_ids || !topk_w || !aligned(topk_ids, 4) || !aligned(topk_w, 4)) return MOE_ERR_INVALID_ARG;
  if (scores && !aligned(scores, 4)) return MOE_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the GEMM's planes (or, unsplit, its scores) go to the workspace; the
  // top-k kernel adds the planes and writes the scores when asked
  float* planes = static_cast<float*>(workspace);
  hipError_t e = moe_host::launch_router_gemm(x, w_pair, T, E, K, p, planes, s);
  if (e == hipSuccess)
    e = moe_host::launch_router_topk(planes, p.S, scores, T, E, k, renormalize, n_shared, topk_ids,
                                     topk_w, s);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_build_routing_mxfp8(const int32_t* topk_ids, int T, int k, int E, int H, int I,
                            void* routing, size_t routing_bytes, void* stream) {
  return build_routing(MOE_DTYPE_MXFP8, topk_ids, T, k, E, H, I, routing, routing_bytes, stream);
}

int moe_forward_mxfp8(const void* x, const float* topk_w, const void* routing, const moe_packed_weights_t* w1,
    const uint8_t* w1_scale, const moe_packed_weights_t* w2, const uint8_t* w2_scale, int T, int k, int E,
    int H, int I, void* workspace, size_t workspace_bytes, void* out, void* stream) {
  const int rc = check_packed(MOE_DTYPE_MXFP8, w1, w2, T, k, E, H, I);
  if (rc != MOE_OK || T == 0) return rc;
  return forward_mx(x, topk_w, routing, packed_data(w1), w1_scale, packed_data(w2), w2_scale, T, k, E, H, I, workspace,
                    workspace_bytes, out, stream);
}

int moe_build_routing_fp8_block(const int32_t* topk_ids, int T, int k, int E, int H, int I,
                                void* routing, size_t routing_bytes, void* stream) {
  return build_routing(MOE_DTYPE_FP8_BLOCK, topk_ids, T, k, E, H, I, routing, routing_bytes, stream);
}

int moe_forward_fp8_block(const void* x, const float* topk_w, const void* routing, const moe_packed_weights_t* w1,
    const float* w1_scale, const moe_packed_weights_t* w2, const float* w2_scale, int T, int k, int E,
    int H, int I, void* workspace, size_t workspace_bytes, void* out, void* stream) {
  const int rc = check_packed(MOE_DTYPE_FP8_BLOCK, w1, w2, T, k, E, H, I);
  if (rc != MOE_OK || T == 0) return rc;
  return forward_fp8b(x, topk_w, routing, packed_data(w1), w1_scale, packed_data(w2), w2_scale, T, k, E, H, I,
                      workspace, workspace_bytes, out, stream);
}

int moe_build_routing_int4(const int32_t* topk_ids, int T, int k, int E, int H, int I,
                           void* routing, size_t routing_bytes, void* stream) {
  return build_routing(MOE_DTYPE_INT4_W4A16, topk_ids, T, k, E, H, I, routing, routing_bytes, stream);
}

int moe_forward_int4(const void* x, const float* topk_w, const void* routing, const moe_packed_weights_t* w1,
    const float* w1_scale, const moe_packed_weights_t* w2, const float* w2_scale, int T, int k, int E,
    int H, int I, void* workspace, size_t workspace_bytes, void* out, void* stream) {
  const int rc = check_packed(MOE_DTYPE_INT4_W4A16, w1, w2, T, k, E, H, I);
  if (rc != MOE_OK || T == 0) return rc;
  return forward_w4(MOE_DTYPE_INT4_W4A16, x, topk_w, routing, packed_data(w1), w1_scale, packed_data(w2), w2_scale, T,
                    k, E, H, I, workspace, workspace_bytes, out, stream);
}

int moe_build_routing_int8_w8a16(const int32_t* topk_ids, int T, int k, int E, int H, int I,
                                 void* routing, size_t routing_bytes, void* stream) {
  return build_routing(MOE_DTYPE_INT8_W8A16, topk_ids, T, k, E, H, I, routing, routing_bytes, stream);
}

int moe_forward_int8_w8a16(const void* x, const float* topk_w, const void* routing, const moe_packed_weights_t* w1,
    const float* w1_scale, const moe_packed_weights_t* w2, const float* w2_scale, int T, int k, int E,
    int H, int I, void* workspace, size_t workspace_bytes, void* out, void* stream) {
  const int rc = check_packed(MOE_DTYPE_INT8_W8A16, w1, w2, T, k, E, H, I);
  if (rc != MOE_OK || T == 0) return rc;
  return forward_w4(MOE_DTYPE_INT8_W8A16, x, topk_w, routing, packed_data(w1), w1_scale, packed_data(w2), w2_scale,
                    T, k, E, H, I, workspace, workspace_bytes, out, stream);
}

int moe_build_routing_int8(const int32_t* topk_ids, int T, int k, int E, int H, int I,
                           void* routing, size_t routing_bytes, void* stream) {
  return build_routing(MOE_DTYPE_INT8_W8A8, topk_ids, T, k, E, H, I, routing, routing_bytes, stream);
}

int moe_forward_int8(const void* x, const float* topk_w, const void* routing, const moe_packed_weights_t* w1,
    const float* w1_scale, const moe_packed_weights_t* w2, const float* w2_scale, int T, int k, int E,
    int H, int I, void* workspace, size_t workspace_bytes, void* out, void* stream) {
  const int rc = check_packed(MOE_DTYPE_INT8_W8A8, w1, w2, T, k, E, H, I);
  if (rc != MOE_OK || T == 0) return rc;
  return forward_i8(x, topk_w, routing, packed_data(w1), w1_scale, packed_data(w2), w2_scale, T, k, E, H, I, workspace,
                    workspace_bytes, out, stream);
}

int moe_forward_bf16(const void* x, const float* topk_w, const void* routing,
                     const moe_packed_weights_t* w1, const moe_packed_weights_t* w2, int T, int k, int E,
                     int H, int I, void* workspace, size_t workspace_bytes, void* out, void* stream) {
  const int rc = check_packed(MOE_DTYPE_BF16, w1, w2, T, k, E, H, I);
  if (rc != MOE_OK || T == 0) return rc;
  return forward(MOE_DTYPE_BF16, x, topk_w, routing, packed_data(w1), nullptr, packed_data(w2), nullptr, T,
                 k, E, H, I, workspace, workspace_bytes, out, stream);
}

int moe_forward_fp8(const void* x, const float* topk_w, const void* routing, const moe_packed_weights_t* w1,
    const float* w1_scale, const moe_packed_weights_t* w2, const float* w2_scale, int T, int k, int E,
    int H, int I, void* workspace, size_t workspace_bytes, void* out, void* stream) {
  const int rc = check_packed(MOE_DTYPE_FP8_W8A8, w1, w2, T, k, E, H, I);
  if (rc != MOE_OK || T == 0) return rc;
  return forward(MOE_DTYPE_FP8_W8A8, x, topk_w, routing, packed_data(w1), w1_scale, packed_data(w2), w2_scale, T, k,
                 E, H, I, workspace, workspace_bytes, out, stream);
}

int moe_route_forward_bf16(const int32_t* topk_ids, const void* x, const float* topk_w, void* routing,
                           size_t routing_bytes, const moe_packed_weights_t* w1, const moe_packed_weights_t* w2,
                           int T, int k, int E, int H, int I, void* workspace, size_t workspace_bytes,
                           void* out, void* stream) {
  const int rc = check_packed(MOE_DTYPE_BF16, w1, w2, T, k, E, H, I);
  if (rc != MOE_OK || T == 0) return rc;
  return route_forward(MOE_DTYPE_BF16, topk_ids, x, topk_w, routing, routing_bytes, packed_data(w1), nullptr,
                       packed_data(w2), nullptr, T, k, E, H, I, workspace, workspace_bytes, out, stream);
}

int moe_route_forward_fp8(const int32_t* topk_ids, const void* x, const float* topk_w, void* routing,
                          size_t routing_bytes, const moe_packed_weights_t* w1, const float* w1_scale,
                          const moe_packed_weights_t* w2, const float* w2_scale, int T, int k, int E, int H,
                          int I, void* workspace, size_t workspace_bytes, void* out, void* stream) {
  const int rc = check_packed(MOE_DTYPE_FP8_W8A8, w1, w2, T, k, E, H, I);
  if (rc != MOE_OK || T == 0) return rc;
  return route_forward(MOE_DTYPE_FP8_W8A8, topk_ids, x, topk_w, routing, routing_bytes, packed_data(w1),
                       w1_scale, packed_data(w2), w2_scale, T, k, E, H, I, workspace, workspace_bytes, out,
                       stream);
}

int moe_route_forward_int8(const int32_t* topk_ids, const void* x, const float* topk_w, void* routing,
                           size_t routing_bytes, const moe_packed_weights_t* w1, const float* w1_scale,
                           const moe_packed_weights_t* w2, const float* w2_scale, int T, int k, int E, int H,
                           int I, void* workspace, size_t workspace_bytes, void* out, void* stream) {
  const int rc = check_packed(MOE_DTYPE_INT8_W8A8, w1, w2, T, k, E, H, I);
  if (rc != MOE_OK || T == 0) return rc;
  return route_forward(MOE_DTYPE_INT8_W8A8, topk_ids, x, topk_w, routing, routing_bytes, packed_data(w1),
                       w1_scale, packed_data(w2), w2_scale, T, k, E, H, I, workspace, workspace_bytes, out,
                       stream);
}

int moe_route_forward_fp8_block(const int32_t* topk_ids, const void* x, const float* topk_w, void* routing,
                                size_t routing_bytes, const moe_packed_weights_t* w1, const float* w1_scale,
                                const moe_packed_weights_t* w2, const float* w2_scale, int T, int k, int E,
                                int H, int I, void* workspace, size_t workspace_bytes, void* out,
                                void* stream) {
  const int rc = check_packed(MOE_DTYPE_FP8_BLOCK, w1, w2, T, k, E, H, I);
  if (rc != MOE_OK || T == 0) return rc;
  return route_forward(MOE_DTYPE_FP8_BLOCK, topk_ids, x, topk_w, routing, routing_bytes, packed_data(w1),
                       w1_scale, packed_data(w2), w2_scale, T, k, E, H, I, workspace, workspace_bytes, out,
                       stream);
}

int moe_route_forward_mxfp8(const int32_t* topk_ids, const void* x, const float* topk_w, void* routing,
                            size_t routing_bytes, const moe_packed_weights_t* w1, const uint8_t* w1_scale,
                            const moe_packed_weights_t* w2, const uint8_t* w2_scale, int T, int k, int E, int H,
                            int I, void* workspace, size_t workspace_bytes, void* out, void* stream) {
  const int rc = check_packed(MOE_DTYPE_MXFP8, w1, w2, T, k, E, H, I);
  if (rc != MOE_OK || T == 0) return rc;
  return route_forward(MOE_DTYPE_MXFP8, topk_ids, x, topk_w, routing, routing_bytes, packed_data(w1),
                       w1_scale, packed_data(w2), w2_scale, T, k, E, H, I, workspace, workspace_bytes, out,
                       stream);
}

int moe_route_forward_int4(const int32_t* topk_ids, const void* x, const float* topk_w, void* routing,
                           size_t routing_bytes, const moe_packed_weights_t* w1, const float* w1_scale,
                           const moe_packed_weights_t* w2, const float* w2_scale, int T, int k, int E, int H,
                           int I, void* workspace, size_t workspace_bytes, void* out, void* stream) {
  const int rc = check_packed(MOE_DTYPE_INT4_W4A16, w1, w2, T, k, E, H, I);
  if (rc != MOE_OK || T == 0) return rc;
  return route_forward(MOE_DTYPE_INT4_W4A16, topk_ids, x, topk_w, routing, routing_bytes, packed_data(w1),
                       w1_scale, packed_data(w2), w2_scale, T, k, E, H, I, workspace, workspace_bytes, out,
                       stream);
}

int moe_route_forward_int8_w8a16(const int32_t* topk_ids, const void* x, const float* topk_w, void* routing,
                                 size_t routing_bytes, const moe_packed_weights_t* w1, const float* w1_scale,
                                 const moe_packed_weights_t* w2, const float* w2_scale, int T, int k, int E,
                                 int H, int I, void* workspace, size_t workspace_bytes, void* out,
                                 void* stream) {
  const int rc = check_packed(MOE_DTYPE_INT8_W8A16, w1, w2, T, k, E, H, I);
  if (rc != MOE_OK || T == 0) return rc;
  return route_forward(MOE_DTYPE_INT8_W8A16, topk_ids, x, topk_w, routing, routing_bytes, packed_data(w1),
                       w1_scale, packed_data(w2), w2_scale, T, k, E, H, I, workspace, workspace_bytes, out,
                       stream);
}

int moe_forward_fp8_noalloc(const void* x, const float* topk_w, const void* routing,
                            const moe_packed_weights_t* w1, const float* w1_scale,
                            const moe_packed_weights_t* w2, const float* w2_scale, int T, int k, int E,
                            int H, int I, void* out, void* stream) {
  int rc = check_packed(MOE_DTYPE_FP8_W8A8, w1, w2, T, k, E, H, I);
  if (rc != MOE_OK || T == 0) return rc;
  moe_workspace_layout_t W;
  workspace_layout(MOE_DTYPE_FP8_W8A8, T, k, H, I, make_plan(MOE_DTYPE_FP8_W8A8, T, k, E, H, I), &W);
  if (W.total_bytes > MOE_STATIC_WORKSPACE_BYTES) return MOE_ERR_BUFFER_TOO_SMALL;
  void* ws = nullptr;
  if ((rc = scratch_address(&ws)) != MOE_OK) return rc;
  return forward(MOE_DTYPE_FP8_W8A8, x, topk_w, routing, packed_data(w1), w1_scale, packed_data(w2),
                 w2_scale, T, k, E, H, I, ws, MOE_STATIC_WORKSPACE_BYTES, out, stream);
}

int moe_set_stage_events(void* const* events, int n) {
  if (!events) {
    g_events_on = false;
    return MOE_OK;
  }
  if (n < 10) return MOE_ERR_INVALID_ARG;
  int pairs = 0;
  for (int st = 0; st < 5; st++) {
    if (!events[2 * st] != !events[2 * st + 1]) return MOE_ERR_INVALID_ARG;
    if (events[2 * st]) pairs++;
  }
  if (pairs == 0) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < 10; i++) g_events[i] = events[i];
  g_events_on = true;
  return MOE_OK;
}

int moe_stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words, void* stream) {
  if (!buf || !sink || sink_words < 1 || bytes % 16 || !aligned(buf, 16) || !aligned(sink, 4))
    return MOE_ERR_INVALID_ARG;
  if (bytes == 0) return MOE_OK;
  int cus = 0;
  const int rc = cu_count(&cus);
  if (rc != MOE_OK) return rc;
  const int groups = (int)std::min<size_t>(sink_words, (size_t)cus * 8);
  const hipError_t e = moe_host::launch_stream_read(buf, bytes, sink, groups, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_tile_copy_read(int pattern, const void* buf, size_t bytes, int row_bytes, int reps, uint32_t* sink,
                       size_t sink_words, void* stream) {
  if (pattern < 0 || pattern > 2 || !buf || !sink || !aligned(buf, 16) || !aligned(sink, 4) || reps < 0 ||
      row_bytes <= 0 || row_bytes % 2048)
    return MOE_ERR_INVALID_ARG;
  int cus = 0;
  const int rc = cu_count(&cus);
  if (rc != MOE_OK) return rc;
  if (cus < 128) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (bytes < moe_host::tile_copy_bytes(cus, row_bytes) || sink_words < (size_t)cus) return MOE_ERR_BUFFER_TOO_SMALL;
  if (reps == 0) return MOE_OK;
  const hipError_t e =
      moe_host::launch_tile_copy(pattern, buf, row_bytes, reps, sink, cus, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_device_cu_count(void) {
  int n = 0;
  const int rc = cu_count(&n);
  return rc == MOE_OK ? n : rc;
}

}  // extern "C"
