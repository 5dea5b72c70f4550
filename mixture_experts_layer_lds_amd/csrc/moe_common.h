// Shared device/host definitions of the MI355X fused-MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef long i64x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kMaxPairs = 65536;
constexpr int kMaxExperts = 511;   // keys of the routing sort (ids and the dropped bucket) fit nine bits
constexpr int kMaxTopK = 16;

// Routing-buffer header fields (int32 index into the 64-byte header).
constexpr int kHdrNumTasks = 0;
constexpr int kHdrNumDropped = 1;
constexpr int kHdrBlockM = 2;
constexpr int kHdrNumPairs = 3;
constexpr int kHdrNumExperts = 4;
constexpr int kHdrMaxTasks = 5;
constexpr int kHdrMaxExpertTiles = 6;   // largest number of row tiles of one expert

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

// fp32 -> OCP e4m3 code, round to nearest even, saturating to +-448.  The
// hardware conversion rounds to nearest even but turns magnitudes above the
// largest finite value into NaN, so the input is clamped first.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float v) {
  v = __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xffu;
}

// Four fp32 -> four e4m3 codes packed little-endian in one word.
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4_sat(float a, float b, float c, float d) {
  a = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
  b = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
  c = __builtin_fminf(__builtin_fmaxf(c, -448.0f), 448.0f);
  d = __builtin_fminf(__builtin_fmaxf(d, -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Scale pair of the per-row activation quantisation: scale = fp32(amax/448),
// inv = fp32(448/amax), both divisions in fp64; an all-zero row gets 1 and 1.
__device__ __forceinline__ void e4m3_row_scales(float amax, float* scale, float* inv) {
  if (amax > 0.0f) {
    *scale = (float)((double)amax / 448.0);
    *inv = (float)(448.0 / (double)amax);
  } else {
    *scale = 1.0f;
    *inv = 1.0f;
  }
}

// acc += A * B^T over 128 bytes of K of e4m3 data, on the full-rate gfx950
// instruction (v_mfma_scale_f32_16x16x128_f8f6f4, both block scales 2^0).
// (a0, a1) and (b0, b1) are the lane's 16-byte fragments of two consecutive
// 64-byte K steps in the packed lane order (lane l: row/column l % 16,
// bytes 16*(l/16) of each step).  The instruction's K order (measured on
// the device) puts a lane's first 16 bytes at K 16*(l/16).. and its last 16
// at K 64 + 16*(l/16)..; with the two steps' fragments in that order its K
// is exactly the memory order of the 128 bytes.
__device__ __forceinline__ void mfma_fp8_k128(f32x4& acc, const u32x4& a0, const u32x4& a1,
                                              const u32x4& b0, const u32x4& b1) {
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                   (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                   (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
}

// As mfma_fp8_k128, with each operand's two 16-byte fragments already in
// one 8-dword tuple (first step in the low half).
__device__ __forceinline__ void mfma_fp8_unit(f32x4& acc, const i32x8& a, const i32x8& b) {
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
}

// As mfma_fp8_k128 with MX block scales: sa / sb hold, in their low byte,
// the e8m0 code (2^(c-127)) of K block l/16 of the lane's row / column
// (the instruction takes lane 16*g + r's scale for row r's 32 values
// K 32*g.. of the unit).
__device__ __forceinline__ void mfma_mx_k128(f32x4& acc, const u32x4& a0, const u32x4& a1,
                                             const u32x4& b0, const u32x4& b1, int sa, int sb) {
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                   (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                   (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

// Max of v over the 16 lanes that share (lane >> 4).
__device__ __forceinline__ float max16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Max of v over a workgroup of NT threads (NT / 64 <= 8 waves), returned to
// every thread.
template <int NT>
__device__ float block_max_f32(float v) {
  __shared__ float s_max[NT / 64];
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = s_max[0];
#pragma unroll
  for (int w = 1; w < NT / 64; w++) r = __builtin_fmaxf(r, s_max[w]);
  return r;
}

// Largest |v| of a row of n fp32 values (n % 4 == 0) by a workgroup of NT
// threads (NT / 64 <= 8 waves), returned to every thread.
template <int NT>
__device__ float row_amax_f32(const float* __restrict__ v, int n) {
  __shared__ float s_max[NT / 64];
  const f32x4* row = reinterpret_cast<const f32x4*>(v);
  float m = 0.0f;
  for (int i = threadIdx.x; i < n / 4; i += NT) {
    const f32x4 a = row[i];
    m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(a[0]), __builtin_fabsf(a[1])),
                                           __builtin_fmaxf(__builtin_fabsf(a[2]), __builtin_fabsf(a[3]))));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = s_max[0];
#pragma unroll
  for (int w = 1; w < NT / 64; w++) r = __builtin_fmaxf(r, s_max[w]);
  return r;
}

}  // namespace moe

// Host-side launch helpers implemented by the kernel translation units.
namespace moe_host {

// Router top-k over fp32 logits[T][E] into ids/w [T][k + n_shared]; with
// S > 1 the logits are the sum of S planes [S][T][E] (added in ascending
// plane order), written to logits_out when it is not null.
hipError_t launch_router_topk(const float* logits, int S, float* logits_out, int T, int E, int k,
                              int renorm, int n_shared, int32_t* ids, float* w, hipStream_t s);

// Precision-aware router GEMM.
struct RouterGemmArgs {
  const void* x;        // bf16 [T][K]
  const void* w_hi;     // packed bf16 W_high, rows padded to 16
  const void* w_lo;     // packed bf16 W_low (the residual x 256)
  float* out;           // [S][T][N] partial planes, or [T][N] scores when S == 1
  int T, N, K, S;
  int tb_count, nb_count;
  long slice_stride;    // floats between planes (T * N)
};
struct RouterGemmPlan {
  int mb = 1, nb = 1, waves = 4, S = 1;   // token / expert 16-blocks per item, waves, K slices
  int tb_count = 1, nb_count = 1;
};
RouterGemmPlan plan_router_gemm(int T, int N, int K, int cus);
size_t router_partial_bytes(int T, int N, const RouterGemmPlan& p);
hipError_t launch_router_split(const float* w, int N, int K, void* pair, hipStream_t s);
hipError_t launch_router_gemm(const void* x, const void* pair, int T, int N, int K,
                              const RouterGemmPlan& p, float* out, hipStream_t s);
hipError_t launch_router_reduce(const float* partials, int S, int T, int N, float* out, hipStream_t s);
// Largest E the router kernel takes.
int router_max_experts();

// The routing build of a decode batch (at most 64 pairs) folded into the
// first kernel of the forward pass: every workgroup sorts the pairs in
// registers, and workgroup 0 also writes the routing buffer's parts, byte
// for byte what the routing build writes.  ids == nullptr: the kernel reads
// a routing buffer built before it.
struct DecodeRouteOut {
  const int32_t* ids;          // the T * k expert ids
  int32_t* header;             // 16 ints
  int32_t* expert_offsets;     // E + 1
  int32_t* sorted_pairs;       // T * k
  int32_t* pair_pos;           // T * k
  moe_task_t* tasks;           // max_tasks
  int E, block_m, max_tasks;
};

hipError_t launch_route(const int32_t* ids, int P, int E, int block_m, int max_tasks,
                        void* routing, const moe_routing_layout_t& L, hipStream_t s);
// Bytes of the routing work area (per-segment key counts) for P pairs.
size_t route_scratch_bytes(int P);

// Per-token e4m3 quantisation of bf16 rows x[T][H]; when zero_rows is not
// null the same launch also clears zero_rows[0 .. T*zk) (row amax slots);
// when scale_rows is not null it also writes each token's scale at the
// sorted rows pair_pos[t*zk + j] of its zk pairs.
// With route (T * zk <= 64) the launch also does the routing build, and the
// sorted rows of the pairs come from there instead of pair_pos.
hipError_t launch_quant_rows_bf16(const uint16_t* x, int T, int H, uint8_t* xq, float* scale,
                                  float* zero_rows, int zk, const int32_t* pair_pos,
                                  float* scale_rows, hipStream_t s,
                                  const DecodeRouteOut* route = nullptr);

// SiLU-and-mul of the gate-up partial sums g[S][P][2I] for the valid sorted
// rows; writes bf16 h[P][I] (fp8 = false) or e4m3 codes h[P][I] + scales.
// With x_scale (fp8 strips), the slice sums of row r are first multiplied
// by x_scale[sorted_pairs[r] / k].
hipError_t launch_act(const float* g, int S, int P, int I, const int32_t* expert_offsets, int E,
                      bool fp8, const float* x_scale, const int32_t* sorted_pairs, int k, void* h,
                      float* h_scale, hipStream_t s);

// out[t] = bf16(sum_j w[t][j] * row_scale[r] * sum_s y[s][r]) over valid
// pairs, r = pos[t*k+j]; y is fp32 [S][P][H] (y_bf16 = false) or bf16
// [P][H] (S = 1); row_scale null means 1.
hipError_t launch_reduce(const void* y, bool y_bf16, int S, int P, const float* topk_w,
                         const int32_t* pair_pos, const int32_t* expert_offsets, const float* row_scale,
                         int E, int T, int k, int H, uint16_t* out, hipStream_t s);

// Byte permutation of W[E][rows][row_bytes] into 1 KiB MFMA-fragment chunks.
hipError_t launch_pack(const void* w, int E, int rows, int row_bytes, void* packed,
                       hipStream_t s);

// LDS-tiled grouped GEMM (128-row task tiles).  Gate-up mode writes
// SiLU(gate)*up (bf16, or fp32 + row amax on the fp8 path); down mode writes
// bf16 rows.
struct TiledArgs {
  const void* a;                // gate-up: x / xq [T][K] (gathered); down: h / hq [P][K]
  const float* a_scale;         // fp8: x scales [T] / h scales [P]
  const void* b;                // packed weights, w_rows rows per expert
  const float* b_scale;         // fp8: [E][w_rows]
  const int32_t* sorted_pairs;
  const int32_t* header;
  const moe_task_t* tasks;
  void* c;                      // gate-up: h [P][N_out]; down: y [P][N_out] bf16
  float* row_amax;              // fp8 gate-up: [P] atomic-max slots (pre-cleared)
  int K;                        // reduction length (elements)
  int N_out;                    // output columns (I for gate-up, H for down)
  int w_rows;                   // weight rows per expert (2I or H)
  int topk;
  int max_tasks;
};

hipError_t launch_tiled_gemm(const TiledArgs& a, bool gateup, bool fp8, int bm, int bn, int grid,
                             hipStream_t s);

// Strip GEMM (A in an LDS ring shared by 8 waves, weights streamed to
// registers): work items of 256 output columns of one task tile and one K
// slice.  On fp8 only the weight column scale is applied; the consumer
// applies the row scale.
struct StripArgs {
  const void* a;                // gathered: x / xq [T][K]; contiguous: h / hq [P][K]
  const void* b;                // packed weights [E][N][K]
  const float* b_scale;         // fp8: [E][N]
  const int32_t* sorted_pairs;  // gathered: pair index of each sorted row
  const int32_t* header;
  const moe_task_t* tasks;
  void* c;                      // fp32 [split][P][N], or bf16 [P][N] when out_bf16
  int K;                        // reduction length (elements)
  int N;                        // output columns, a multiple of 256
  int P;
  int topk;
  int max_tasks;
  int split;                    // K slices
  int out_bf16;                 // 1: bf16 rows (split == 1)
  // gate-up with one K slice: a wave's two 16-row weight blocks are a gate
  // block and the matching up block, and c receives h = SiLU(gate) * up,
  // [P][N/2]: bf16, or on fp8 fp32 with the weight and x scales applied
  int act;
  const float* x_scale_rows;    // fp8 / int8 act: x scale of each sorted row [P + 16]
  // block fp8 (b_scale then [E][N/128][K/128]): group scales of the sorted
  // rows, unit-major [K/128][P]
  const float* rs_u;
  // MXFP8: e8m0 codes of a's rows ([T][K/32] per token when gathered, else
  // [P][K/32] per sorted row) and of the weights [E][N][K/32]
  const uint8_t* a_mx;
  const uint8_t* b_mx;
  // 1: strip j of a tile runs its K stages rotated by (j mod 16) x (stages / 16),
  // so the strips that share the tile's token rows read different rows' lines at
  // any moment; 0: every strip in K order
  int rotate;
};

// (mb, ks, nbuf) = 16-row blocks per tile, 64-byte K steps per stage, stages in flight.
// variant (with fp8 set): 1 int8 w8a8 codes and the integer MFMA, scales as
// on fp8; 2 block fp8, 3 MXFP8 (even ks, K % 128 == 0, one K slice with act).
bool strip_config_supported(int mb, int ks, int nbuf, bool fp8);
hipError_t launch_strip_gemm(const StripArgs& a, bool gather, bool fp8, int mb, int ks, int nbuf,
                             int grid, hipStream_t s, int variant = 0);

// Register-streaming GEMM with the reduction split over the W waves of a
// workgroup (few rows per expert).  Gate-up mode writes SiLU(gate)*up (bf16,
// or fp32 + row amax on fp8); down mode writes bf16 rows (fp8: weight column
// scale applied, row scale left to the reduction).
struct StreamArgs {
  const void* a;                // gate-up: x / xq [T][K] (gathered); down: h / hq [P][K]
  const void* b;                // packed weights, w_rows rows per expert
  const float* b_scale;         // fp8: [E][w_rows]
  const float* row_scale;       // fp8 gate-up: activation scale of each sorted row [P + 16]
  const int32_t* sorted_pairs;
  const int32_t* header;
  const moe_task_t* tasks;
  void* c;                      // gate-up: h [P][N_out] (bf16, or fp32 on fp8); down: y [P][N_out] bf16
  const uint8_t* a_mx;          // MX: e8m0 codes of a's rows [rows][K/32] (gate-up: token rows)
  const uint8_t* b_mx;          // MX: e8m0 codes of the weights [E][w_rows][K/32]
  int P;                        // block fp8: sorted rows (stride of the unit-major row scales)
  int K;                        // reduction length (elements)
  int N_out;                    // output columns (I for gate-up, H for down)
  int w_rows;                   // weight rows per expert (2I or H)
  int topk;
  int max_tasks;
  DecodeRouteOut route;         // bf16 gate-up, at most 64 pairs: the routing build folded in
};

// bf16 gate-up on 16-row tiles with half-width items (8 h columns each; K
// steps a multiple of 2 * waves).
// With a.route.ids set (at most 64 pairs) the launch also does the routing build.
hipError_t launch_stream_half_gateup(const StreamArgs& a, int waves, int grid, hipStream_t s);
// Down GEMM and top-k weighted sum of a single token in one launch (T = 1,
// at most 16 pairs; `half`: at most 8): one workgroup of `waves` waves per
// 16 output columns (`half`: 8), writing the bf16 token row `out`; topk_w
// [k], h_scale (fp8) per sorted row.  (waves, u) in (4, 2), (8, 2), (16, 2),
// (8, 4), (16, 4); the K steps (K * element bytes / 64) a multiple of u
// (`half`: 2u).
// i8 (with fp8): int8 w8a8 codes on the integer MFMA.
hipError_t launch_stream_down_reduce(const StreamArgs& a, bool fp8, int waves, int u, bool half,
                                     const float* topk_w, const float* h_scale, uint16_t* out, hipStream_t s,
                                     bool i8 = false);
// (mb, waves, u) = 16-row blocks per tile, waves per workgroup, K steps per stage.
bool stream_config_supported(int mb, int waves, int u);
// kind: 0 per-channel scales (bf16, or fp8 by `fp8`), 1 MXFP8 block scales,
// 2 int8 w8a8 (per-channel scales).
// nb: weight blocks per item, 2, or 4 (two-step stages): MX or int8 w8a8 on
// 64-row tiles with one or two waves, bf16 (kind 0, !fp8) on 32-row tiles
// with one, two or four waves.  a.route.ids set (the routing build folded
// in): bf16 gate-up on 16-row tiles with nb = 2 only.
hipError_t launch_stream_gemm(const StreamArgs& a, bool gateup, bool fp8, int kind, int mb, int waves,
                              int u, int grid, hipStream_t s, int nb = 2);
// int8 w8a8: per-token quantisation of bf16 x (row-amax slots cleared,
// per-sorted-row scales written as the fp8 variant) and per-row
// requantisation of fp32 h (the row amax found from the row).
// With route (T * zk <= 64) the x quantisation also does the routing build.
hipError_t launch_quant_rows_i8(const uint16_t* x, int T, int H, int8_t* xq, float* scale,
                                float* zero_rows, int zk, const int32_t* pair_pos, float* scale_rows,
                                hipStream_t s, const DecodeRouteOut* route = nullptr);
hipError_t launch_requant_rows_i8(const float* h32, int P, int I, const int32_t* expert_offsets, int E,
                                  int8_t* hq, float* h_scale, hipStream_t s);
// int8 w8a16 register-streaming GEMM: a bf16 rows, b packed int8 weights
// with per-row fp32 scales b_scale [E][w_rows]; gate-up writes bf16
// SiLU(gate)*up, down bf16 rows.
hipError_t launch_stream_w8(const StreamArgs& a, bool gateup, int mb, int waves, int grid, hipStream_t s,
                            int nb = 2);
// Block-scaled fp8 register-streaming GEMM (K % 128 == 0): a e4m3 rows, b
// packed e4m3 weights.  block: unit-major group scales row_scale [K/128][P]
// (per sorted row), b_scale fp32 [E][w_rows/128][K/128]; gate-up writes fp32
// SiLU(gate)*up, down bf16 rows.  !block (per-channel fp8 w8a8): row_scale
// the per-sorted-row x scales, b_scale [E][w_rows]; gate-up writes fp32
// SiLU(gate)*up (the requantisation pass finds the row amax), down applies
// the weight row scales only.
// nb: weight blocks per item, 2, or 4 (block scales, 64-row tiles, waves <= 2).
hipError_t launch_stream_fp8b(const StreamArgs& a, bool gateup, bool block, int mb, int waves, int grid,
                              hipStream_t s, int nb = 2);
// Group (128-value) fp8 quantisation: bf16 token rows x (scales also per
// token [T][H/128] and per sorted row of each of the token's zk pairs,
// unit-major [H/128][P]); fp32 rows h of the valid sorted rows (scales
// unit-major [I/128][P]).
// With route (P = T * zk <= 64) the launch also does the routing build.
hipError_t launch_quant_groups_bf16(const uint16_t* x, int T, int H, uint8_t* xq, float* group_scale,
                                    float* rows_scale, int P, int zk, const int32_t* pair_pos,
                                    hipStream_t s, const DecodeRouteOut* route = nullptr);
hipError_t launch_requant_groups(const float* h, int P, int I, const int32_t* expert_offsets, int E,
                                 uint8_t* hq, float* rows_scale, hipStream_t s);
// int4 w4a16 register-streaming GEMM: a bf16 activations, b packed int4
// weights, b_scale fp32 [E][w_rows][K/128] group scales; gate-up writes bf16
// SiLU(gate)*up, down bf16 rows.
hipError_t launch_stream_w4(const StreamArgs& a, bool gateup, int mb, int waves, int grid, hipStream_t s,
                            int nb = 2);
// MXFP8 quantisation: bf16 rows x[T][H] -> e4m3 xq + e8m0 codes [T][H/32];
// fp32 rows h[P][I] (valid sorted rows only) -> hq + codes [P][I/32].
// With route (P <= 64 pairs) the launch also does the routing build.
hipError_t launch_mx_quant_bf16(const uint16_t* x, int T, int H, uint8_t* xq, uint8_t* sx, hipStream_t s,
                                const DecodeRouteOut* route = nullptr, int P = 0);
hipError_t launch_mx_requant(const float* h, int P, int I, const int32_t* expert_offsets, int E,
                             uint8_t* hq, uint8_t* sh, hipStream_t s);

// Streaming read of `bytes` (multiple of 16) of buf by `groups` workgroups,
// one folded word per workgroup written to sink.
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int groups, hipStream_t s);
// Token-tile copy measurement (one workgroup per CU, cus >= 128): the bytes
// its buffer must hold, and the launch.
size_t tile_copy_bytes(int cus, int row_bytes);
hipError_t launch_tile_copy(int pattern, const void* buf, int row_bytes, int reps, uint32_t* sink, int cus,
                            hipStream_t s);

// fp32 rows -> e4m3 codes with the row amax held in h_scale (replaced by the scale).
hipError_t launch_requant_rows(const float* h32, int P, int I, const int32_t* expert_offsets,
                               int E, uint8_t* hq, float* h_scale, bool find_amax, hipStream_t s);

}  // namespace moe_host
