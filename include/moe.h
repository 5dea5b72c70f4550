/*
 * moe.h -- C ABI of the fused Mixture-of-Experts layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer (HPC-Ops x SGLang blog, section "MoE: reducing overhead around
 * small expert GEMMs") computes, for every token t with top-k expert ids
 * e_j and routing weights w[t][j],
 *
 *     out[t] = sum_j w[t][j] * W2[e_j] ( SiLU(W1g[e_j] x[t]) * (W1u[e_j] x[t]) )
 *
 * as a pipeline of hand-written HIP kernels: a routing/index build that
 * counting-sorts token-expert pairs in LDS into contiguous per-expert
 * ranges plus a per-tile task map; a grouped gate-up GEMM on MFMA that
 * reads tokens through the route index (no gather buffer); one fused
 * kernel for SiLU-and-mul and, on the fp8 path, the per-row FP8
 * requantisation; a grouped down GEMM; and a top-k weighted reduction back
 * to token order.
 *
 * Conventions for every entry point
 *  - Pointers marked (device) are device memory on the current HIP device;
 *    (host) are host memory.  The caller owns every buffer: the library
 *    never allocates or frees memory and keeps no per-call state.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every device-side step is enqueued asynchronously on it; no call
 *    synchronises, allocates or reads device memory from the host, so the
 *    calls can be captured into a HIP graph.  Grids depend only on the
 *    host-side sizes, so one capture serves any routing at those sizes.
 *  - Shapes: T tokens (0 <= T, T*k <= 65536), k experts per token
 *    (1..16), E experts (1..511: the keys of the routing sort, expert ids
 *    plus one dropped bucket, are nine bits wide; fused shared experts
 *    count as experts), hidden size H and expert intermediate
 *    size I (positive multiples of 64, at most 65536).
 *  - Layouts (row-major, last index contiguous):
 *      x        [T][H]      bf16 hidden states
 *      topk_ids [T][k]      int32 expert ids; an id outside [0, E) marks a
 *                           dropped pair (it adds nothing to the output);
 *                           duplicate ids of one token are separate pairs
 *      topk_w   [T][k]      fp32 routing weights
 *      W1       [E][2I][H]  gate rows [0, I), up rows [I, 2I)
 *      W2       [E][H][I]
 *      out      [T][H]      bf16
 *    The forward calls take W1 and W2 pre-packed by moe_pack_weights (same
 *    byte size, MFMA-fragment order), through the moe_packed_weights_t
 *    descriptor that moe_pack_weights fills; everything else is row-major.
 *    bf16 is IEEE binary16-brain (1/8/7); fp8 is OCP E4M3 ("e4m3fn",
 *    max finite 448).
 *  - Stage order: [fp8: quantise x] -> gate-up GEMM -> SiLU-and-mul
 *    [+ fp8 requant] -> down GEMM -> top-k weighted reduction, all on
 *    `stream`.
 *  - Return value: MOE_OK (0) or a negative moe_status_t.  Argument errors
 *    are detected on the host before anything is enqueued; nothing is
 *    launched when a call fails.  T == 0 returns MOE_OK with no launch.
 *    No C++ exception crosses this interface.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,        /* null pointer, bad count, misaligned buffer */
    MOE_ERR_UNSUPPORTED_SHAPE = -2,  /* H or I not a multiple of 64, T*k > 65536, ... */
    MOE_ERR_BUFFER_TOO_SMALL = -3,   /* routing buffer or workspace smaller than required */
    MOE_ERR_HIP = -4                 /* a HIP runtime call or kernel launch failed */
} moe_status_t;

typedef enum {
    MOE_DTYPE_BF16 = 0,      /* bf16 activations and weights, fp32 accumulation */
    MOE_DTYPE_FP8_W8A8 = 1,  /* e4m3 weights (per-output-channel fp32 scales) and
                                e4m3 activations (per-row fp32 scales) */
    MOE_DTYPE_MXFP8 = 2,     /* OCP MXFP8: e4m3 values with one e8m0 scale per 32
                                consecutive K values, weights and activations */
    MOE_DTYPE_INT8_W8A8 = 3, /* int8 weights (per-output-channel fp32 scales) and
                                int8 activations (per-row fp32 scales) */
    MOE_DTYPE_INT4_W4A16 = 4, /* int4 weights (fp32 scale per 128 K values of a row),
                                 bf16 activations */
    MOE_DTYPE_FP8_BLOCK = 5,  /* e4m3 weights with an fp32 scale per 128 x 128 block,
                                 e4m3 activations with one per 128-value row group */
    MOE_DTYPE_INT8_W8A16 = 6  /* int8 weights (per-output-channel fp32 scales),
                                 bf16 activations */
} moe_dtype_t;

/* One row tile of the task map: rows [row_begin, row_begin + rows) of the
 * expert-sorted order, all routed to `expert`; rows <= block_m. */
typedef struct {
    int32_t expert;
    int32_t row_begin;
    int32_t rows;
    int32_t reserved;   /* 0 */
} moe_task_t;

/* First 64 bytes of a routing buffer, written by moe_build_routing_*. */
typedef struct {
    int32_t num_tasks;     /* valid entries of the task map */
    int32_t num_dropped;   /* pairs whose id is outside [0, E) */
    int32_t block_m;       /* tile height the task map was cut with */
    int32_t num_pairs;     /* P = T * k */
    int32_t num_experts;   /* E */
    int32_t max_tasks;     /* capacity of the task map */
    int32_t max_expert_tiles; /* largest number of tiles of one expert (0 if none) */
    int32_t reserved[9];
} moe_routing_header_t;

/* Byte offsets of the parts of a routing buffer (all 16-byte aligned). */
typedef struct {
    size_t header;           /* moe_routing_header_t */
    size_t expert_offsets;   /* int32 [E+1]: expert e owns sorted rows
                                [expert_offsets[e], expert_offsets[e+1]);
                                expert_offsets[E] = number of valid pairs */
    size_t sorted_pairs;     /* int32 [P]: pair index p = t*k + j at each sorted
                                row; valid pairs ascending in p within each
                                expert, then dropped pairs ascending in p */
    size_t pair_pos;         /* int32 [P]: sorted row of pair p (inverse) */
    size_t tasks;            /* moe_task_t [max_tasks]: expert-major row tiles */
    size_t scratch;          /* work area of the routing build (large P only;
                                contents unspecified afterwards) */
    size_t total_bytes;      /* minimum size of the routing buffer */
    int32_t block_m;         /* tile height chosen for these sizes and dtype */
    int32_t max_tasks;       /* P / block_m + min(E, P) */
} moe_routing_layout_t;

/* Byte offsets of the parts of a forward workspace (all 256-byte aligned);
 * an offset of (size_t)-1 marks a part these sizes do not use.  Three tilings
 * exist, chosen by a fixed function of the sizes and dtype (`tiling`):
 *  0 register streaming (few rows per expert, e.g. decode): the waves of a
 *    workgroup split each reduction and add their sums in LDS; SiLU(gate)*up
 *    is formed in the gate-up GEMM's epilogue and the down rows are bf16;
 *  2 strips (token rows staged in LDS, weights streamed to registers; a few
 *    dozen to ~80 rows per expert): the GEMMs may split their reduction into
 *    split_k1 / split_k2 slices whose fp32 partial sums the next kernel adds
 *    in ascending slice order; with split_k1 == 1 the gate-up epilogue
 *    forms SiLU(gate)*up (fp8: in fp32, then requantised); strips with
 *    split_k2 == 1 write bf16 down rows;
 *  1 LDS tiles of both operands (many rows per expert): no split;
 *    SiLU(gate)*up is formed in the gate-up GEMM's epilogue and the down rows
 *    are bf16. */
typedef struct {
    size_t xq;          /* fp8: uint8 [T][H]   per-token e4m3 codes of x */
    size_t x_scale;     /* fp8: fp32  [T]      per-token scales of x */
    size_t x_scale_rows;/* fp8, tiling 0, and tiling 2 with split_k1 == 1:
                           fp32 [P + 16] the token's scale at each sorted row */
    size_t g;           /* tiling 2 with split_k1 > 1: fp32 [split_k1][P][2I]
                           gate-up partial sums (weight scales only on fp8);
                           fp8 otherwise: fp32 [P][I] SiLU(gate)*up before
                           requantisation; unused on bf16 outside tiling 2
                           with split_k1 > 1 */
    size_t h;           /* bf16 [P][I] SiLU(gate)*up (bf16), or uint8 e4m3 codes [P][I] (fp8) */
    size_t h_scale;     /* fp8: fp32  [P]      per-row scales of h */
    size_t y;           /* tiling 2 with split_k2 > 1: fp32 [split_k2][P][H]
                           unweighted down partial sums; otherwise bf16
                           [P][H] unweighted down rows (fp8, tilings 0 and 2:
                           weight scales only); unused (SIZE_MAX) on bf16,
                           fp8 and int8 w8a8 at T = 1 with tiling 0 and an
                           even number of 64-byte steps in an I row, where the
                           down launch adds the token's top-k rows itself */
    size_t total_bytes; /* minimum size of the workspace */
    int32_t split_k1;   /* slices of the gate-up reduction over H (1 unless tiling 2) */
    int32_t split_k2;   /* slices of the down reduction over I */
    int32_t tiling;     /* 0 register streaming, 1 LDS tiles, 2 strips */
} moe_workspace_layout_t;

/* A weight tensor packed by moe_pack_weights, as the forward calls take W1
 * and W2 (a host struct; the bytes it names are device memory).
 * moe_pack_weights fills every field, and `check` binds the others
 * together: a forward call accepts a descriptor only if it was made by
 * moe_pack_weights for that call's dtype, expert count and matrix shape
 * (W1: rows = 2I, cols = H; W2: rows = H, cols = I), and returns
 * MOE_ERR_INVALID_ARG for anything else, including row-major weights or a
 * hand-made descriptor.  The check runs on the host and reads no device
 * memory.  The descriptor owns nothing; it is valid while the packed buffer
 * lives and is unchanged. */
typedef struct {
    const void *data;   /* device: the packed bytes */
    int32_t dtype;      /* moe_dtype_t the bytes were packed for */
    int32_t experts;    /* E */
    int32_t rows;       /* rows per expert */
    int32_t cols;       /* elements per row (the reduction length) */
    uint64_t check;     /* written by moe_pack_weights */
} moe_packed_weights_t;

/* Human-readable name of a status code (static string). */
const char *moe_status_string(int status);

/* Layout of the routing buffer for these sizes (host-only computation).
 * dtype is a moe_dtype_t; `out` is a host pointer.  The tile height is a
 * fixed function of (dtype, T, k, E, H, I), shared by the routing build and
 * the forward pass. */
int moe_routing_layout(int T, int k, int E, int H, int I, int dtype,
                       moe_routing_layout_t *out /* host */);

/* Layout of the forward workspace for these sizes (host-only). */
int moe_workspace_layout(int T, int k, int E, int H, int I, int dtype,
                         moe_workspace_layout_t *out /* host */);

/* One-time weight pre-pack (done when weights are loaded, like the blog's
 * router weights that are preprocessed once and reused across requests and
 * graph replays).  w (device) is a row-major [E][rows][cols] tensor of
 * dtype elements (bf16, or e4m3 codes for MOE_DTYPE_FP8_W8A8); packed
 * (device, same byte size, must not overlap w) receives it cut into blocks
 * of 16 rows x 64 bytes, each stored as one contiguous 1 KiB chunk whose
 * 16-byte piece l holds row (l % 16), bytes 16*(l / 16).. of the block;
 * chunks are ordered (expert, 16-row block, 64-byte step).  Pack W1 with
 * rows = 2I, cols = H and W2 with rows = H, cols = I.  Requires rows % 16
 * == 0 and cols * element size % 64 == 0; both pointers 16-byte aligned.
 * Scales are not packed.  On MOE_OK, desc (host, not NULL) describes
 * `packed` for the forward calls; on an error it is left unchanged. */
int moe_pack_weights(const void *w, int E, int rows, int cols, int dtype, void *packed,
                     moe_packed_weights_t *desc /* host, out */, void *stream);

/* Descriptor (host, no device access) for bytes that are already in the
 * packed order of moe_pack_weights: a device copy of a packed buffer, or
 * packed weights stored once and loaded again.  Same size and pointer rules
 * as moe_pack_weights.  The library cannot tell packed bytes from row-major
 * ones; this explicit call is the caller's statement that `packed` holds
 * the output of moe_pack_weights for these sizes and dtype. */
int moe_describe_packed_weights(const void *packed, int E, int rows, int cols, int dtype,
                                moe_packed_weights_t *desc /* host, out */);

/* Routing & index build (blog section "MoE", routing & index build): one
 * workgroup counting-sorts the P = T*k pairs by expert id in LDS, writing
 * the header, expert offsets, route index (sorted_pairs, pair_pos) and the
 * per-tile task map into `routing` (device, 16-byte aligned, at least
 * moe_routing_layout().total_bytes).  The order is deterministic: stable in
 * the pair index.  topk_ids (device) is [T][k] int32.  The _bf16 and _fp8
 * variants differ only in the tile height they cut the task map with,
 * which must match the forward call of the same dtype. */
int moe_build_routing_bf16(const int32_t *topk_ids, int T, int k, int E, int H, int I,
                           void *routing, size_t routing_bytes, void *stream);
int moe_build_routing_fp8(const int32_t *topk_ids, int T, int k, int E, int H, int I,
                          void *routing, size_t routing_bytes, void *stream);

/* Router top-k (blog section "Router GEMM": the router's fp32 expert
 * scores decide, through a top-k choice, which experts run; SGLang tuning
 * guide, model-config section: shared experts fused into the expert tensor
 * as extra expert ids).  The step before the routing build: from logits
 * (device) fp32 [T][E], for each token, softmax over the E scores, the k
 * largest in descending order (equal scores: ascending expert id; a NaN
 * logit ranks as -infinity), their weights renormalised to sum to one
 * (renormalize = 1) or left as softmax probabilities over all E
 * (renormalize = 0), then n_shared columns for the fused shared experts:
 * ids E .. E+n_shared-1 with weight 1.  Writes topk_ids (device) int32
 * [T][k+n_shared] and topk_w (device) fp32 [T][k+n_shared], which the
 * routing build and the forward pass take with k' = k+n_shared and
 * E' = E+n_shared (expert E+s is the s-th shared expert's weights).
 * The ranking compares the fp32 logits exactly, so the ids are a
 * deterministic function of the input; weights are fp32 and meaningful
 * when the selected logits are finite.  Requires 1 <= k <= E <= 256,
 * n_shared >= 0, k + n_shared <= 16, E + n_shared <= 511, renormalize in
 * {0, 1}; buffers 4-byte aligned.  T == 0 returns MOE_OK with no launch. */
int moe_router_topk(const float *logits, int T, int E, int k, int renormalize, int n_shared,
                    int32_t *topk_ids, float *topk_w, void *stream);

/* Precision-aware router GEMM (blog section "Router GEMM", precision-aware
 * BF16 formulation): fp32 router weights W [N][K], bf16 hidden states
 * x [T][K], fp32 scores [T][N].  W is split once (at weight load) into
 * W_high = W truncated to bf16 and W_low = RNE bf16 of (W - W_high) * 256,
 * and the scores are x . W_high + (x . W_low) / 256: two bf16 MFMA products
 * sharing each activation fragment, fp32 accumulation, the 1/256 applied in
 * the epilogue.  Against an fp32-weight product the split keeps the error
 * per weight below 2^-15 |W|.  Requires K a multiple of 64 (at most 65536),
 * 1 <= N <= 65536.
 *
 * moe_router_pair_bytes: size (host) of the split pair: 4 * N16 * K bytes,
 * N16 = N rounded up to a multiple of 16.
 * moe_router_split_weights: w (device) fp32 [N][K] row-major -> w_pair
 * (device, 16-byte aligned, at least moe_router_pair_bytes): W_high then
 * W_low, each N16 * K bf16 in the fragment order of moe_pack_weights (rows
 * N..N16-1 zero). */
int moe_router_pair_bytes(int N, int K, size_t *bytes /* host */);
int moe_router_split_weights(const float *w, int N, int K, void *w_pair, size_t w_pair_bytes,
                             void *stream);

/* Workspace (host query) of moe_router_gemm / moe_router_gemm_topk for these
 * sizes: partial-score planes when few tokens split K over workgroups. */
int moe_router_workspace_bytes(int T, int N, int K, size_t *bytes /* host */);

/* scores (device) fp32 [T][N] = router GEMM of x (device, bf16 [T][K],
 * 16-byte aligned) with the split pair w_pair.  workspace (device, 16-byte
 * aligned) of at least moe_router_workspace_bytes (may be NULL when that is
 * 0).  Deterministic: partial planes are added in a fixed order.  T == 0
 * returns MOE_OK with no launch. */
int moe_router_gemm(const void *x, const void *w_pair, int T, int N, int K, void *workspace,
                    size_t workspace_bytes, float *scores, void *stream);

/* Router GEMM followed by the router top-k (moe_router_topk) on its
 * scores, N = E experts (E <= 256), in two launches: the top-k kernel adds
 * the GEMM's partial planes as it loads them.  scores (device, fp32
 * [T][E]) receives the scores when not NULL.  topk_ids / topk_w as in
 * moe_router_topk; same argument rules as both calls. */
int moe_router_gemm_topk(const void *x, const void *w_pair, int T, int E, int K, int k,
                         int renormalize, int n_shared, void *workspace, size_t workspace_bytes,
                         float *scores, int32_t *topk_ids, float *topk_w, void *stream);

/* bf16 forward (blog section "MoE", gate-up & activation, PDL chaining;
 * operator table: BF16 hidden states).  x (device) bf16 [T][H]; topk_w
 * (device) fp32 [T][k]; routing (device) built by moe_build_routing_bf16
 * with the same sizes; w1 and w2 (host) descriptors, from moe_pack_weights
 * with dtype MOE_DTYPE_BF16, of bf16 W1 [E][2I][H] and W2 [E][H][I]
 * (any other descriptor: MOE_ERR_INVALID_ARG); workspace (device, 256-byte aligned, at least
 * moe_workspace_layout().total_bytes); out (device) bf16 [T][H].
 * Experts that receive no pair are never read.  Accumulation is fp32; the
 * intermediate SiLU(gate)*up and the per-pair down rows are stored as bf16;
 * the top-k reduction adds the pairs of a token in ascending j in fp32. */
int moe_forward_bf16(const void *x, const float *topk_w, const void *routing,
                     const moe_packed_weights_t *w1, const moe_packed_weights_t *w2,
                     int T, int k, int E, int H, int I,
                     void *workspace, size_t workspace_bytes, void *out, void *stream);

/* fp8 w8a8 forward (operator table: FP8 E4M3 expert weights; gate-up &
 * activation: FP8 requant before the down GEMM).  As moe_forward_bf16,
 * except: w1/w2 (host) describe e4m3 codes (packed by moe_pack_weights with
 * dtype MOE_DTYPE_FP8_W8A8), w1_scale (device) fp32 [E][2I] and
 * w2_scale (device) fp32 [E][H] are per-output-channel scales.  x is
 * quantised per token and SiLU(gate)*up per (token, expert) row with the
 * rule scale = fp32(amax/448), code = e4m3_rne_satfinite(fp32(v *
 * fp32(448/amax))) (an all-zero row gets scale 1); the e4m3 codes and
 * scales are left in the workspace (see moe_workspace_layout_t). */
int moe_forward_fp8(const void *x, const float *topk_w, const void *routing,
                    const moe_packed_weights_t *w1, const float *w1_scale,
                    const moe_packed_weights_t *w2, const float *w2_scale,
                    int T, int k, int E, int H, int I,
                    void *workspace, size_t workspace_bytes, void *out, void *stream);

/* Routing build and forward pass in one call (blog section "MoE", PDL
 * chaining, and its observation that at decode the metadata build costs
 * about as much as the expert GEMMs).  Results are those of
 * moe_build_routing_bf16 / _fp8 on topk_ids followed by moe_forward_bf16 /
 * _fp8: `routing` (device, 16-byte aligned, routing_bytes >=
 * moe_routing_layout().total_bytes) receives the same bytes, `out` and the
 * workspace the same values.  topk_ids (device) int32 [T][k]; the other
 * arguments as in the forward calls.  A decode batch of at most 64 pairs
 * (T * k <= 64) on the register-streaming plan is routed inside the
 * forward's first kernel (bf16: the gate-up GEMM, on 16-row tiles; fp8: the
 * x quantisation), whose workgroup 0 also writes the routing buffer: one
 * dependent launch fewer.  Otherwise the routing build is launched first.
 * All arguments are checked before anything is enqueued. */
int moe_route_forward_bf16(const int32_t *topk_ids, const void *x, const float *topk_w,
                           void *routing, size_t routing_bytes,
                           const moe_packed_weights_t *w1, const moe_packed_weights_t *w2,
                           int T, int k, int E, int H, int I,
                           void *workspace, size_t workspace_bytes, void *out, void *stream);
int moe_route_forward_fp8(const int32_t *topk_ids, const void *x, const float *topk_w,
                          void *routing, size_t routing_bytes,
                          const moe_packed_weights_t *w1, const float *w1_scale,
                          const moe_packed_weights_t *w2, const float *w2_scale,
                          int T, int k, int E, int H, int I,
                          void *workspace, size_t workspace_bytes, void *out, void *stream);
/* The same for the quantised layers below: moe_build_routing_int8 /
 * _fp8_block / _mxfp8 / _int4 / _int8_w8a16 followed by the forward call of
 * the same dtype, in one call, with the same results; at most 64 pairs on
 * the register-streaming plan are routed inside the x quantisation (int8
 * w8a8, block fp8, MXFP8) or the gate-up GEMM on 16-row tiles (int4 w4a16,
 * int8 w8a16). */
int moe_route_forward_int8(const int32_t *topk_ids, const void *x, const float *topk_w,
                           void *routing, size_t routing_bytes,
                           const moe_packed_weights_t *w1, const float *w1_scale,
                           const moe_packed_weights_t *w2, const float *w2_scale,
                           int T, int k, int E, int H, int I,
                           void *workspace, size_t workspace_bytes, void *out, void *stream);
int moe_route_forward_fp8_block(const int32_t *topk_ids, const void *x, const float *topk_w,
                                void *routing, size_t routing_bytes,
                                const moe_packed_weights_t *w1, const float *w1_scale,
                                const moe_packed_weights_t *w2, const float *w2_scale,
                                int T, int k, int E, int H, int I,
                                void *workspace, size_t workspace_bytes, void *out, void *stream);
int moe_route_forward_mxfp8(const int32_t *topk_ids, const void *x, const float *topk_w,
                            void *routing, size_t routing_bytes,
                            const moe_packed_weights_t *w1, const uint8_t *w1_scale,
                            const moe_packed_weights_t *w2, const uint8_t *w2_scale,
                            int T, int k, int E, int H, int I,
                            void *workspace, size_t workspace_bytes, void *out, void *stream);
int moe_route_forward_int4(const int32_t *topk_ids, const void *x, const float *topk_w,
                           void *routing, size_t routing_bytes,
                           const moe_packed_weights_t *w1, const float *w1_scale,
                           const moe_packed_weights_t *w2, const float *w2_scale,
                           int T, int k, int E, int H, int I,
                           void *workspace, size_t workspace_bytes, void *out, void *stream);
int moe_route_forward_int8_w8a16(const int32_t *topk_ids, const void *x, const float *topk_w,
                                 void *routing, size_t routing_bytes,
                                 const moe_packed_weights_t *w1, const float *w1_scale,
                                 const moe_packed_weights_t *w2, const float *w2_scale,
                                 int T, int k, int E, int H, int I,
                                 void *workspace, size_t workspace_bytes, void *out, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the fp8
 * w8a8 forward of moe_forward_fp8, same arguments and results, without the
 * workspace argument.  Its workspace is a fixed array in device memory that
 * the library holds on every GPU it runs on until the process ends,
 * MOE_STATIC_WORKSPACE_BYTES (64 MiB) per GPU: enough for decode and small
 * batches (moe_workspace_layout().total_bytes tells; DeepSeek-V3-shaped
 * layers up to T = 128 tokens).  A call whose workspace would be larger
 * returns MOE_ERR_BUFFER_TOO_SMALL before anything is enqueued.  Nothing is
 * allocated or freed: the first call on a device looks up the array's
 * device address (hipGetSymbolAddress) and keeps it, so make that first
 * call outside graph capture.  Every call on a GPU shares that GPU's
 * array, which keeps the last call's contents (no part of it needs to start
 * at any value): calls that overlap on one GPU, on different streams or
 * threads, race.  The intermediate codes and scales are not readable by
 * the caller (they are on moe_forward_fp8's workspace). */
#define MOE_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
int moe_forward_fp8_noalloc(const void *x, const float *topk_w, const void *routing,
                            const moe_packed_weights_t *w1, const float *w1_scale,
                            const moe_packed_weights_t *w2, const float *w2_scale,
                            int T, int k, int E, int H, int I, void *out, void *stream);

/* MXFP8 (SGLang tuning guide, block shapes: gfx95 devices keep MXFP8's
 * [1, 32] blocks).  Routing build: as moe_build_routing_bf16, with the
 * tile height of the MXFP8 forward.  Forward: as moe_forward_fp8 except the
 * scales: w1_scale (device) uint8 e8m0 codes [E][2I][H/32] and w2_scale
 * (device) uint8 [E][H][I/32], code c meaning 2^(c - 127), one per 32
 * consecutive values of a weight row (4-byte aligned); w1/w2 (host)
 * describe e4m3 codes packed by moe_pack_weights with dtype MOE_DTYPE_MXFP8
 * (the fp8 layout).
 * x is quantised per token and SiLU(gate)*up per (token, expert) row in
 * blocks of 32 by the OCP rule: scale 2^s, s = floor(log2(max|v|)) - 8
 * clamped to [-127, 127] (-127 for an all-zero block), codes =
 * e4m3_rne_satfinite(v * 2^-s); codes and scale codes stay in the
 * workspace.  The block scales are applied by the scaled MFMA instruction
 * inside the K loop.  H and I must be multiples of 128. */
int moe_build_routing_mxfp8(const int32_t *topk_ids, int T, int k, int E, int H, int I,
                            void *routing, size_t routing_bytes, void *stream);
int moe_forward_mxfp8(const void *x, const float *topk_w, const void *routing,
                      const moe_packed_weights_t *w1, const uint8_t *w1_scale,
                      const moe_packed_weights_t *w2, const uint8_t *w2_scale,
                      int T, int k, int E, int H, int I,
                      void *workspace, size_t workspace_bytes, void *out, void *stream);

/* int8 w8a8 with per-channel weight scales (SGLang tuning guide: the
 * int8_w8a8 dtype with per-channel quantisation).  As the fp8 pair, with
 * int8 codes: w1/w2 (host) describe int8 [E][2I][H] / [E][H][I] packed by
 * moe_pack_weights with dtype MOE_DTYPE_INT8_W8A8, w1_scale / w2_scale
 * fp32 per output row.  x is quantised per token and SiLU(gate)*up per
 * (token, expert) row by scale = fp32(amax/127), code =
 * clamp(round_half_even(fp32(v * fp32(127/amax))), -127, 127) (an
 * all-zero row: scale 1); the products run on the int8 MFMA with int32
 * accumulation. */
int moe_build_routing_int8(const int32_t *topk_ids, int T, int k, int E, int H, int I,
                           void *routing, size_t routing_bytes, void *stream);
int moe_forward_int8(const void *x, const float *topk_w, const void *routing,
                     const moe_packed_weights_t *w1, const float *w1_scale,
                     const moe_packed_weights_t *w2, const float *w2_scale,
                     int T, int k, int E, int H, int I,
                     void *workspace, size_t workspace_bytes, void *out, void *stream);

/* Block-scaled fp8 (SGLang tuning guide: block_shape [128, 128], the
 * quantisation of DeepSeek-V3 checkpoints).  As the fp8 pair except the
 * scales: w1_scale (device) fp32 [E][2I/128][H/128] and w2_scale (device)
 * fp32 [E][H/128][I/128], one per 128 x 128 block of the weight matrix;
 * x is quantised per token and SiLU(gate)*up per (token, expert) row in
 * groups of 128 values, each group by the per-row rule of moe_forward_fp8.
 * w1/w2 (host) describe codes packed by moe_pack_weights with dtype MOE_DTYPE_FP8_BLOCK (the
 * fp8 layout).  H and I must be multiples of 128. */
int moe_build_routing_fp8_block(const int32_t *topk_ids, int T, int k, int E, int H, int I,
                                void *routing, size_t routing_bytes, void *stream);
int moe_forward_fp8_block(const void *x, const float *topk_w, const void *routing,
                          const moe_packed_weights_t *w1, const float *w1_scale,
                          const moe_packed_weights_t *w2, const float *w2_scale,
                          int T, int k, int E, int H, int I,
                          void *workspace, size_t workspace_bytes, void *out, void *stream);

/* int4 w4a16 (SGLang tuning guide dtype list: int4_w4a16).  w1 / w2 (host)
 * describe uint8 [E][2I][H/2] / [E][H][I/2] (device): two's-complement
 * int4 codes, two a byte, the lower K index in the low nibble, packed by
 * moe_pack_weights with dtype MOE_DTYPE_INT4_W4A16 (cols = the K length);
 * w1_scale (device) fp32 [E][2I][H/128], w2_scale (device) fp32
 * [E][H][I/128]: weight (n, k) = code * scale[n][k / 128].  x and the
 * intermediate stay bf16 (bf16 MFMA on weights converted in registers,
 * fp32 accumulation, the group scale applied per 128 K values).  H and I
 * must be multiples of 128. */
int moe_build_routing_int4(const int32_t *topk_ids, int T, int k, int E, int H, int I,
                           void *routing, size_t routing_bytes, void *stream);
int moe_forward_int4(const void *x, const float *topk_w, const void *routing,
                     const moe_packed_weights_t *w1, const float *w1_scale,
                     const moe_packed_weights_t *w2, const float *w2_scale,
                     int T, int k, int E, int H, int I,
                     void *workspace, size_t workspace_bytes, void *out, void *stream);

/* int8 w8a16 (SGLang tuning guide dtype list: int8_w8a16, weight-only
 * int8).  w1 / w2 (host) describe int8 [E][2I][H] / [E][H][I] (device),
 * packed by moe_pack_weights with dtype MOE_DTYPE_INT8_W8A16; w1_scale
 * (device) fp32 [E][2I], w2_scale (device) fp32 [E][H]: weight (n, k) =
 * code * scale[n].  x and the intermediate stay bf16 (bf16 MFMA on weights
 * converted in registers, fp32 accumulation, the row scale applied to the
 * sums).  Register streaming at every T.  Errors as moe_forward_bf16. */
int moe_build_routing_int8_w8a16(const int32_t *topk_ids, int T, int k, int E, int H, int I,
                                 void *routing, size_t routing_bytes, void *stream);
int moe_forward_int8_w8a16(const void *x, const float *topk_w, const void *routing,
                           const moe_packed_weights_t *w1, const float *w1_scale,
                           const moe_packed_weights_t *w2, const float *w2_scale,
                           int T, int k, int E, int H, int I,
                           void *workspace, size_t workspace_bytes, void *out, void *stream);

/* Measurement hook.  When `events` is non-NULL (n >= 10 hipEvent_t
 * handles, host array), every later forward call records events[2*s]
 * before and events[2*s+1] after stage s on its stream, for the stages it
 * runs: 0 activation quantisation (fp8), 1 gate-up GEMM, 2 SiLU-and-mul /
 * requantisation, 3 down GEMM, 4 top-k reduction.  A stage whose two
 * entries are both NULL is not recorded (each record costs a few
 * microseconds of stream time); a pair with one NULL entry, or no
 * non-NULL pair, is an invalid argument.  NULL `events` switches the hook
 * off.  The setting is process-wide and not thread-safe; do not enable it
 * while a forward call is being captured into a graph. */
int moe_set_stage_events(void *const *events, int n);

/* Measurement aid (the attainable HBM read rate that the weight stream of the
 * layer is set against): reads `bytes` of buf (device, 16-byte aligned,
 * bytes a multiple of 16) once, with non-temporal 16-byte loads in whole
 * 1 KiB runs per wave and 32 KiB contiguous chunks per workgroup, spread
 * over every compute unit, and writes one word per workgroup to sink
 * (device, 4-byte aligned, sink_words >= 1 words; min(sink_words, 8 x
 * compute units) workgroups run).  The words are a fold of the data read
 * and carry no other meaning.  bytes == 0 returns MOE_OK with no launch. */
int moe_stream_read(const void *buf, size_t bytes, uint32_t *sink, size_t sink_words, void *stream);

/* Measurement aid (what a token-tile copy into LDS costs, apart from the
 * GEMMs around it): one workgroup of 8 waves per compute unit copies, reps
 * times, every 1 KiB chunk of a 160-row x row_bytes tile (row-major in buf,
 * device) into LDS with direct global->LDS copies, the workgroups of one XCD
 * in groups of 16 on the same tile, so that after the first pass the copies
 * hit L2.  pattern selects the lanes' sources of one chunk: 0 = 1 KiB
 * contiguous (as the packed weights are copied), 1 = 16 rows x 64 bytes with
 * lane l on row l % 16 (MFMA lane order), 2 = the same 16 x 64 bytes with
 * each row's 64 bytes on one quad of lanes (the token-chunk layout of the
 * LDS-staged GEMMs).  row_bytes: a positive multiple of 2048; bytes: the
 * size of buf, at least (compute units / 128) x 8 x 160 x row_bytes
 * (MOE_ERR_BUFFER_TOO_SMALL otherwise); sink (device, 4-byte aligned) takes
 * one word per workgroup, sink_words >= compute units.  Needs >= 128 compute
 * units (MOE_ERR_UNSUPPORTED_SHAPE).  Bytes moved = compute units x reps x
 * 160 x row_bytes.  reps == 0 returns MOE_OK with no launch. */
int moe_tile_copy_read(int pattern, const void *buf, size_t bytes, int row_bytes, int reps, uint32_t *sink,
                       size_t sink_words, void *stream);

/* Number of compute units of the current device as cached by the library
 * (queried once per device), or a negative status. */
int moe_device_cu_count(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
