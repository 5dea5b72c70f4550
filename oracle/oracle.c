/*
 * Plain CPU oracle of the fused Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the benchmark's CPU-baseline leg use it.  It shares no code,
 * header, table or constant generator with the HIP library.
 *
 * What it computes (HPC-Ops x SGLang blog, section "MoE: reducing overhead
 * around small expert GEMMs"): the routed SwiGLU mixture
 *
 *     out[t] = sum_j w[t][j] * W2[e_j] * ( SiLU(W1g[e_j] x[t]) * (W1u[e_j] x[t]) )
 *
 * The fused pipeline of that section (routing and index build, gate-up
 * through the route index, SiLU-and-mul with FP8 requant, down GEMM, top-k
 * weighted reduction back to token order) changes the data flow, not the
 * result, so this oracle is the plain definition: a loop over tokens, and
 * for each token a loop over its k experts in ascending j, in fp64.
 *
 * Readings of points the pages leave open (each also listed in the design
 * notes of the repository):
 *  - W1[e] is [2I][H]: rows [0,I) gate, rows [I,2I) up (the SGLang guide,
 *    section 4.1, stacks gate and up into 2*I rows and halves N after
 *    silu_and_mul).  W2[e] is [H][I].
 *  - SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g)).
 *  - The routing weight multiplies the down projection's output of that
 *    pair, in the top-k weighted reduction.
 *  - An expert id outside [0, E) marks a dropped pair: it belongs to no
 *    expert and adds nothing to the output.  Duplicate ids of one token are
 *    separate pairs and both count.
 *  - Within an expert's contiguous range of the routing, pairs are in
 *    ascending pair index p = t*k + j (a stable counting sort).
 *  - The per-tile task map is a flat expert-major list of row tiles of
 *    height BM; a partial last tile carries its row count.
 *  - FP8 is OCP E4M3 ("e4m3fn": bias 7, max finite 448, no infinities,
 *    NaN = S.1111.111).  Per-row activation quantisation: amax = max|v|,
 *    scale = fp32(amax/448), inv = fp32(448/amax) (both divisions in fp64,
 *    then rounded to fp32), code = e4m3_rne_satfinite(fp32(v * inv)); an
 *    all-zero row gets scale 1 and all codes 0.  x is quantised per token;
 *    the intermediate is quantised per (token, expert) row.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off (no -ffast-math), so every fp64
 * sum keeps the order written here.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double BF16_VALUE[65536];
static double E4M3_VALUE[256];
static int tables_ready = 0;

/* Value tables built from the two format definitions (sign, biased
 * exponent, mantissa), not from any bit reinterpretation. */
void oracle_init(void)
{
    if (tables_ready)
        return;
    for (int c = 0; c < 65536; c++) {
        int s = c >> 15, ex = (c >> 7) & 0xFF, m = c & 0x7F;
        double v;
        if (ex == 0xFF)
            v = m ? NAN : INFINITY;
        else if (ex == 0)
            v = ldexp((double)m, -126 - 7);          /* 0.m * 2^-126 */
        else
            v = ldexp(128.0 + m, ex - 127 - 7);      /* 1.m * 2^(ex-127) */
        BF16_VALUE[c] = s ? -v : v;
    }
    for (int c = 0; c < 256; c++) {
        int s = c >> 7, ex = (c >> 3) & 0xF, m = c & 7;
        double v;
        if (ex == 15 && m == 7)
            v = NAN;
        else if (ex == 0)
            v = ldexp((double)m, -6 - 3);            /* 0.m * 2^-6 */
        else
            v = ldexp(8.0 + m, ex - 7 - 3);          /* 1.m * 2^(ex-7) */
        E4M3_VALUE[c] = s ? -v : v;
    }
    tables_ready = 1;
}

double oracle_bf16_value(int code) { oracle_init(); return BF16_VALUE[code & 0xFFFF]; }
double oracle_e4m3_value(int code) { oracle_init(); return E4M3_VALUE[code & 0xFF]; }

/* Nearest E4M3 value to v, ties to the even mantissa (code LSB 0),
 * saturating to +-448.  Codes 0..126 are the non-negative finite values in
 * ascending order, so the two neighbours of |v| are found by bisection. */
int oracle_e4m3_encode(float v)
{
    oracle_init();
    if (isnan(v))
        return 0x7F;
    int sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (a >= 448.0)
        return sign | 0x7E;
    int lo = 0, hi = 126;                 /* invariant: E4M3_VALUE[lo] <= a */
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (E4M3_VALUE[mid] <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    int c = lo;
    if (lo < 126) {
        double below = a - E4M3_VALUE[lo];
        double above = E4M3_VALUE[lo + 1] - a;
        if (above < below || (above == below && (lo & 1)))
            c = lo + 1;
    }
    return sign | c;
}

/* Per-row activation quantisation rule (see header).  v holds fp32 values. */
void oracle_quant_row(const float *v, int n, uint8_t *codes, float *scale)
{
    float amax = 0.0f;
    for (int i = 0; i < n; i++) {
        float a = fabsf(v[i]);
        if (a > amax)
            amax = a;
    }
    if (amax == 0.0f) {
        *scale = 1.0f;
        memset(codes, 0, (size_t)n);
        return;
    }
    float s = (float)((double)amax / 448.0);
    float inv = (float)(448.0 / (double)amax);
    for (int i = 0; i < n; i++) {
        float prod = v[i] * inv;          /* one fp32 multiply */
        codes[i] = (uint8_t)oracle_e4m3_encode(prod);
    }
    *scale = s;
}

/* Per-token quantisation of bf16 rows x[T][H] (the fp8 path's first step). */
void oracle_quant_rows_bf16(const uint16_t *x, int T, int H, uint8_t *codes, float *scales)
{
    oracle_init();
    float *row = (float *)malloc(sizeof(float) * (size_t)(H > 0 ? H : 1));
    for (int t = 0; t < T; t++) {
        for (int h = 0; h < H; h++)
            row[h] = (float)BF16_VALUE[x[(size_t)t * H + h]];
        oracle_quant_row(row, H, codes + (size_t)t * H, scales + t);
    }
    free(row);
}

/* ------------------------------------------------------------------------
 * Routing and index build (blog section "MoE", routing & index build):
 * a counting pass over the top-k expert ids that gives every expert a
 * contiguous output range, the route index (sorted position -> pair and
 * its inverse) and a per-tile task map.
 *
 *   ids[P]      expert id of pair p = t*k + j
 *   offsets[E+1] start of each expert's range; offsets[E] = valid pairs
 *   sorted[P]   pair index at each sorted position; dropped pairs fill
 *               [offsets[E], P) in ascending p
 *   pos[P]      inverse of sorted
 *   tasks[4*n]  {expert, row_begin, rows, 0} row tiles of height BM,
 *               expert-major; experts without pairs emit none
 * Returns 0, or -1 if max_tasks is too small.
 * ---------------------------------------------------------------------- */
int oracle_route(const int32_t *ids, int P, int E, int BM,
                 int32_t *offsets, int32_t *sorted, int32_t *pos,
                 int32_t *tasks, int max_tasks, int32_t *num_tasks, int32_t *num_dropped)
{
    int32_t *count = (int32_t *)calloc((size_t)E + 1, sizeof(int32_t));
    int32_t *cursor = (int32_t *)calloc((size_t)E + 1, sizeof(int32_t));
    for (int p = 0; p < P; p++) {
        int e = ids[p];
        if (e >= 0 && e < E)
            count[e]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; e++)
        offsets[e + 1] = offsets[e] + count[e];
    for (int e = 0; e < E; e++)
        cursor[e] = offsets[e];
    int dropped_cursor = offsets[E];
    for (int p = 0; p < P; p++) {
        int e = ids[p];
        int r;
        if (e >= 0 && e < E)
            r = cursor[e]++;
        else
            r = dropped_cursor++;
        sorted[r] = p;
        pos[p] = r;
    }
    *num_dropped = P - offsets[E];
    int n = 0, rc = 0;
    for (int e = 0; e < E; e++) {
        for (int m0 = 0; m0 < count[e]; m0 += BM) {
            if (n >= max_tasks) {
                rc = -1;
                continue;
            }
            int rows = count[e] - m0 < BM ? count[e] - m0 : BM;
            tasks[4 * n + 0] = e;
            tasks[4 * n + 1] = offsets[e] + m0;
            tasks[4 * n + 2] = rows;
            tasks[4 * n + 3] = 0;
            n++;
        }
    }
    *num_tasks = n;
    free(count);
    free(cursor);
    return rc;
}

/* ------------------------------------------------------------------------
 * Forward pass.  Matrices are viewed through a tag so one plain loop serves
 * fp64, fp32, bf16-code and e4m3-code storage; a row is decoded to fp64
 * before use.
 * ---------------------------------------------------------------------- */
enum { K_F64 = 0, K_F32 = 1, K_BF16 = 2, K_E4M3 = 3 };

static void load_row(int kind, const void *base, size_t off, int n, double *dst)
{
    switch (kind) {
    case K_F64: { const double *p = (const double *)base + off; for (int i = 0; i < n; i++) dst[i] = p[i]; break; }
    case K_F32: { const float *p = (const float *)base + off; for (int i = 0; i < n; i++) dst[i] = (double)p[i]; break; }
    case K_BF16: { const uint16_t *p = (const uint16_t *)base + off; for (int i = 0; i < n; i++) dst[i] = BF16_VALUE[p[i]]; break; }
    case K_E4M3: { const uint8_t *p = (const uint8_t *)base + off; for (int i = 0; i < n; i++) dst[i] = E4M3_VALUE[p[i]]; break; }
    }
}

static double dot(const double *a, const double *b, int n)
{
    double s = 0.0;
    for (int i = 0; i < n; i++)
        s += a[i] * b[i];
    return s;
}

static double silu(double g) { return g / (1.0 + exp(-g)); }

/* One token of the unquantised layer (x, W1, W2 of any kind). */
static void token_plain(int xkind, const void *x, int wkind, const void *W1, const void *W2,
                        const float *topk_w, const int32_t *ids, int t, int k, int E, int H, int I,
                        double *acc)
{
    double *xr = (double *)malloc(sizeof(double) * (size_t)H);
    double *wr = (double *)malloc(sizeof(double) * (size_t)(H > I ? H : I));
    double *a = (double *)malloc(sizeof(double) * (size_t)I);
    load_row(xkind, x, (size_t)t * H, H, xr);
    for (int m = 0; m < H; m++)
        acc[m] = 0.0;
    for (int j = 0; j < k; j++) {
        int p = t * k + j;
        int e = ids[p];
        if (e < 0 || e >= E)
            continue;
        double w = (double)topk_w[p];
        for (int n = 0; n < I; n++) {
            load_row(wkind, W1, ((size_t)e * 2 * I + n) * H, H, wr);
            double g = dot(wr, xr, H);
            load_row(wkind, W1, ((size_t)e * 2 * I + I + n) * H, H, wr);
            double u = dot(wr, xr, H);
            a[n] = silu(g) * u;
        }
        for (int m = 0; m < H; m++) {
            load_row(wkind, W2, ((size_t)e * H + m) * I, I, wr);
            double y = dot(wr, a, I);
            acc[m] += w * y;
        }
    }
    free(xr);
    free(wr);
    free(a);
}

/* rows[0..nrows) are the tokens to evaluate (NULL: all T, nrows = T);
 * out is [nrows][H] fp64. */
static void forward_plain(int xkind, const void *x, int wkind, const void *W1, const void *W2,
                          const float *topk_w, const int32_t *ids, int T, int k, int E, int H, int I,
                          const int32_t *rows, int nrows, double *out)
{
    oracle_init();
    if (!rows)
        nrows = T;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; r++) {
        int t = rows ? rows[r] : r;
        token_plain(xkind, x, wkind, W1, W2, topk_w, ids, t, k, E, H, I, out + (size_t)r * H);
    }
}

void oracle_forward_f64(const double *x, const float *topk_w, const int32_t *ids,
                        const double *W1, const double *W2, int T, int k, int E, int H, int I,
                        const int32_t *rows, int nrows, double *out)
{
    forward_plain(K_F64, x, K_F64, W1, W2, topk_w, ids, T, k, E, H, I, rows, nrows, out);
}

void oracle_forward_f32(const float *x, const float *topk_w, const int32_t *ids,
                        const float *W1, const float *W2, int T, int k, int E, int H, int I,
                        const int32_t *rows, int nrows, double *out)
{
    forward_plain(K_F32, x, K_F32, W1, W2, topk_w, ids, T, k, E, H, I, rows, nrows, out);
}

void oracle_forward_bf16(const uint16_t *x, const float *topk_w, const int32_t *ids,
                         const uint16_t *W1, const uint16_t *W2, int T, int k, int E, int H, int I,
                         const int32_t *rows, int nrows, double *out)
{
    forward_plain(K_BF16, x, K_BF16, W1, W2, topk_w, ids, T, k, E, H, I, rows, nrows, out);
}

/* One token of the fp8 w8a8 layer.  x is bf16; W1/W2 are e4m3 codes with
 * one fp32 scale per output channel (s1[e][2I], s2[e][H]). */
static void token_fp8(const uint16_t *x, const float *topk_w, const int32_t *ids,
                      const uint8_t *W1, const float *s1, const uint8_t *W2, const float *s2,
                      int t, int k, int E, int H, int I, double *acc,
                      uint8_t *xq_out, float *sx_out, uint8_t *hq_out, float *sh_out)
{
    float *xf = (float *)malloc(sizeof(float) * (size_t)H);
    uint8_t *xq = (uint8_t *)malloc((size_t)H);
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    double *wr = (double *)malloc(sizeof(double) * (size_t)(H > I ? H : I));
    float *af = (float *)malloc(sizeof(float) * (size_t)I);
    uint8_t *hq = (uint8_t *)malloc((size_t)I);
    double *hd = (double *)malloc(sizeof(double) * (size_t)I);
    float sx;

    for (int h = 0; h < H; h++)
        xf[h] = (float)BF16_VALUE[x[(size_t)t * H + h]];
    oracle_quant_row(xf, H, xq, &sx);
    if (xq_out) {
        memcpy(xq_out, xq, (size_t)H);
        *sx_out = sx;
    }
    load_row(K_E4M3, xq, 0, H, xd);
    for (int m = 0; m < H; m++)
        acc[m] = 0.0;
    for (int j = 0; j < k; j++) {
        int p = t * k + j;
        int e = ids[p];
        if (e < 0 || e >= E)
            continue;
        double w = (double)topk_w[p];
        for (int n = 0; n < I; n++) {
            load_row(K_E4M3, W1, ((size_t)e * 2 * I + n) * H, H, wr);
            double g = (double)sx * (double)s1[(size_t)e * 2 * I + n] * dot(wr, xd, H);
            load_row(K_E4M3, W1, ((size_t)e * 2 * I + I + n) * H, H, wr);
            double u = (double)sx * (double)s1[(size_t)e * 2 * I + I + n] * dot(wr, xd, H);
            af[n] = (float)(silu(g) * u);
        }
        float sh;
        oracle_quant_row(af, I, hq, &sh);
        if (hq_out) {
            memcpy(hq_out + (size_t)j * I, hq, (size_t)I);
            sh_out[j] = sh;
        }
        load_row(K_E4M3, hq, 0, I, hd);
        for (int m = 0; m < H; m++) {
            load_row(K_E4M3, W2, ((size_t)e * H + m) * I, I, wr);
            double y = (double)sh * (double)s2[(size_t)e * H + m] * dot(wr, hd, I);
            acc[m] += w * y;
        }
    }
    free(xf); free(xq); free(xd); free(wr); free(af); free(hq); free(hd);
}

/* fp8 w8a8 forward.  Optional outputs (may be NULL): xq_out [nrows][H] and
 * sx_out [nrows] (the token's quantised activations), hq_out [nrows][k][I]
 * and sh_out [nrows][k] (each pair's quantised intermediate; rows of
 * dropped pairs are left untouched). */
void oracle_forward_fp8(const uint16_t *x, const float *topk_w, const int32_t *ids,
                        const uint8_t *W1, const float *s1, const uint8_t *W2, const float *s2,
                        int T, int k, int E, int H, int I, const int32_t *rows, int nrows,
                        double *out, uint8_t *xq_out, float *sx_out, uint8_t *hq_out, float *sh_out)
{
    oracle_init();
    if (!rows)
        nrows = T;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; r++) {
        int t = rows ? rows[r] : r;
        token_fp8(x, topk_w, ids, W1, s1, W2, s2, t, k, E, H, I, out + (size_t)r * H,
                  xq_out ? xq_out + (size_t)r * H : NULL, sx_out ? sx_out + r : NULL,
                  hq_out ? hq_out + (size_t)r * k * I : NULL, sh_out ? sh_out + (size_t)r * k : NULL);
    }
}

/*
 * Router top-k (HPC-Ops x SGLang blog, section "Router GEMM: balancing
 * routing precision and throughput": the router's fp32 expert scores feed
 * a top-k choice that decides which experts run; SGLang fused-MoE tuning
 * guide, section on model-config parsing: shared experts fused into the
 * expert tensor as extra expert ids).  The steps, in order, for one token:
 *
 *  1. softmax over all E scores: p_e = exp(l_e - max) / sum_e' exp(l_e' - max);
 *  2. top-k: the k experts of largest p_e, listed by descending p_e, equal
 *     scores by ascending expert id.  Softmax is strictly increasing in the
 *     logit, so the ranking is made on the fp32 logits themselves: ranking
 *     the rounded probabilities would invent ties that the exact softmax
 *     does not have;
 *  3. renormalise (when asked): w_j = p_j / sum of the k selected p;
 *     otherwise w_j = p_j;
 *  4. shared experts: n_shared extra columns j = k .. k+n_shared-1 hold
 *     expert ids E, E+1, ... with weight 1 (every token runs them, and
 *     their output adds to the routed mixture unscaled).
 *
 * A NaN logit ranks as -infinity.  Weights are exact fp64 arithmetic on
 * the fp32 inputs; they are meaningful only when the selected logits are
 * finite.  ids is [T][k+n_shared], w is [T][k+n_shared] fp64.
 */
static double rank_value(float v) { return isnan(v) ? -INFINITY : (double)v; }

void oracle_router_topk(const float *logits, int T, int E, int k, int renormalize,
                        int n_shared, int32_t *ids, double *w)
{
    const int ncol = k + n_shared;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        const float *l = logits + (size_t)t * E;
        double *p = malloc(sizeof(double) * (size_t)E);
        char *taken = calloc((size_t)E, 1);
        double mx = -INFINITY;
        for (int e = 0; e < E; e++)
            if (rank_value(l[e]) > mx)
                mx = rank_value(l[e]);
        double total = 0.0;
        for (int e = 0; e < E; e++) {
            p[e] = exp(rank_value(l[e]) - mx);
            total += p[e];
        }
        for (int e = 0; e < E; e++)
            p[e] /= total;
        int32_t *row_ids = ids + (size_t)t * ncol;
        double *row_w = w + (size_t)t * ncol;
        double sel_sum = 0.0;
        for (int j = 0; j < k; j++) {   /* selection: best remaining, lowest id on ties */
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (taken[e])
                    continue;
                if (best < 0 || rank_value(l[e]) > rank_value(l[best]))
                    best = e;
            }
            taken[best] = 1;
            row_ids[j] = best;
            row_w[j] = p[best];
            sel_sum += p[best];
        }
        if (renormalize)
            for (int j = 0; j < k; j++)
                row_w[j] /= sel_sum;
        for (int s = 0; s < n_shared; s++) {
            row_ids[k + s] = E + s;
            row_w[k + s] = 1.0;
        }
        free(p);
        free(taken);
    }
}

/*
 * int8 w8a8 with per-channel weight scales (SGLang tuning guide: the
 * int8_w8a8 dtype with per-channel quantisation, for channel-INT8 MoE
 * checkpoints).  Symmetric per-row rule, the fp8 rule with 127 for 448:
 * amax = max|v|, scale = fp32(amax/127), inv = fp32(127/amax) (divisions in
 * fp64), code = clamp(round_half_even(fp32(v * inv)), -127, 127); an
 * all-zero row gets scale 1 and codes 0.  Weights carry one fp32 scale per
 * output row; x is quantised per token and the intermediate per (token,
 * expert) row.  int8 dot products are exact in fp64.
 */
void oracle_int8_quant_row(const float *v, int n, int8_t *q, float *scale)
{
    float amax = 0.0f;
    for (int i = 0; i < n; i++)
        if (fabsf(v[i]) > amax)
            amax = fabsf(v[i]);
    if (amax == 0.0f) {
        *scale = 1.0f;
        memset(q, 0, (size_t)n);
        return;
    }
    const float inv = (float)(127.0 / (double)amax);
    for (int i = 0; i < n; i++) {
        float prod = v[i] * inv;                      /* one fp32 multiply */
        double r = nearbyint((double)prod);           /* ties to even (default mode) */
        if (r > 127.0)
            r = 127.0;
        if (r < -127.0)
            r = -127.0;
        q[i] = (int8_t)r;
    }
    *scale = (float)((double)amax / 127.0);
}

void oracle_int8_quant_rows_bf16(const uint16_t *x, int T, int H, int8_t *q, float *scales)
{
    oracle_init();
    float *row = (float *)malloc(sizeof(float) * (size_t)(H > 0 ? H : 1));
    for (int t = 0; t < T; t++) {
        for (int h = 0; h < H; h++)
            row[h] = (float)BF16_VALUE[x[(size_t)t * H + h]];
        oracle_int8_quant_row(row, H, q + (size_t)t * H, scales + t);
    }
    free(row);
}

static double dot_i8(const int8_t *a, const int8_t *b, int n)
{
    long long s = 0;
    for (int i = 0; i < n; i++)
        s += (long long)a[i] * (long long)b[i];
    return (double)s;
}

static void token_int8(const uint16_t *x, const float *topk_w, const int32_t *ids,
                       const int8_t *W1, const float *s1, const int8_t *W2, const float *s2,
                       int t, int k, int E, int H, int I, double *acc,
                       int8_t *xq_out, float *sx_out, int8_t *hq_out, float *sh_out)
{
    float *xf = (float *)malloc(sizeof(float) * (size_t)H);
    int8_t *xq = (int8_t *)malloc((size_t)H);
    float *af = (float *)malloc(sizeof(float) * (size_t)I);
    int8_t *hq = (int8_t *)malloc((size_t)I);
    float sx, sh;
    for (int h = 0; h < H; h++)
        xf[h] = (float)BF16_VALUE[x[(size_t)t * H + h]];
    oracle_int8_quant_row(xf, H, xq, &sx);
    if (xq_out) {
        memcpy(xq_out, xq, (size_t)H);
        *sx_out = sx;
    }
    for (int m = 0; m < H; m++)
        acc[m] = 0.0;
    for (int j = 0; j < k; j++) {
        int p = t * k + j;
        int e = ids[p];
        if (e < 0 || e >= E)
            continue;
        double w = (double)topk_w[p];
        for (int n = 0; n < I; n++) {
            size_t rg = (size_t)e * 2 * I + n, ru = rg + I;
            double g = (double)sx * (double)s1[rg] * dot_i8(W1 + rg * H, xq, H);
            double u = (double)sx * (double)s1[ru] * dot_i8(W1 + ru * H, xq, H);
            af[n] = (float)(silu(g) * u);
        }
        oracle_int8_quant_row(af, I, hq, &sh);
        if (hq_out) {
            memcpy(hq_out + (size_t)j * I, hq, (size_t)I);
            sh_out[j] = sh;
        }
        for (int m = 0; m < H; m++) {
            size_t r2 = (size_t)e * H + m;
            acc[m] += w * ((double)sh * (double)s2[r2] * dot_i8(W2 + r2 * I, hq, I));
        }
    }
    free(xf); free(xq); free(af); free(hq);
}

void oracle_forward_int8(const uint16_t *x, const float *topk_w, const int32_t *ids,
                         const int8_t *W1, const float *s1, const int8_t *W2, const float *s2,
                         int T, int k, int E, int H, int I, const int32_t *rows, int nrows,
                         double *out, int8_t *xq_out, float *sx_out, int8_t *hq_out, float *sh_out)
{
    oracle_init();
    if (!rows)
        nrows = T;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; r++) {
        int t = rows ? rows[r] : r;
        token_int8(x, topk_w, ids, W1, s1, W2, s2, t, k, E, H, I, out + (size_t)r * H,
                   xq_out ? xq_out + (size_t)r * H : NULL, sx_out ? sx_out + r : NULL,
                   hq_out ? hq_out + (size_t)r * k * I : NULL, sh_out ? sh_out + (size_t)r * k : NULL);
    }
}

/*
 * Block-scaled fp8 w8a8 (SGLang tuning guide: block_shape [128, 128], the
 * quantisation of DeepSeek-V3's checkpoints).  Weights: e4m3 codes with one
 * fp32 scale per 128 x 128 block of a [rows][K] matrix (scale[r/128][k/128]).
 * Activations: e4m3 codes with one fp32 scale per 128 consecutive K values
 * of a row (per-token groups), quantised by the per-row rule of the fp8
 * path applied to each group.  A dot product is the sum over the 128-value
 * groups of (group scale of x) * (block scale of w) * (integer-exact sum of
 * code products).
 */
void oracle_quant_groups(const float *v, int n, uint8_t *codes, float *scales)
{
    for (int g = 0; g < n / 128; g++)
        oracle_quant_row(v + 128 * g, 128, codes + 128 * g, scales + g);
}

static double dot_blocked(const uint8_t *wq, const float *wscale_row, const uint8_t *xq,
                          const float *xscale, int K)
{
    double s = 0.0;
    for (int g = 0; g < K / 128; g++) {
        double part = 0.0;
        for (int k = 128 * g; k < 128 * (g + 1); k++)
            part += E4M3_VALUE[wq[k]] * E4M3_VALUE[xq[k]];
        s += (double)xscale[g] * (double)wscale_row[g] * part;
    }
    return s;
}

static void token_fp8b(const uint16_t *x, const float *topk_w, const int32_t *ids,
                       const uint8_t *W1, const float *s1, const uint8_t *W2, const float *s2,
                       int t, int k, int E, int H, int I, double *acc,
                       uint8_t *xq_out, float *sx_out, uint8_t *hq_out, float *sh_out)
{
    float *xf = (float *)malloc(sizeof(float) * (size_t)H);
    uint8_t *xq = (uint8_t *)malloc((size_t)H);
    float *sx = (float *)malloc(sizeof(float) * (size_t)H / 128);
    float *af = (float *)malloc(sizeof(float) * (size_t)I);
    uint8_t *hq = (uint8_t *)malloc((size_t)I);
    float *sh = (float *)malloc(sizeof(float) * (size_t)I / 128);
    for (int h = 0; h < H; h++)
        xf[h] = (float)BF16_VALUE[x[(size_t)t * H + h]];
    oracle_quant_groups(xf, H, xq, sx);
    if (xq_out) {
        memcpy(xq_out, xq, (size_t)H);
        memcpy(sx_out, sx, sizeof(float) * (size_t)H / 128);
    }
    for (int m = 0; m < H; m++)
        acc[m] = 0.0;
    const int kb1 = H / 128, kb2 = I / 128;
    for (int j = 0; j < k; j++) {
        int p = t * k + j;
        int e = ids[p];
        if (e < 0 || e >= E)
            continue;
        double w = (double)topk_w[p];
        for (int n = 0; n < I; n++) {
            size_t rg = (size_t)e * 2 * I + n, ru = rg + I;
            /* scale rows of W1[e]: block row (row / 128) of [2I/128][H/128] */
            const float *sg = s1 + ((size_t)e * (2 * I / 128) + (size_t)n / 128) * kb1;
            const float *su = s1 + ((size_t)e * (2 * I / 128) + (size_t)(I + n) / 128) * kb1;
            double g = dot_blocked(W1 + rg * H, sg, xq, sx, H);
            double u = dot_blocked(W1 + ru * H, su, xq, sx, H);
            af[n] = (float)(silu(g) * u);
        }
        oracle_quant_groups(af, I, hq, sh);
        if (hq_out) {
            memcpy(hq_out + (size_t)j * I, hq, (size_t)I);
            memcpy(sh_out + (size_t)j * (I / 128), sh, sizeof(float) * (size_t)I / 128);
        }
        for (int m = 0; m < H; m++) {
            size_t r2 = (size_t)e * H + m;
            const float *s2r = s2 + ((size_t)e * (H / 128) + (size_t)m / 128) * kb2;
            acc[m] += w * dot_blocked(W2 + r2 * I, s2r, hq, sh, I);
        }
    }
    free(xf); free(xq); free(sx); free(af); free(hq); free(sh);
}

/* Block-scaled fp8 forward.  s1 fp32 [E][2I/128][H/128], s2 fp32
 * [E][H/128][I/128].  Optional outputs: xq_out [nrows][H], sx_out
 * [nrows][H/128], hq_out [nrows][k][I], sh_out [nrows][k][I/128]. */
void oracle_forward_fp8_block(const uint16_t *x, const float *topk_w, const int32_t *ids,
                              const uint8_t *W1, const float *s1, const uint8_t *W2, const float *s2,
                              int T, int k, int E, int H, int I, const int32_t *rows, int nrows,
                              double *out, uint8_t *xq_out, float *sx_out, uint8_t *hq_out,
                              float *sh_out)
{
    oracle_init();
    if (!rows)
        nrows = T;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; r++) {
        int t = rows ? rows[r] : r;
        token_fp8b(x, topk_w, ids, W1, s1, W2, s2, t, k, E, H, I, out + (size_t)r * H,
                   xq_out ? xq_out + (size_t)r * H : NULL,
                   sx_out ? sx_out + (size_t)r * (H / 128) : NULL,
                   hq_out ? hq_out + (size_t)r * k * I : NULL,
                   sh_out ? sh_out + (size_t)r * k * (I / 128) : NULL);
    }
}

/*
 * int4 w4a16 (SGLang tuning guide dtype list: int4_w4a16): int4 weights
 * with one fp32 scale per 128 consecutive K values of a row (a group), bf16
 * activations.  Weight element (n, k) = q * scale[n][k / 128] with q a
 * two's-complement nibble in [-8, 7]; bytes hold two elements, the lower
 * K index in the low nibble.  The activations are not quantised: the layer
 * is the bf16 layer on the dequantised weights, in fp64 here.
 */
static int nibble(const uint8_t *row, int k)
{
    const int v = (row[k / 2] >> (4 * (k & 1))) & 0xF;
    return v >= 8 ? v - 16 : v;
}

static void w4_row(const uint8_t *codes, const float *scales, int n, double *dst)
{
    for (int k = 0; k < n; k++)
        dst[k] = (double)nibble(codes, k) * (double)scales[k / 128];
}

static void token_w4a16(const uint16_t *x, const float *topk_w, const int32_t *ids,
                        const uint8_t *W1, const float *s1, const uint8_t *W2, const float *s2,
                        int t, int k, int E, int H, int I, double *acc)
{
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    double *wr = (double *)malloc(sizeof(double) * (size_t)(H > I ? H : I));
    double *hd = (double *)malloc(sizeof(double) * (size_t)I);
    for (int h = 0; h < H; h++)
        xd[h] = BF16_VALUE[x[(size_t)t * H + h]];
    for (int m = 0; m < H; m++)
        acc[m] = 0.0;
    for (int j = 0; j < k; j++) {
        int p = t * k + j;
        int e = ids[p];
        if (e < 0 || e >= E)
            continue;
        double w = (double)topk_w[p];
        for (int n = 0; n < I; n++) {
            size_t rg = (size_t)e * 2 * I + n, ru = rg + I;
            w4_row(W1 + rg * (H / 2), s1 + rg * (H / 128), H, wr);
            double g = dot(wr, xd, H);
            w4_row(W1 + ru * (H / 2), s1 + ru * (H / 128), H, wr);
            double u = dot(wr, xd, H);
            hd[n] = silu(g) * u;
        }
        for (int m = 0; m < H; m++) {
            size_t r2 = (size_t)e * H + m;
            w4_row(W2 + r2 * (I / 2), s2 + r2 * (I / 128), I, wr);
            acc[m] += w * dot(wr, hd, I);
        }
    }
    free(xd); free(wr); free(hd);
}

void oracle_forward_w4a16(const uint16_t *x, const float *topk_w, const int32_t *ids,
                          const uint8_t *W1, const float *s1, const uint8_t *W2, const float *s2,
                          int T, int k, int E, int H, int I, const int32_t *rows, int nrows,
                          double *out)
{
    oracle_init();
    if (!rows)
        nrows = T;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; r++) {
        int t = rows ? rows[r] : r;
        token_w4a16(x, topk_w, ids, W1, s1, W2, s2, t, k, E, H, I, out + (size_t)r * H);
    }
}

/* dequantised int4 rows: codes [rows][n/2], scales [rows][n/128] -> dst [rows][n] */
void oracle_w4_dequant(const uint8_t *codes, const float *scales, int rows, int n, double *dst)
{
    for (long r = 0; r < rows; r++)
        w4_row(codes + r * (n / 2), scales + r * (n / 128), n, dst + r * n);
}

/*
 * int8 w8a16 (SGLang tuning guide dtype list: int8_w8a16, weight-only
 * int8): int8 weight codes with one fp32 scale per weight row (per output
 * channel), bf16 activations.  Weight element (n, k) = q[n][k] * scale[n].
 * The activations are not quantised: the layer is the bf16 layer on the
 * dequantised weights, in fp64 here.
 */
static void w8_row(const int8_t *codes, float scale, int n, double *dst)
{
    for (int k = 0; k < n; k++)
        dst[k] = (double)codes[k] * (double)scale;
}

static void token_w8a16(const uint16_t *x, const float *topk_w, const int32_t *ids,
                        const int8_t *W1, const float *s1, const int8_t *W2, const float *s2,
                        int t, int k, int E, int H, int I, double *acc)
{
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    double *wr = (double *)malloc(sizeof(double) * (size_t)(H > I ? H : I));
    double *hd = (double *)malloc(sizeof(double) * (size_t)I);
    for (int h = 0; h < H; h++)
        xd[h] = BF16_VALUE[x[(size_t)t * H + h]];
    for (int m = 0; m < H; m++)
        acc[m] = 0.0;
    for (int j = 0; j < k; j++) {
        int p = t * k + j;
        int e = ids[p];
        if (e < 0 || e >= E)
            continue;
        double w = (double)topk_w[p];
        for (int n = 0; n < I; n++) {
            size_t rg = (size_t)e * 2 * I + n, ru = rg + I;
            w8_row(W1 + rg * H, s1[rg], H, wr);
            double g = dot(wr, xd, H);
            w8_row(W1 + ru * H, s1[ru], H, wr);
            double u = dot(wr, xd, H);
            hd[n] = silu(g) * u;
        }
        for (int m = 0; m < H; m++) {
            size_t r2 = (size_t)e * H + m;
            w8_row(W2 + r2 * I, s2[r2], I, wr);
            acc[m] += w * dot(wr, hd, I);
        }
    }
    free(xd); free(wr); free(hd);
}

void oracle_forward_w8a16(const uint16_t *x, const float *topk_w, const int32_t *ids,
                          const int8_t *W1, const float *s1, const int8_t *W2, const float *s2,
                          int T, int k, int E, int H, int I, const int32_t *rows, int nrows,
                          double *out)
{
    oracle_init();
    if (!rows)
        nrows = T;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; r++) {
        int t = rows ? rows[r] : r;
        token_w8a16(x, topk_w, ids, W1, s1, W2, s2, t, k, E, H, I, out + (size_t)r * H);
    }
}

/*
 * MXFP8 block-scaled fp8 (SGLang tuning guide, section on block shapes:
 * gfx95 devices keep MXFP8's [1, 32] block shape instead of remapping it
 * to [128, 128]).  OCP Microscaling format: every 32 consecutive elements
 * along the reduction dimension share one E8M0 scale X = 2^(c - 127)
 * (c = 0..254) and hold E4M3 elements; the value is X * element.
 * Quantisation of a block (the OCP rule): shared exponent
 *   s = floor(log2(max |v|)) - 8   (8 = the largest E4M3 exponent),
 * clamped to [-127, 127]; an all-zero block takes s = -127;
 * element = e4m3_rne_satfinite(v / 2^s).  v / 2^s is exact in fp32.
 */
static int mx_shared_exp(float amax)
{
    if (!(amax > 0.0f))
        return -127;
    int e;
    frexp((double)amax, &e);          /* amax = m * 2^e, m in [0.5, 1) */
    int s = (e - 1) - 8;              /* floor(log2(amax)) - 8 */
    if (s < -127)
        s = -127;
    if (s > 127)
        s = 127;
    return s;
}

void oracle_mx_quant_block(const float *v, uint8_t *codes, uint8_t *scale_code)
{
    float amax = 0.0f;
    for (int i = 0; i < 32; i++)
        if (fabsf(v[i]) > amax)
            amax = fabsf(v[i]);
    const int s = mx_shared_exp(amax);
    for (int i = 0; i < 32; i++)
        codes[i] = (uint8_t)oracle_e4m3_encode((float)ldexp((double)v[i], -s));
    *scale_code = (uint8_t)(s + 127);
}

/* rows x n values (n % 32 == 0) -> codes [rows][n], scales [rows][n/32] */
void oracle_mx_quant_rows(const float *v, int rows, int n, uint8_t *codes, uint8_t *scales)
{
    oracle_init();
    for (long r = 0; r < rows; r++)
        for (int b = 0; b < n / 32; b++)
            oracle_mx_quant_block(v + r * n + 32 * b, codes + r * n + 32 * b, scales + r * (n / 32) + b);
}

void oracle_mx_quant_rows_bf16(const uint16_t *x, int T, int H, uint8_t *codes, uint8_t *scales)
{
    oracle_init();
    float *row = (float *)malloc(sizeof(float) * (size_t)(H > 0 ? H : 1));
    for (int t = 0; t < T; t++) {
        for (int h = 0; h < H; h++)
            row[h] = (float)BF16_VALUE[x[(size_t)t * H + h]];
        oracle_mx_quant_rows(row, 1, H, codes + (size_t)t * H, scales + (size_t)t * (H / 32));
    }
    free(row);
}

/* dequantised MX row: n values from codes and per-32 scale codes */
static void mx_row(const uint8_t *codes, const uint8_t *scales, int n, double *dst)
{
    for (int i = 0; i < n; i++)
        dst[i] = ldexp(E4M3_VALUE[codes[i]], (int)scales[i / 32] - 127);
}

static void token_mxfp8(const uint16_t *x, const float *topk_w, const int32_t *ids,
                        const uint8_t *W1, const uint8_t *s1, const uint8_t *W2, const uint8_t *s2,
                        int t, int k, int E, int H, int I, double *acc,
                        uint8_t *xq_out, uint8_t *sx_out, uint8_t *hq_out, uint8_t *sh_out)
{
    float *xf = (float *)malloc(sizeof(float) * (size_t)H);
    uint8_t *xq = (uint8_t *)malloc((size_t)H);
    uint8_t *sx = (uint8_t *)malloc((size_t)H / 32);
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    double *wr = (double *)malloc(sizeof(double) * (size_t)(H > I ? H : I));
    float *af = (float *)malloc(sizeof(float) * (size_t)I);
    uint8_t *hq = (uint8_t *)malloc((size_t)I);
    uint8_t *sh = (uint8_t *)malloc((size_t)I / 32);
    double *hd = (double *)malloc(sizeof(double) * (size_t)I);

    for (int h = 0; h < H; h++)
        xf[h] = (float)BF16_VALUE[x[(size_t)t * H + h]];
    oracle_mx_quant_rows(xf, 1, H, xq, sx);
    if (xq_out) {
        memcpy(xq_out, xq, (size_t)H);
        memcpy(sx_out, sx, (size_t)H / 32);
    }
    mx_row(xq, sx, H, xd);
    for (int m = 0; m < H; m++)
        acc[m] = 0.0;
    for (int j = 0; j < k; j++) {
        int p = t * k + j;
        int e = ids[p];
        if (e < 0 || e >= E)
            continue;
        double w = (double)topk_w[p];
        for (int n = 0; n < I; n++) {
            size_t rg = (size_t)e * 2 * I + n, ru = rg + I;
            mx_row(W1 + rg * H, s1 + rg * (H / 32), H, wr);
            double g = dot(wr, xd, H);
            mx_row(W1 + ru * H, s1 + ru * (H / 32), H, wr);
            double u = dot(wr, xd, H);
            af[n] = (float)(silu(g) * u);
        }
        oracle_mx_quant_rows(af, 1, I, hq, sh);
        if (hq_out) {
            memcpy(hq_out + (size_t)j * I, hq, (size_t)I);
            memcpy(sh_out + (size_t)j * (I / 32), sh, (size_t)I / 32);
        }
        mx_row(hq, sh, I, hd);
        for (int m = 0; m < H; m++) {
            size_t r2 = (size_t)e * H + m;
            mx_row(W2 + r2 * I, s2 + r2 * (I / 32), I, wr);
            acc[m] += w * dot(wr, hd, I);
        }
    }
    free(xf); free(xq); free(sx); free(xd); free(wr); free(af); free(hq); free(sh); free(hd);
}

/* MXFP8 forward: x bf16 [T][H]; W1/W2 e4m3 codes with e8m0 scale codes
 * s1 [E][2I][H/32], s2 [E][H][I/32]; x quantised per token and the
 * SiLU-and-mul intermediate per (token, expert) row, both in MX blocks of
 * 32.  Optional outputs as oracle_forward_fp8, with scale codes
 * sx_out [nrows][H/32] and sh_out [nrows][k][I/32]. */
void oracle_forward_mxfp8(const uint16_t *x, const float *topk_w, const int32_t *ids,
                          const uint8_t *W1, const uint8_t *s1, const uint8_t *W2, const uint8_t *s2,
                          int T, int k, int E, int H, int I, const int32_t *rows, int nrows,
                          double *out, uint8_t *xq_out, uint8_t *sx_out, uint8_t *hq_out,
                          uint8_t *sh_out)
{
    oracle_init();
    if (!rows)
        nrows = T;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; r++) {
        int t = rows ? rows[r] : r;
        token_mxfp8(x, topk_w, ids, W1, s1, W2, s2, t, k, E, H, I, out + (size_t)r * H,
                    xq_out ? xq_out + (size_t)r * H : NULL,
                    sx_out ? sx_out + (size_t)r * (H / 32) : NULL,
                    hq_out ? hq_out + (size_t)r * k * I : NULL,
                    sh_out ? sh_out + (size_t)r * k * (I / 32) : NULL);
    }
}

/*
 * Precision-aware router GEMM (HPC-Ops x SGLang blog, section "Router
 * GEMM", "a precision-aware BF16 formulation"): the router keeps fp32
 * weights W [N][K] while the hidden states x [T][K] are bf16.  W is split
 * once into two bf16 parts:
 *
 *   W_high = W cut to bf16 by truncation (the low 16 bits of the fp32
 *            pattern dropped: rounds toward zero);
 *   W_low  = bf16 of the residual scaled by 256, (W - W_high) * 256, with
 *            round-to-nearest-even (the residual and the scaling are exact
 *            in fp32, so only this rounding loses anything);
 *
 * so that W ~ W_high + W_low / 256, and the scores are two bf16 products
 * combined with the scale in the epilogue:
 *
 *   score[t][n] = sum_k x[t][k] W_high[n][k] + (sum_k x[t][k] W_low[n][k]) / 256.
 *
 * Both sums in fp64 here (bf16 x bf16 products are exact in fp64).
 */

/* bf16 code nearest to a finite fp32 value, ties to the even code, found
 * from the value table: the truncated code and the next code away from
 * zero bracket v. */
static uint16_t bf16_rne(float v)
{
    uint32_t u;
    memcpy(&u, &v, 4);
    const uint16_t c0 = (uint16_t)(u >> 16);
    const uint16_t c1 = (uint16_t)(c0 + 1);
    const double dv = (double)v;
    const double d0 = fabs(dv - BF16_VALUE[c0]);
    const double d1 = fabs(BF16_VALUE[c1] - dv);
    if (d0 < d1)
        return c0;
    if (d1 < d0)
        return c1;
    return (c0 & 1) ? c1 : c0;
}

void oracle_router_split(const float *w, long n, uint16_t *hi, uint16_t *lo)
{
    oracle_init();
    for (long i = 0; i < n; i++) {
        uint32_t u;
        memcpy(&u, &w[i], 4);
        hi[i] = (uint16_t)(u >> 16);                                  /* truncation */
        const float high = (float)BF16_VALUE[hi[i]];
        const float resid = (w[i] - high) * 256.0f;                   /* exact in fp32 */
        lo[i] = bf16_rne(resid);
    }
}

void oracle_router_scores(const uint16_t *x, const uint16_t *hi, const uint16_t *lo, int T, int N,
                          int K, double *out)
{
    oracle_init();
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        const uint16_t *xr = x + (size_t)t * K;
        for (int n = 0; n < N; n++) {
            const uint16_t *hr = hi + (size_t)n * K;
            const uint16_t *lr = lo + (size_t)n * K;
            double s_hi = 0.0, s_lo = 0.0;
            for (int k = 0; k < K; k++) {
                const double xv = BF16_VALUE[xr[k]];
                s_hi += xv * BF16_VALUE[hr[k]];
                s_lo += xv * BF16_VALUE[lr[k]];
            }
            out[(size_t)t * N + n] = s_hi + s_lo / 256.0;
        }
    }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
