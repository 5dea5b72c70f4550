// Router top-k (HPC-Ops x SGLang blog, section "Router GEMM: balancing
// routing precision and throughput": the router's fp32 expert scores feed a
// top-k choice that decides which experts run, and a small score change can
// flip the k-th choice, so the choice here is exact; SGLang fused-MoE tuning
// guide, model-config section: shared experts fused into the expert tensor
// as extra expert ids).
//
// For every token: softmax over the E scores, the k largest (descending,
// equal scores by ascending expert id), optionally renormalised over the
// k, then n_shared shared-expert columns (ids E, E+1, ... with weight 1).
// The output is the topk_ids / topk_w pair that the routing build and the
// forward pass take.
//
// Mapping: a group of L lanes of one wave serves one token (L a power of
// two with 4L >= E); lane s of the group keeps logits 4s .. 4s+3 in
// registers, read once.  Softmax is strictly increasing, so the ranking is
// made on the logits themselves, bit-exactly.  Round j: every lane offers
// its largest live logit (the lowest id among its equal ones); a butterfly
// max over the group gives the round's value; a ballot picks the lowest
// lane offering it, whose expert then has the lowest id among the equal
// values; that lane retires the logit.  The weights come last, in fp32:
// exp(s_j - s_0) over the sum of the k terms (renormalised) or over the
// sum of all E terms.
#include "moe_common.h"

namespace moe {

constexpr int kRouterThreads = 256;
constexpr int kRouterMaxExperts = 4 * kWave;   // 4 logits per lane, one wave per token

template <int L>
__global__ void __launch_bounds__(kRouterThreads)
router_topk_kernel(const float* __restrict__ logits, int T, int E, int k, int renorm,
                   int n_shared, int vec, int32_t* __restrict__ ids, float* __restrict__ w) {
  constexpr int kSlots = (kMaxTopK + L - 1) / L;   // selected entries kept per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int sl = lane & (L - 1);
  const long t = (long)blockIdx.x * (kRouterThreads / L) + threadIdx.x / L;
  if (t >= T) return;   // whole groups leave together: no later exchange reads them
  const uint64_t gmask = L == kWave ? ~0ull : ((1ull << L) - 1) << (lane & ~(L - 1));

  const float* row = logits + t * E;
  const int e0 = 4 * sl;
  float v[4];
  if (vec) {   // E % 4 == 0 and 16-byte aligned rows
    float4 q = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    if (e0 < E) q = *reinterpret_cast<const float4*>(row + e0);
    v[0] = q.x, v[1] = q.y, v[2] = q.z, v[3] = q.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = e0 + i < E ? row[e0 + i] : -INFINITY;
  }
  unsigned live = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    if (e0 + i < E) live |= 1u << i;
    if (__builtin_isnan(v[i])) v[i] = -INFINITY;   // NaN ranks as -infinity
  }
  const unsigned valid = live;

  float s0 = 0.f, sel_sum = 0.f;
  float my_s[kSlots];
  int my_e[kSlots];
#pragma unroll
  for (int q = 0; q < kSlots; q++) my_s[q] = 0.f, my_e[q] = 0;
#pragma unroll
  for (int j = 0; j < kMaxTopK; j++) {
    if (j >= k) continue;   // k is the same for every lane; the loop unrolls fully
    float bv = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < 4; i++)
      if (((live >> i) & 1u) && (bi < 0 || v[i] > bv)) bv = v[i], bi = i;
    float m = bv;
#pragma unroll
    for (int o = L / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, L));
    // k <= E leaves a live logit in the group, so the ballot is never empty
    const uint64_t cand = __ballot(bi >= 0 && bv == m) & gmask;
    const int wl = __builtin_ctzll(cand);
    const int e = __shfl(e0 + bi, wl, kWave);
    if (lane == wl) live &= ~(1u << bi);
    if (j == 0) s0 = m;
    sel_sum += expf(m - s0);
    if (sl == j % L) my_s[j / L] = m, my_e[j / L] = e;
  }

  float denom = sel_sum;
  if (!renorm) {
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++)
      if ((valid >> i) & 1u) part += expf(v[i] - s0);
#pragma unroll
    for (int o = L / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, L);
    denom = part;
  }
  const int ncol = k + n_shared;
  int32_t* orow_ids = ids + t * ncol;
  float* orow_w = w + t * ncol;
#pragma unroll
  for (int q = 0; q < kSlots; q++) {
    const int j = q * L + sl;
    if (j < k) {
      orow_ids[j] = my_e[q];
      orow_w[j] = expf(my_s[q] - s0) / denom;
    }
  }
  for (int s = sl; s < n_shared; s += L) {
    orow_ids[k + s] = E + s;
    orow_w[k + s] = 1.f;
  }
}

}  // namespace moe

namespace moe_host {

int router_max_experts() { return moe::kRouterMaxExperts; }

hipError_t launch_router_topk(const float* logits, int T, int E, int k, int renorm, int n_shared,
                              int32_t* ids, float* w, hipStream_t s) {
  int L = 1;
  while (4 * L < E) L *= 2;
  const int vec = (E % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0) ? 1 : 0;
  const long per_block = moe::kRouterThreads / L;
  const dim3 grid((unsigned)((T + per_block - 1) / per_block));
  const dim3 block(moe::kRouterThreads);
#define MOE_ROUTER_CASE(LL)                                                                  \
  case LL:                                                                                   \
    hipLaunchKernelGGL(moe::router_topk_kernel<LL>, grid, block, 0, s, logits, T, E, k, renorm, \
                       n_shared, vec, ids, w);                                               \
    break;
  switch (L) {
    MOE_ROUTER_CASE(1)
    MOE_ROUTER_CASE(2)
    MOE_ROUTER_CASE(4)
    MOE_ROUTER_CASE(8)
    MOE_ROUTER_CASE(16)
    MOE_ROUTER_CASE(32)
    MOE_ROUTER_CASE(64)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_ROUTER_CASE
  return hipGetLastError();
}

}  // namespace moe_host
