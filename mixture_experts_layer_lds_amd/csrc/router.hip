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
// made on the logits themselves, bit-exactly, as order-preserving 32-bit
// keys (equal floats, +0 and -0 included, give equal keys; NaN takes the
// key of -infinity).  Round j: every lane offers its largest live key; the
// group maximum comes from DPP lane permutations inside each 16-lane row
// (quad swaps, half-row and row mirrors) and, for groups of 32 or 64
// lanes, a read of each row's result into scalar registers.  Three ballots
// (equal to the maximum; and the two bits of the offering lane's slot)
// name the lowest offering lane and its slot, which is the lowest expert
// id among the equal keys; that lane retires the logit.  No exchange goes
// through the LDS crossbar, which keeps the round's dependency chain short
// (decode batches are latency-bound).  The weights come last, in fp32:
// exp(s_j - s_0) over the sum of the k terms (renormalised) or over the
// sum of all E terms, both sums reduced with the same permutations so that
// every lane of a group holds the same bits.
#include "moe_common.h"

namespace moe {

constexpr int kRouterThreads = 256;
constexpr int kRouterMaxExperts = 4 * kWave;   // 4 logits per lane, one wave per token

// Order-preserving key of an fp32 score: a > b as floats <=> key(a) > key(b).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  if ((b & 0x7fffffffu) > 0x7f800000u) b = 0xff800000u;   // NaN ranks as -infinity
  if (b == 0x80000000u) b = 0u;                           // -0 ranks with +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within 16

// Maximum over each group of L lanes, returned to every lane of the group.
template <int L>
__device__ __forceinline__ uint32_t group_max(uint32_t v, int lane) {
  if constexpr (L >= 2) v = max(v, dpp_u<kDppXor1>(v));
  if constexpr (L >= 4) v = max(v, dpp_u<kDppXor2>(v));
  if constexpr (L >= 8) v = max(v, dpp_u<kDppHalfMirror>(v));
  if constexpr (L >= 16) v = max(v, dpp_u<kDppMirror>(v));
  if constexpr (L >= 32) {
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    if constexpr (L == 64) v = max(max(r0, r1), max(r2, r3));
    else v = lane < 32 ? max(r0, r1) : max(r2, r3);
  }
  return v;
}

// Sum over each group of L lanes; every lane of the group gets the same bits.
template <int L>
__device__ __forceinline__ float group_sum(float v, int lane) {
  if constexpr (L >= 2) v += dpp_f<kDppXor1>(v);
  if constexpr (L >= 4) v += dpp_f<kDppXor2>(v);
  if constexpr (L >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (L >= 16) v += dpp_f<kDppMirror>(v);
  if constexpr (L >= 32) {
    auto rd = [](float x, int l) __attribute__((always_inline)) {
      return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
    };
    const float r0 = rd(v, 0), r1 = rd(v, 16), r2 = rd(v, 32), r3 = rd(v, 48);
    if constexpr (L == 64) v = (r0 + r1) + (r2 + r3);
    else v = lane < 32 ? r0 + r1 : r2 + r3;
  }
  return v;
}

template <int L>
__global__ void __launch_bounds__(kRouterThreads)
router_topk_kernel(const float* __restrict__ logits, int S, long slice_stride,
                   float* __restrict__ logits_out, int T, int E, int k, int renorm, int n_shared,
                   int vec, int32_t* __restrict__ ids, float* __restrict__ w) {
  constexpr int kSlots = (kMaxTopK + L - 1) / L;   // selected entries kept per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int sl = lane & (L - 1);
  const int base = lane & ~(L - 1);
  const long t = (long)blockIdx.x * (kRouterThreads / L) + threadIdx.x / L;
  // Groups past the last token run on the last token's row and store
  // nothing, so every lane takes part in every exchange.
  const bool active = t < T;
  const float* row = logits + (active ? t : T - 1) * (long)E;
  const int e0 = 4 * sl;
  // S planes of partial scores (the router GEMM's K slices) are added in
  // ascending plane order as they are loaded; S = 1 is a plain logits row.
  float v[4];
  if (vec) {   // E % 4 == 0 and 16-byte aligned rows
    float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
    if (e0 < E) {
      q = *reinterpret_cast<const float4*>(row + e0);
      for (int p = 1; p < S; p++) {
        const float4 r = *reinterpret_cast<const float4*>(row + p * slice_stride + e0);
        q.x += r.x, q.y += r.y, q.z += r.z, q.w += r.w;
      }
    }
    v[0] = q.x, v[1] = q.y, v[2] = q.z, v[3] = q.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[i] = 0.f;
      if (e0 + i < E) {
        v[i] = row[e0 + i];
        for (int p = 1; p < S; p++) v[i] += row[p * slice_stride + e0 + i];
      }
    }
  }
  if (logits_out && active) {
#pragma unroll
    for (int i = 0; i < 4; i++)
      if (e0 + i < E) logits_out[t * E + e0 + i] = v[i];
  }
  // Keys of the lane's 4 slots (0 for slots past E: every real key is
  // above 0), sorted once into descending order, equal keys by ascending
  // slot; a round then offers key[0] and the winner shifts its list.
  uint32_t key[4], key0[4];
  int slot[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    key0[i] = e0 + i < E ? order_key(v[i]) : 0u;
    key[i] = key0[i];
    slot[i] = i;
  }
  // Compare-exchange on (key, then lower slot first): a total order, so the
  // 4-input network sorts to the unique order whatever the ties.
  auto cas = [&](int a, int b) __attribute__((always_inline)) {   // a < b
    if (key[b] > key[a] || (key[b] == key[a] && slot[b] < slot[a])) {
      const uint32_t tk = key[a];
      key[a] = key[b], key[b] = tk;
      const int ts = slot[a];
      slot[a] = slot[b], slot[b] = ts;
    }
  };
  cas(0, 1), cas(2, 3), cas(0, 2), cas(1, 3), cas(1, 2);

  uint32_t my_key[kSlots];
  int my_e[kSlots];
#pragma unroll
  for (int q = 0; q < kSlots; q++) my_key[q] = 0u, my_e[q] = 0;
  uint32_t top = 0u;
#pragma unroll
  for (int j = 0; j < kMaxTopK; j++) {
    if (j >= k) continue;   // k is the same for every lane; the loop unrolls fully
    const uint32_t m = group_max<L>(key[0], lane);
    // k <= E leaves a live key in every group, so each group has an offer == m
    const bool offer = key[0] == m;
    const uint64_t eq = __ballot(offer);
    const uint64_t b0 = __ballot(offer && (slot[0] & 1));
    const uint64_t b1 = __ballot(offer && (slot[0] & 2));
    int wl, wbi;
    if constexpr (L == kWave) {
      wl = __builtin_ctzll(eq);
      wbi = (int)((b0 >> wl) & 1u) | ((int)((b1 >> wl) & 1u) << 1);
    } else {
      const uint32_t geq = (uint32_t)(eq >> base) & (uint32_t)((1ull << L) - 1);
      wl = __builtin_ctz(geq);
      const int at = base + wl;
      wbi = (int)((b0 >> at) & 1u) | ((int)((b1 >> at) & 1u) << 1);
    }
    if (sl == wl) {
      key[0] = key[1], key[1] = key[2], key[2] = key[3], key[3] = 0u;
      slot[0] = slot[1], slot[1] = slot[2], slot[2] = slot[3];
    }
    if (j == 0) top = m;
    if (sl == j % L) my_key[j / L] = m, my_e[j / L] = 4 * wl + wbi;
  }

  const float s0 = key_value(top);
  float terms[kSlots];
  float part = 0.f;
#pragma unroll
  for (int q = 0; q < kSlots; q++) {
    terms[q] = 0.f;
    if (q * L + sl < k) terms[q] = expf(key_value(my_key[q]) - s0);
    part += terms[q];
  }
  if (!renorm) {   // denominator over all E experts instead of the k selected
    part = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++)
      if (e0 + i < E) part += expf(key_value(key0[i]) - s0);
  }
  const float denom = group_sum<L>(part, lane);
  if (!active) return;
  const int ncol = k + n_shared;
  int32_t* orow_ids = ids + t * ncol;
  float* orow_w = w + t * ncol;
#pragma unroll
  for (int q = 0; q < kSlots; q++) {
    const int j = q * L + sl;
    if (j < k) {
      orow_ids[j] = my_e[q];
      orow_w[j] = terms[q] / denom;
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

hipError_t launch_router_topk(const float* logits, int S, float* logits_out, int T, int E, int k,
                              int renorm, int n_shared, int32_t* ids, float* w, hipStream_t s) {
  int L = 1;
  while (4 * L < E) L *= 2;
  const int vec = (E % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0) ? 1 : 0;
  const long per_block = moe::kRouterThreads / L;
  const dim3 grid((unsigned)((T + per_block - 1) / per_block));
  const dim3 block(moe::kRouterThreads);
#define MOE_ROUTER_CASE(LL)                                                                  \
  case LL:                                                                                   \
    hipLaunchKernelGGL(moe::router_topk_kernel<LL>, grid, block, 0, s, logits, S, (long)T * E,   \
                       logits_out, T, E, k, renorm, n_shared, vec, ids, w);                    \
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
