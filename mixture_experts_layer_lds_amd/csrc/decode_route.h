// Routing & index build of one decode token inside the first kernel of the
// forward pass (HPC-Ops x SGLang blog, section "MoE": at decode the
// metadata build costs about as much as the expert GEMMs, so it is not left
// as a launch of its own).
//
// One token, k <= 16 pairs, at most one row tile per expert (k no larger
// than the tile height): the counting sort of the routing build reduces to
// comparisons between the k keys, which one wave holds in k lanes.  Every
// workgroup computes it in registers (a few hundred cycles) and takes its
// tasks from there; workgroup 0 also writes the routing buffer, with the
// same bytes as the routing build (the stable order by expert id, dropped
// pairs last in pair order, one task per expert present, the header).
#pragma once

#include "moe_common.h"

namespace moe {

struct DecodeRoute {
  int key;      // lane < k: its pair's expert id, or E when dropped; else -1
  int less;     // pairs with a smaller key: the first sorted row of the key
  int pos;      // the pair's sorted row
  int rows;     // pairs with the same key
  int tidx;     // task of the key's expert (meaningful where `first`)
  bool first;   // first pair, in pair order, of a valid expert
  int ntasks;   // experts present (wave-uniform)
  int nvalid;   // pairs with a valid expert id (wave-uniform)
};

// The token's pairs sorted by one wave (all 64 lanes active).  ids: k
// expert ids; an id outside [0, E) drops its pair.
__device__ __forceinline__ DecodeRoute decode_route(const int32_t* __restrict__ ids, int k, int E,
                                                    int lane) {
  DecodeRoute r;
  const int id = ids[lane < k ? lane : 0];
  r.key = lane < k ? ((id >= 0 && id < E) ? id : E) : -1;
  int less = 0, before = 0, same = 0;
  for (int q = 0; q < k; q++) {
    const int kq = __builtin_amdgcn_readlane(r.key, q);
    less += kq < r.key;
    before += (kq == r.key) & (q < lane);
    same += kq == r.key;
  }
  r.less = less;
  r.pos = less + before;
  r.rows = same;
  r.first = lane < k && r.key < E && before == 0;
  const uint64_t firsts = __ballot(r.first);
  int tidx = 0;
  for (int q = 0; q < k; q++)
    tidx += (int)((firsts >> q) & 1ull) & (__builtin_amdgcn_readlane(r.key, q) < r.key);
  r.tidx = tidx;
  r.ntasks = __popcll(firsts);
  r.nvalid = __popcll(__ballot(lane < k && r.key < E));
  return r;
}

// Task ti (< ntasks) as the routing build writes it, in scalar registers.
__device__ __forceinline__ moe_task_t decode_task(const DecodeRoute& r, int ti) {
  const uint64_t m = __ballot(r.first && r.tidx == ti);
  const int L = __builtin_ctzll(m);
  moe_task_t t;
  t.expert = __builtin_amdgcn_readlane(r.key, L);
  t.row_begin = __builtin_amdgcn_readlane(r.less, L);
  t.rows = __builtin_amdgcn_readlane(r.rows, L);
  t.reserved = 0;
  return t;
}

// The routing buffer's parts, by the nthreads threads of one workgroup
// (each wave having computed r itself).
__device__ __forceinline__ void decode_route_write(const DecodeRoute& r, const moe_host::DecodeRouteOut& o,
                                                   int k, int tid, int nthreads, int lane, int wave) {
  if (tid < 16) {
    int v = 0;
    if (tid == kHdrNumTasks) v = min(r.ntasks, o.max_tasks);
    else if (tid == kHdrNumDropped) v = k - r.nvalid;
    else if (tid == kHdrBlockM) v = o.block_m;
    else if (tid == kHdrNumPairs) v = k;
    else if (tid == kHdrNumExperts) v = o.E;
    else if (tid == kHdrMaxTasks) v = o.max_tasks;
    else if (tid == kHdrMaxExpertTiles) v = r.nvalid > 0 ? 1 : 0;
    o.header[tid] = v;
  }
  // offsets[e] = pairs with a key below e (offsets[E]: the valid pairs)
  int keys[kMaxTopK];
#pragma unroll
  for (int q = 0; q < kMaxTopK; q++) keys[q] = q < k ? __builtin_amdgcn_readlane(r.key, q) : 0x7fffffff;
  for (int e = tid; e <= o.E; e += nthreads) {
    int c = 0;
#pragma unroll
    for (int q = 0; q < kMaxTopK; q++) c += keys[q] < e;
    o.expert_offsets[e] = c;
  }
  if (wave == 0 && lane < k) {
    o.sorted_pairs[r.pos] = lane;
    o.pair_pos[lane] = r.pos;
    if (r.first && r.tidx < o.max_tasks) {
      moe_task_t t;
      t.expert = r.key;
      t.row_begin = r.less;
      t.rows = r.rows;
      t.reserved = 0;
      o.tasks[r.tidx] = t;
    }
  }
}

}  // namespace moe
