// Routing & index build of a decode batch inside the first kernel of the
// forward pass (HPC-Ops x SGLang blog, section "MoE": at decode the metadata
// build costs about as much as the expert GEMMs, so it is not left as a
// launch of its own).
//
// At most 64 token-expert pairs: the counting sort of the routing build
// reduces to comparisons between the P keys, which one wave holds one per
// lane.  Every workgroup computes it in registers (about a hundred
// instructions)
// and takes its tasks from there; workgroup 0 also writes the routing
// buffer, with the same bytes as the routing build: pairs in the stable
// order of their expert id (dropped pairs last, in pair order), each
// expert's range cut into tiles of block_m rows, tasks in expert order, the
// header.
#pragma once

#include "moe_common.h"

namespace moe {

constexpr int kDecodeRoutePairs = kWave;   // pairs one wave sorts

struct DecodeRoute {
  int key;      // lane p < P: pair p's expert id, or E when dropped; else -1
  int less;     // pairs with a smaller key: the first sorted row of the key
  int pos;      // pair p's sorted row
  int count;    // pairs with the same key
  int tiles;    // where `first`: row tiles of the key's expert, else 0
  int tidx;     // where `first`: the expert's first task
  int spair;    // lane r < P: the pair at sorted row r
  int skey;     // lane r < P: the key of sorted row r
  bool first;   // first pair, in pair order, of a valid expert
  int ntasks;   // tasks of all experts (wave-uniform)
  int max_tiles;   // most tiles of one expert (wave-uniform)
  int nvalid;   // pairs with a valid expert id (wave-uniform)
};

// The P (<= 64) pairs sorted by one wave (all 64 lanes active).  ids: P
// expert ids; an id outside [0, E) drops its pair.  The comparisons run bit
// by bit over the nine key bits, most significant first: a lane's class
// (the lanes that agree with it on the bits so far) loses to it the members
// whose current bit is 0 where its own is 1 (they have smaller keys), then
// keeps those with its own bit.  After the last bit the class is the lanes
// of its key.  Counted once over all pairs (the key's first sorted row) and
// once over the first pair of every expert (the expert's place among the
// experts present).
__device__ __forceinline__ DecodeRoute decode_route(const int32_t* __restrict__ ids, int P, int E,
                                                    int block_m, int lane) {
  DecodeRoute r;
  const int id = ids[lane < P ? lane : 0];
  const bool have = lane < P;
  r.key = have ? ((id >= 0 && id < E) ? id : E) : -1;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  uint64_t bits[9];   // lanes whose key has bit b set (keys < 512)
  uint64_t eq = __ballot(have);
  int less = 0;
#pragma unroll
  for (int bit = 8; bit >= 0; bit--) {
    const bool set = (r.key >> bit) & 1;
    bits[bit] = __ballot(have && set);
    less += set ? __popcll(eq & ~bits[bit]) : 0;
    eq &= set ? bits[bit] : ~bits[bit];
  }
  r.less = less;
  r.count = __popcll(eq);
  const int before = __popcll(eq & below);
  r.pos = less + before;
  r.first = have && r.key < E && before == 0;
  const uint64_t firsts = __ballot(r.first);
  uint64_t eqf = firsts;
  int tless = 0;
#pragma unroll
  for (int bit = 8; bit >= 0; bit--) {
    const bool set = (r.key >> bit) & 1;
    tless += set ? __popcll(eqf & ~bits[bit]) : 0;
    eqf &= set ? bits[bit] : ~bits[bit];
  }
  r.tiles = r.first ? (r.count + block_m - 1) / block_m : 0;
  // experts of more than one tile (a hot expert; usually none) add their
  // extra tiles to the experts above them
  int tidx = tless, total = __popcll(firsts), most = firsts ? 1 : 0;
  uint64_t multi = __ballot(r.tiles > 1);
  while (multi) {
    const int q = __builtin_ctzll(multi);
    multi &= multi - 1;
    const int tq = __builtin_amdgcn_readlane(r.tiles, q);
    tidx += __builtin_amdgcn_readlane(r.key, q) < r.key ? tq - 1 : 0;
    total += tq - 1;
    most = max(most, tq);
  }
  r.tidx = tidx;
  r.ntasks = total;
  r.max_tiles = most;
  r.nvalid = __popcll(__ballot(have && r.key < E));
  // the inverse of pos: pair p sends its index and key to lane pos (lanes
  // past P to themselves, which no pair's row names)
  const int dst = 4 * (have ? r.pos : lane);
  r.spair = __builtin_amdgcn_ds_permute(dst, lane);
  r.skey = __builtin_amdgcn_ds_permute(dst, r.key);
  return r;
}

// Task ti (< ntasks) as the routing build writes it, in scalar registers.
__device__ __forceinline__ moe_task_t decode_task(const DecodeRoute& r, int ti, int block_m) {
  const uint64_t m = __ballot(r.tiles > 0 && r.tidx <= ti && ti < r.tidx + r.tiles);
  const int L = __builtin_ctzll(m);
  const int j = ti - __builtin_amdgcn_readlane(r.tidx, L);
  moe_task_t t;
  t.expert = __builtin_amdgcn_readlane(r.key, L);
  t.row_begin = __builtin_amdgcn_readlane(r.less, L) + j * block_m;
  t.rows = min(block_m, __builtin_amdgcn_readlane(r.count, L) - j * block_m);
  t.reserved = 0;
  return t;
}

// The pair at sorted row `row` (< P), to every lane that asks (all lanes
// active).
__device__ __forceinline__ int decode_sorted_pair(const DecodeRoute& r, int row) {
  return __shfl(r.spair, row, kWave);
}

// The routing buffer's parts, by the nthreads threads of one workgroup
// (each wave having computed r itself).
__device__ __forceinline__ void decode_route_write(const DecodeRoute& r, const moe_host::DecodeRouteOut& o,
                                                   int P, int tid, int nthreads, int lane, int wave) {
  if (tid < 16) {
    int v = 0;
    if (tid == kHdrNumTasks) v = min(r.ntasks, o.max_tasks);
    else if (tid == kHdrNumDropped) v = P - r.nvalid;
    else if (tid == kHdrBlockM) v = o.block_m;
    else if (tid == kHdrNumPairs) v = P;
    else if (tid == kHdrNumExperts) v = o.E;
    else if (tid == kHdrMaxTasks) v = o.max_tasks;
    else if (tid == kHdrMaxExpertTiles) v = r.max_tiles;
    o.header[tid] = v;
  }
  // offsets[e] = pairs with a key below e (offsets[E]: the valid pairs): the
  // sorted rows' keys do not decrease, so a binary search over them
  for (int e0 = 0; e0 <= o.E; e0 += nthreads) {
    const int e = e0 + tid;
    int c = 0;
#pragma unroll
    for (int step = kWave; step >= 1; step >>= 1) {
      const int kk = __shfl(r.skey, min(c + step, kWave) - 1, kWave);
      if (c + step <= P && kk < e) c += step;
    }
    if (e <= o.E) o.expert_offsets[e] = c;
  }
  if (wave == 0 && lane < P) {
    o.sorted_pairs[r.pos] = lane;
    o.pair_pos[lane] = r.pos;
    for (int j = 0; j < r.tiles; j++) {
      if (r.tidx + j >= o.max_tasks) break;
      moe_task_t t;
      t.expert = r.key;
      t.row_begin = r.less + j * o.block_m;
      t.rows = min(o.block_m, r.count - j * o.block_m);
      t.reserved = 0;
      o.tasks[r.tidx + j] = t;
    }
  }
}

}  // namespace moe
