// Routing & index build (HPC-Ops x SGLang blog, section "MoE", routing &
// index build): from the top-k expert ids, a counting pass in on-chip
// memory groups the token-expert pairs into contiguous per-expert ranges,
// builds the route index and cuts each range into row tiles for the
// grouped GEMMs.
//
// One workgroup of 1024 threads does the whole build in LDS; global memory
// sees only the id reads and the output writes (no global atomics).  The
// order inside an expert's range is the ascending pair index, which makes
// the result a deterministic function of the ids:
//
//  A. each of the 16 waves owns one contiguous segment of pairs and walks
//     it 64 pairs at a time; the rank of a pair among the earlier lanes
//     holding the same key (expert id, or E for a dropped pair) comes from
//     nine ballots over the key bits and a popcount, and the wave's own LDS
//     counter row for that key (read by every lane of the key group, then
//     advanced by its first lane) turns it into the pair's rank inside the
//     segment.  No barrier is needed: a wave only touches its own row;
//  B. one thread per key turns the 16 segment counts into segment bases
//     (a prefix over waves) and the key total; one wave scans the totals
//     into the start row of every key;
//  C. every wave re-walks its segment: row = start[key] + base[wave][key] +
//     rank, so pair p lands after every earlier pair of its key;
//  D. per-expert tile counts ceil(c_e / block_m), scanned to task offsets;
//     one thread per expert writes its tiles.
#include "moe_common.h"

namespace moe {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kKeys = kMaxExperts + 1;   // expert ids plus the dropped bucket
constexpr int kBatch = 8;                // 64-pair steps whose loads are issued together

// Largest of in[0..n) (n >= 0; 0 when empty) by one wave, returned to every lane.
__device__ int wave_max_tiles(const int* in, int n, int lane) {
  int m = 0;
  for (int i = lane; i < n; i += kWave) m = max(m, in[i]);
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) m = max(m, __shfl_xor(m, o, kWave));
  return m;
}

// Exclusive prefix sum of in[0..n) into out[0..n) by one wave (n <= 64*64);
// in and out may alias.  Returns the total to every lane.
__device__ int wave_exclusive_scan(const int* in, int* out, int n, int lane) {
  const int per = (n + kWave - 1) / kWave;
  const int b = lane * per;
  const int e = min(b + per, n);
  int s = 0;
  for (int i = b; i < e; i++) s += in[i];
  int incl = s;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  int run = incl - s;
  for (int i = b; i < e; i++) {
    int v = in[i];
    out[i] = run;
    run += v;
  }
  return __shfl(incl, kWave - 1, kWave);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its global stores (a fenced __syncthreads() would wait
// out the store latency at every phase).  Global memory is never used to
// pass data between threads of this kernel: each thread reads back only its
// own writes.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

__global__ void __launch_bounds__(kRouteThreads)
route_kernel(const int32_t* __restrict__ ids, int P, int E, int block_m, int max_tasks,
             int32_t* __restrict__ header, int32_t* __restrict__ expert_offsets,
             int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos,
             moe_task_t* __restrict__ tasks) {
  __shared__ int s_count[kKeys];
  __shared__ int s_start[kKeys + 1];
  __shared__ int s_wcount[kRouteWaves][kKeys];
  __shared__ int s_task0[kKeys];
  __shared__ int s_total_tasks, s_max_tiles;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int nkeys = E + 1;

  for (int kk = lane; kk < nkeys; kk += kWave) s_wcount[wave][kk] = 0;   // a wave's own row
  lds_barrier();

  // segment of this wave: a multiple of 64 pairs
  const int seg = ((P + kRouteWaves - 1) / kRouteWaves + kWave - 1) / kWave * kWave;
  const int p0 = min(P, wave * seg), p1 = min(P, p0 + seg);
  const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int* wrow = s_wcount[wave];

  // A. ranks inside the segment.  A segment holds at most kBatch 64-pair
  // steps (P <= kOneGroupPairs), so one batch of loads covers it, and the
  // keys and ranks stay in registers until phase C.
  // Unconditional loads of a clamped index (p1 - 1 >= 0 as P >= 1): a load
  // under a branch gets its own wait, which would serialise the batch.
  // Waves and 64-pair steps past the pairs skip the work (wave-uniform tests).
  int keys[kBatch], ranks[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; u++) keys[u] = -1;
  if (p0 < p1) {
#pragma unroll
    for (int u = 0; u < kBatch; u++) keys[u] = ids[min(p0 + u * kWave + lane, p1 - 1)];
#pragma unroll
    for (int u = 0; u < kBatch; u++) {
      const int p = p0 + u * kWave + lane;
      const int e = keys[u];
      keys[u] = p < p1 ? ((e >= 0 && e < E) ? e : E) : -1;   // -1: beyond the segment
    }
  }
#pragma unroll
  for (int u = 0; u < kBatch; u++) {
    ranks[u] = 0;
    if (p0 + u * kWave >= p1) continue;
    const int key = keys[u];
    const bool have = key >= 0;
    uint64_t same = __ballot(have);
#pragma unroll
    for (int bit = 0; bit < 9; bit++) {   // keys < 512
      const bool set = (key >> bit) & 1;
      const uint64_t m = __ballot(have && set);
      same &= set ? m : ~m;
    }
    const int below = __popcll(same & lanes_below);
    int before = 0;
    if (have) before = wrow[key];
    __builtin_amdgcn_wave_barrier();      // every lane has read the counter ...
    if (have && below == 0) wrow[key] = before + __popcll(same);   // ... before its first lane advances it
    __builtin_amdgcn_wave_barrier();
    ranks[u] = before + below;
  }
  lds_barrier();

  // B. per-key totals and per-wave segment bases
  for (int kk = tid; kk < nkeys; kk += kRouteThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kRouteWaves; w++) {
      const int c = s_wcount[w][kk];
      s_wcount[w][kk] = run;
      run += c;
    }
    s_count[kk] = run;
  }
  lds_barrier();
  if (wave == 0) wave_exclusive_scan(s_count, s_start, nkeys, lane);
  lds_barrier();
  for (int i = tid; i < nkeys; i += kRouteThreads) {
    if (i < E) s_task0[i] = (s_count[i] + block_m - 1) / block_m;
    expert_offsets[i] = s_start[i];   // key E: number of valid pairs
  }

  // C. scatter
#pragma unroll
  for (int u = 0; u < kBatch; u++) {
    const int p = p0 + u * kWave + lane;
    if (p0 + u * kWave < p1 && keys[u] >= 0) {
      const int r = s_start[keys[u]] + wrow[keys[u]] + ranks[u];
      sorted_pairs[r] = p;
      pair_pos[p] = r;
    }
  }
  lds_barrier();

  // D. task map
  if (wave == 0) {
    const int most = wave_max_tiles(s_task0, E, lane);
    const int total = wave_exclusive_scan(s_task0, s_task0, E, lane);
    if (lane == 0) {
      s_total_tasks = total;
      s_max_tiles = most;
    }
  }
  lds_barrier();
  for (int e = tid; e < E; e += kRouteThreads) {
    const int c = s_count[e];
    int t = s_task0[e];
    for (int m0 = 0; m0 < c && t < max_tasks; m0 += block_m, t++) {
      moe_task_t task;
      task.expert = e;
      task.row_begin = s_start[e] + m0;
      task.rows = min(block_m, c - m0);
      task.reserved = 0;
      tasks[t] = task;
    }
  }
  if (tid < 16) {
    int v = 0;
    if (tid == kHdrNumTasks) v = min(s_total_tasks, max_tasks);
    else if (tid == kHdrNumDropped) v = P - s_start[E];
    else if (tid == kHdrBlockM) v = block_m;
    else if (tid == kHdrNumPairs) v = P;
    else if (tid == kHdrNumExperts) v = E;
    else if (tid == kHdrMaxTasks) v = max_tasks;
    else if (tid == kHdrMaxExpertTiles) v = s_max_tiles;
    header[tid] = v;
  }
}

// ---------------------------------------------------------------------------
// Many pairs (P > kOneGroupPairs): the same stable counting sort spread over
// many workgroups in three launches, so that the scattered writes of the
// route index are not funnelled through one compute unit.
//   count:   one 4-wave workgroup per segment of kSegPairs consecutive pairs:
//            in-wave ranks as in phase A above, then per-wave bases inside the
//            segment; writes each pair's rank inside its segment (into
//            pair_pos) and the segment's per-key counts;
//   scan:    one workgroup: per key, a prefix over segments (segment bases)
//            and the key totals; expert offsets, task map and header as in
//            phases B and D above;
//   scatter: one workgroup per segment: row = base[segment][key] + rank.
constexpr int kOneGroupPairs = 4096;
static_assert(kOneGroupPairs <= kRouteWaves * kWave * kBatch,
              "the one-workgroup build holds each wave's segment in one batch of registers");
constexpr int kSegThreads = 256;
constexpr int kSegWaves = kSegThreads / kWave;                 // 4
constexpr int kSegPairs = kSegWaves * kWave * kBatch;          // 2048: one batch per wave
constexpr int kMaxSegs = kMaxPairs / kSegPairs;                // 32

__global__ void __launch_bounds__(kSegThreads)
route_count_kernel(const int32_t* __restrict__ ids, int P, int E, int32_t* __restrict__ seg_counts,
                   int32_t* __restrict__ pair_pos) {
  __shared__ int s_w[kSegWaves][kKeys];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int nkeys = E + 1;
  for (int kk = lane; kk < nkeys; kk += kWave) s_w[wave][kk] = 0;   // a wave's own row
  lds_barrier();
  const int p0 = blockIdx.x * kSegPairs + wave * kWave * kBatch;
  const int pend = min(P, (int)(blockIdx.x + 1) * kSegPairs);
  const int p1 = min(pend, p0 + kWave * kBatch);
  const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int* wrow = s_w[wave];
  int keys[kBatch], ranks[kBatch];
  if (p0 < p1) {
    int raw[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; u++) raw[u] = ids[min(p0 + u * kWave + lane, p1 - 1)];
#pragma unroll
    for (int u = 0; u < kBatch; u++) {
      const int p = p0 + u * kWave + lane;
      const int e = raw[u];
      keys[u] = p < p1 ? ((e >= 0 && e < E) ? e : E) : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatch; u++) {
      const int key = keys[u];
      const bool have = key >= 0;
      uint64_t same = __ballot(have);
#pragma unroll
      for (int bit = 0; bit < 9; bit++) {
        const bool set = (key >> bit) & 1;
        const uint64_t m = __ballot(have && set);
        same &= set ? m : ~m;
      }
      const int below = __popcll(same & lanes_below);
      int before = 0;
      if (have) before = wrow[key];
      __builtin_amdgcn_wave_barrier();
      if (have && below == 0) wrow[key] = before + __popcll(same);
      __builtin_amdgcn_wave_barrier();
      ranks[u] = before + below;
    }
  }
  lds_barrier();
  // per-wave bases inside the segment, segment counts
  for (int kk = tid; kk < nkeys; kk += kSegThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kSegWaves; w++) {
      const int c = s_w[w][kk];
      s_w[w][kk] = run;
      run += c;
    }
    seg_counts[blockIdx.x * kKeys + kk] = run;
  }
  lds_barrier();
  if (p0 < p1) {
#pragma unroll
    for (int u = 0; u < kBatch; u++) {
      const int p = p0 + u * kWave + lane;
      if (keys[u] >= 0) pair_pos[p] = wrow[keys[u]] + ranks[u];
    }
  }
}

__global__ void __launch_bounds__(kRouteThreads)
route_scan_kernel(int P, int E, int block_m, int max_tasks, int32_t* __restrict__ seg_counts,
                  int32_t* __restrict__ header, int32_t* __restrict__ expert_offsets,
                  moe_task_t* __restrict__ tasks) {
  __shared__ int s_count[kKeys];
  __shared__ int s_start[kKeys + 1];
  __shared__ int s_task0[kKeys];
  __shared__ int s_total_tasks, s_max_tiles;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int nkeys = E + 1;
  const int nseg = (P + kSegPairs - 1) / kSegPairs;
  int bases[kMaxSegs];
  if (tid < nkeys) {
    int c[kMaxSegs];
#pragma unroll
    for (int sgi = 0; sgi < kMaxSegs; sgi++) c[sgi] = seg_counts[min(sgi, nseg - 1) * kKeys + tid];
    int run = 0;
#pragma unroll
    for (int sgi = 0; sgi < kMaxSegs; sgi++) {
      bases[sgi] = run;
      if (sgi < nseg) run += c[sgi];
    }
    s_count[tid] = run;
  }
  lds_barrier();
  if (wave == 0) wave_exclusive_scan(s_count, s_start, nkeys, lane);
  lds_barrier();
  if (tid < nkeys) {
    const int st = s_start[tid];
#pragma unroll
    for (int sgi = 0; sgi < kMaxSegs; sgi++)
      if (sgi < nseg) seg_counts[sgi * kKeys + tid] = st + bases[sgi];
    if (tid < E) s_task0[tid] = (s_count[tid] + block_m - 1) / block_m;
    expert_offsets[tid] = st;
  }
  lds_barrier();
  if (wave == 0) {
    const int most = wave_max_tiles(s_task0, E, lane);
    const int total = wave_exclusive_scan(s_task0, s_task0, E, lane);
    if (lane == 0) {
      s_total_tasks = total;
      s_max_tiles = most;
    }
  }
  lds_barrier();
  for (int e = tid; e < E; e += kRouteThreads) {
    const int c = s_count[e];
    int t = s_task0[e];
    for (int m0 = 0; m0 < c && t < max_tasks; m0 += block_m, t++) {
      moe_task_t task;
      task.expert = e;
      task.row_begin = s_start[e] + m0;
      task.rows = min(block_m, c - m0);
      task.reserved = 0;
      tasks[t] = task;
    }
  }
  if (tid < 16) {
    int v = 0;
    if (tid == kHdrNumTasks) v = min(s_total_tasks, max_tasks);
    else if (tid == kHdrNumDropped) v = P - s_start[E];
    else if (tid == kHdrBlockM) v = block_m;
    else if (tid == kHdrNumPairs) v = P;
    else if (tid == kHdrNumExperts) v = E;
    else if (tid == kHdrMaxTasks) v = max_tasks;
    else if (tid == kHdrMaxExpertTiles) v = s_max_tiles;
    header[tid] = v;
  }
}

__global__ void __launch_bounds__(kSegThreads)
route_scatter_kernel(const int32_t* __restrict__ ids, int P, int E,
                     const int32_t* __restrict__ seg_base, int32_t* __restrict__ sorted_pairs,
                     int32_t* __restrict__ pair_pos) {
  const int tid = threadIdx.x;
  const int p0 = blockIdx.x * kSegPairs;
  const int p1 = min(P, p0 + kSegPairs);
  int raw[kBatch], rk[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; u++) {
    const int pc = min(p0 + u * kSegThreads + tid, p1 - 1);
    raw[u] = ids[pc];
    rk[u] = pair_pos[pc];
  }
  int keys[kBatch], base[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; u++) {
    const int e = raw[u];
    keys[u] = (e >= 0 && e < E) ? e : E;
    base[u] = seg_base[blockIdx.x * kKeys + keys[u]];
  }
#pragma unroll
  for (int u = 0; u < kBatch; u++) {
    const int p = p0 + u * kSegThreads + tid;
    if (p < p1) {
      const int r = base[u] + rk[u];
      sorted_pairs[r] = p;
      pair_pos[p] = r;
    }
  }
}

}  // namespace moe

namespace moe_host {

hipError_t launch_route(const int32_t* ids, int P, int E, int block_m, int max_tasks,
                        void* routing, const moe_routing_layout_t& L, hipStream_t s) {
  char* base = static_cast<char*>(routing);
  int32_t* header = reinterpret_cast<int32_t*>(base + L.header);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.expert_offsets);
  int32_t* sorted = reinterpret_cast<int32_t*>(base + L.sorted_pairs);
  int32_t* pos = reinterpret_cast<int32_t*>(base + L.pair_pos);
  moe_task_t* tasks = reinterpret_cast<moe_task_t*>(base + L.tasks);
  if (P <= moe::kOneGroupPairs) {
    hipLaunchKernelGGL(moe::route_kernel, dim3(1), dim3(moe::kRouteThreads), 0, s, ids, P, E,
                       block_m, max_tasks, header, offsets, sorted, pos, tasks);
    return hipGetLastError();
  }
  int32_t* seg = reinterpret_cast<int32_t*>(base + L.scratch);
  const int nseg = (P + moe::kSegPairs - 1) / moe::kSegPairs;
  hipLaunchKernelGGL(moe::route_count_kernel, dim3(nseg), dim3(moe::kSegThreads), 0, s, ids, P, E,
                     seg, pos);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moe::route_scan_kernel, dim3(1), dim3(moe::kRouteThreads), 0, s, P, E, block_m,
                     max_tasks, seg, header, offsets, tasks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moe::route_scatter_kernel, dim3(nseg), dim3(moe::kSegThreads), 0, s, ids, P, E,
                     seg, sorted, pos);
  return hipGetLastError();
}

size_t route_scratch_bytes(int P) {
  return P <= moe::kOneGroupPairs ? 0
                                  : (size_t)((P + moe::kSegPairs - 1) / moe::kSegPairs) * moe::kKeys * 4;
}

}  // namespace moe_host
