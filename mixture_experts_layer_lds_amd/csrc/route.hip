// Routing & index build (HPC-Ops x SGLang blog, section "MoE", routing &
// index build): from the top-k expert ids, a counting pass in on-chip
// memory groups the token-expert pairs into contiguous per-expert ranges,
// builds the route index and cuts each range into row tiles for the
// grouped GEMMs.
//
// One workgroup of 1024 threads does the whole build in LDS; global memory
// sees only the id reads and one write per output word (no global
// atomics).  The order inside an expert's range is the ascending pair
// index, which makes the result a deterministic function of the ids:
//
//  1. histogram of keys (expert id, or E for a dropped pair) with LDS atomics
//     -- counts are order independent;
//  2. exclusive scan of the counts -> the start row of every key;
//  3. rounds of 1024 consecutive pairs: inside a wave, the rank of a pair
//     among the earlier lanes holding the same key comes from nine ballots
//     over the key bits and a popcount; per-(wave, key) counts in LDS are
//     turned into per-wave base rows by one thread per key, in wave order,
//     so pair p lands at base[wave][key] + rank, after every earlier pair of
//     its key;
//  4. per-expert tile counts ceil(c_e / block_m), scanned to task offsets;
//     one thread per expert writes its tiles.
#include "moe_common.h"

namespace moe {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kKeys = kMaxExperts + 1;   // expert ids plus the dropped bucket

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

__global__ void __launch_bounds__(kRouteThreads)
route_kernel(const int32_t* __restrict__ ids, int P, int E, int block_m, int max_tasks,
             int32_t* __restrict__ header, int32_t* __restrict__ expert_offsets,
             int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos,
             moe_task_t* __restrict__ tasks) {
  __shared__ int s_count[kKeys];
  __shared__ int s_start[kKeys + 1];
  __shared__ int s_cursor[kKeys];
  __shared__ int s_wcount[kRouteWaves][kKeys];
  __shared__ int s_wbase[kRouteWaves][kKeys];
  __shared__ int s_task0[kKeys];
  __shared__ int s_total_tasks;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int nkeys = E + 1;

  for (int i = tid; i < kKeys; i += kRouteThreads) s_count[i] = 0;
  for (int i = tid; i < kRouteWaves * kKeys; i += kRouteThreads) (&s_wcount[0][0])[i] = 0;
  __syncthreads();

  // 1. histogram
  for (int p = tid; p < P; p += kRouteThreads) {
    const int e = ids[p];
    const int key = (e >= 0 && e < E) ? e : E;
    atomicAdd(&s_count[key], 1);
  }
  __syncthreads();

  // 2. start row of every key
  if (wave == 0) {
    wave_exclusive_scan(s_count, s_start, nkeys, lane);
  }
  __syncthreads();
  for (int i = tid; i < nkeys; i += kRouteThreads) {
    s_cursor[i] = s_start[i];
    if (i < E) s_task0[i] = (s_count[i] + block_m - 1) / block_m;
    expert_offsets[i] = s_start[i];   // key E: number of valid pairs
  }
  __syncthreads();

  // 3. stable scatter, 1024 pairs per round
  const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int base = 0; base < P; base += kRouteThreads) {
    const int p = base + tid;
    const bool have = p < P;
    int key = 0;
    if (have) {
      const int e = ids[p];
      key = (e >= 0 && e < E) ? e : E;
    }
    uint64_t same = __ballot(have);
#pragma unroll
    for (int bit = 0; bit < 9; bit++) {   // keys < 512
      const bool set = (key >> bit) & 1;
      const uint64_t m = __ballot(have && set);
      same &= set ? m : ~m;
    }
    const int rank = __popcll(same & lanes_below);
    if (have && rank == 0) s_wcount[wave][key] = __popcll(same);
    __syncthreads();
    for (int kk = tid; kk < nkeys; kk += kRouteThreads) {
      int run = s_cursor[kk];
#pragma unroll
      for (int w = 0; w < kRouteWaves; w++) {
        const int c = s_wcount[w][kk];
        s_wbase[w][kk] = run;
        s_wcount[w][kk] = 0;
        run += c;
      }
      s_cursor[kk] = run;
    }
    __syncthreads();
    if (have) {
      const int r = s_wbase[wave][key] + rank;
      sorted_pairs[r] = p;
      pair_pos[p] = r;
    }
  }

  // 4. task map
  if (wave == 0) {
    const int total = wave_exclusive_scan(s_task0, s_task0, E, lane);
    if (lane == 0) s_total_tasks = total;
  }
  __syncthreads();
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
    header[tid] = v;
  }
}

}  // namespace moe

namespace moe_host {

hipError_t launch_route(const int32_t* ids, int P, int E, int block_m, int max_tasks,
                        void* routing, const moe_routing_layout_t& L, hipStream_t s) {
  char* base = static_cast<char*>(routing);
  hipLaunchKernelGGL(moe::route_kernel, dim3(1), dim3(moe::kRouteThreads), 0, s, ids, P, E,
                     block_m, max_tasks, reinterpret_cast<int32_t*>(base + L.header),
                     reinterpret_cast<int32_t*>(base + L.expert_offsets),
                     reinterpret_cast<int32_t*>(base + L.sorted_pairs),
                     reinterpret_cast<int32_t*>(base + L.pair_pos),
                     reinterpret_cast<moe_task_t*>(base + L.tasks));
  return hipGetLastError();
}

}  // namespace moe_host
