// Device helpers shared by the LDS-staged GEMM kernels: direct global->LDS
// copies, explicit vector-memory waits, a barrier without a memory fence,
// and scalar (constant-cache) loads of wave-uniform records.
#pragma once

#include "moe_common.h"

namespace moe {

typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));

// global_load_lds_dwordx4: each lane copies 16 bytes from src into LDS; one
// wave instruction fills 1 KiB at lds_dst (lane l writes bytes 16l..16l+15).
// Completion is tracked by vmcnt like any vector load.
__device__ __forceinline__ void dma16(const void* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 16, 0, 0);
}

// global_load_lds_dword: each lane copies 4 bytes; one wave instruction fills
// 256 bytes at lds_dst (lane l writes bytes 4l..4l+3).
__device__ __forceinline__ void dma4(const void* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 4, 0, 0);
}

// Workgroup barrier without a memory fence (a fence would drain every
// in-flight load); the empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void barrier_nofence() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding (loads complete in issue order, so every older one is done).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// A wave-uniform address, placed in scalar registers: the compiler may have
// computed it with vector instructions (under scalar-register pressure), and
// a scalar load takes its address from scalar registers only.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return reinterpret_cast<const T*>(((unsigned long long)hi << 32) | lo);
}

// Scalar load of a wave-uniform 16-byte task record.  Its wait is on
// lgkmcnt, so it does not drain in-flight vector loads as a vector load's
// vmcnt wait would.
__device__ __forceinline__ moe_task_t load_task_scalar(const moe_task_t* p) {
  i32x4_t v;
  __asm__ volatile("s_load_dwordx4 %0, %1, 0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(p)) : "memory");
  moe_task_t t;
  t.expert = v[0];
  t.row_begin = v[1];
  t.rows = v[2];
  t.reserved = v[3];
  return t;
}

// Scalar load of 16 consecutive wave-uniform dwords (64 bytes, 4-byte aligned).
__device__ __forceinline__ i32x16_t load16_scalar(const void* p) {
  i32x16_t v;
  __asm__ volatile("s_load_dwordx16 %0, %1, 0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(p)) : "memory");
  return v;
}

// Scalar load of one wave-uniform dword.
__device__ __forceinline__ int load1_scalar(const void* p) {
  int v;
  __asm__ volatile("s_load_dword %0, %1, 0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(p)) : "memory");
  return v;
}

// Lane l receives v[j] for its own j in [0, 16).
__device__ __forceinline__ int pick16(const i32x16_t& v, int j) {
  int r = v[0];
#pragma unroll
  for (int i = 1; i < 16; i++) r = (j == i) ? v[i] : r;
  return r;
}

// Token chunks in LDS (16 gathered rows x one 64-byte K step, one wave copy
// instruction).  The copy gives each quad of lanes one row's 64 contiguous
// bytes: lane l fetches row l / 4, 16-byte piece (l % 4) ^ tok_swz(row).
// Copies in MFMA lane order (lane l: row l % 16) touch 16 rows in every
// quad and move about half as many bytes per CU cycle from L2 (measured on
// gfx950: 35 against 62 GB/s per CU).  Row r thus sits at bytes 64 r of the
// chunk with its pieces permuted by tok_swz(r).  With this permutation the
// MFMA-order fragment reads below (ds_read_b128) run without LDS bank
// conflicts (SQ_LDS_BANK_CONFLICT = 0, 4 LDS cycles per wave read); the
// unpermuted layout and several other per-row permutations measured 2-way
// conflicts.
__device__ __forceinline__ int tok_swz(int row) { return (row >> 1) & 3; }
__device__ __forceinline__ int tok_copy_row(int lane) { return lane >> 2; }
__device__ __forceinline__ int tok_copy_piece(int lane) { return (lane & 3) ^ tok_swz(lane >> 2); }
// Byte offset, in such a chunk, of MFMA lane `lane`'s fragment (row
// lane % 16, piece lane / 16).
__device__ __forceinline__ int tok_frag_off(int lane) {
  const int r = lane & 15;
  return 64 * r + 16 * ((lane >> 4) ^ tok_swz(r));
}

// Lane l receives v[l % 16].
__device__ __forceinline__ int spread16(const i32x16_t& v, int lane) {
  const int j = lane & 15;
  int r = v[0];
#pragma unroll
  for (int i = 1; i < 16; i++) r = (j == i) ? v[i] : r;
  return r;
}

}  // namespace moe
