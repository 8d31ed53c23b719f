// Low-level gfx950 helpers shared by the MFMA kernels: operand vector types,
// buffer descriptors, explicit s_waitcnt forms and the LDS-only barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace seqcomp {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// Raw buffer descriptor over `base` (no stride, no range limit that the
// 32-bit offsets could reach; dword 3 as for gfx9 raw buffers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const char* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, -1, 0x00020000);
}

// Raw buffer descriptor over [base, base + bytes): loads past the range
// return zero and stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ranged_rsrc(const char* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt with vmcnt(n) and the other counters left open (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(N) lgkmcnt(0), expcnt left open.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(N) with vmcnt and expcnt left open: at most N LDS (or
// scalar-memory) operations still outstanding.
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (N << 8) | (3 << 14));
}

// s_waitcnt lgkmcnt(0) with vmcnt and expcnt left open.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Workgroup barrier for pipelined loops.  __syncthreads() also fences global
// memory, which makes the compiler wait for EVERY outstanding load (vmcnt(0))
// and would drain a ring of in-flight copies; here the caller waits for
// exactly the copies it needs, and the empty asm statements keep the compiler
// from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace seqcomp
