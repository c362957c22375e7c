// Asynchronous global -> LDS staging and LDS-read helpers shared by the
// attention kernels (gfx950).
#pragma once

#include "common.hpp"

namespace msa {

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// global -> LDS, 16 bytes per lane, lane l writing at lds_base + 16 l.
// Issued from inline asm so that the compiler does not treat the in-flight
// LDS writes as pending on every later LDS read (it would wait for the whole
// prefetch); completion is awaited explicitly with vmcnt.  The LDS base goes
// through M0, which the compiler does not expect an asm statement to change:
// its previous value is kept in a scalar register and put back.
__device__ __forceinline__ void g2lds16(const void* gaddr, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\t"
               "s_mov_b32 m0, %2\n\t"
               "s_nop 0\n\t"
               "global_load_lds_dwordx4 %1, off\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(gaddr), "s"(lds_base)
               : "memory");
}

// Same, addressed as scalar base + per-lane 32-bit byte offset (the saddr
// form: no 64-bit address arithmetic or registers per lane).
__device__ __forceinline__ void g2lds16_sv(const void* sbase, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\t"
               "s_mov_b32 m0, %3\n\t"
               "s_nop 0\n\t"
               "global_load_lds_dwordx4 %1, %2\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(voff), "s"(sbase), "s"(lds_base)
               : "memory");
}

// Workgroup barrier that does not drain outstanding global loads (unlike
// __syncthreads, whose release fence waits for every in-flight load,
// including the next block's prefetch).  Callers first wait on exactly the
// counters they need; the asm statements keep memory accesses in place.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ unsigned long long uniform64(unsigned long long x) {
  return ((unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32)) << 32) |
         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)x);
}

// The eight K operand fragments of one 32-key chunk (ds_read_b128 each),
// issued back to back and waited for once.  Outputs are early-clobber: a
// load may return while later loads of the block still read their address
// registers.
__device__ __forceinline__ void kfrag_load(u32x4 (&k)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %14\n\t"
      "ds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]),
        "=&v"(k[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
}

}  // namespace msa
