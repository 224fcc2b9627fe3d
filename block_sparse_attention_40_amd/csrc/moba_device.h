// Device-side helpers shared by the MoBA HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moba {

typedef uint16_t bf16raw;  // bfloat16 bit pattern as stored in HBM

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(bf16raw x) {
  return __builtin_bit_cast(float, (uint32_t)x << 16);
}

// Low / high bf16 of a packed 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 pair, packed (lo = a, hi = b); one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Hardware base-2 exponential / logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Element loads widened to fp32 for the two storage types.
__device__ __forceinline__ float load_f32(const float* p) { return *p; }
__device__ __forceinline__ float load_f32(const bf16raw* p) { return bf16_to_f32(*p); }

// Eight consecutive elements widened to fp32 (16-byte or 2x16-byte load).
__device__ __forceinline__ void load8(const bf16raw* p, float* o) {
  u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) { o[2 * i] = bf16lo(w[i]); o[2 * i + 1] = bf16hi(w[i]); }
}
__device__ __forceinline__ void load8(const float* p, float* o) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { o[i] = a[i]; o[4 + i] = b[i]; }
}

// Wait until every vector-memory load issued so far has returned
// (s_waitcnt vmcnt(0)), and keep the scheduler from moving loads across.
__device__ __forceinline__ void drain_vmem() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt = 0; expcnt, lgkmcnt unconstrained
  __builtin_amdgcn_sched_barrier(0);
}

// One 16-byte unit per lane from global memory straight into LDS, at
// lds_base + 16 * lane (global_load_lds_dwordx4 with m0 = lds_base, a
// wave-uniform value; m0 is saved and restored around the load).  Written as
// inline asm, so the compiler neither tracks the load nor waits for it: the
// caller waits (s_waitcnt vmcnt) before the barrier that publishes the data,
// and the memory clobber keeps LDS accesses on their side of the load.
__device__ __forceinline__ void lds_dma16(uint32_t lds_base, const void* gptr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(gptr)
      : "memory");
}

// Order-preserving map of an fp32 score to uint32 (NaN must be removed first).
__device__ __forceinline__ uint32_t orderable(float s) {
  uint32_t u = __builtin_bit_cast(uint32_t, s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace moba
