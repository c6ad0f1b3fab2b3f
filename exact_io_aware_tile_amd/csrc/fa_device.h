// fa_device.h -- gfx950 device helpers: MFMA wrappers, bf16 packing,
// base-2 transcendental wrappers, wave-level reductions, and the LDS-DMA,
// wait and barrier primitives of the prefill pipelines.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

constexpr float kLn2 = 0.693147180559945309417f;

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16).
// Lane l supplies A[l % 32][8 * (l / 32) + j] and B[8 * (l / 32) + j][l % 32]
// for j = 0..7; accumulator register r of lane l holds
// D[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32].
__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(32x32 fp32) += A(32x2 fp32) * B(2x32 fp32); lane l supplies
// A[l % 32][l / 32] and B[l / 32][l % 32]; same accumulator layout.
__device__ __forceinline__ f32x16 mfma_32x32x2_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// bf16 halves of a 32-bit word, widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even) in one 32-bit word, lo first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// max / sum of x over lanes l and l ^ 32 (the two halves of a wave), via
// v_permlane32_swap: swapping a register with itself leaves {x[l], x[l^32]}
// in the two results on every lane, in some order.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One LDS-DMA instruction: lane l's 16 bytes at base + off (base wave-uniform,
// off a per-lane 32-bit byte offset) land at LDS byte address lds + 16 l
// (lds wave-uniform).  Issued from asm so that the compiler does not track
// the LDS write: it cannot tell the stage being filled from the stages being
// read and would otherwise wait for every DMA in flight before the next LDS
// read.  The kernel orders DMA and reads itself (wait_vmcnt + lds_barrier).
// m0 is saved and restored around the instruction, with the one wait state
// gfx9 needs between an m0 write and an LDS DMA.
__device__ __forceinline__ void dma_16b(const void* base, uint32_t off, uint32_t lds) {
  uint32_t m0_save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_save)
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}

// s_waitcnt immediates (gfx9 encoding): vmcnt(N) with expcnt / lgkmcnt left open.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Workgroup barrier for the LDS ring.  __syncthreads() carries a release
// fence, which waits for every outstanding global load -- including the
// LDS-DMA prefetches of later tiles -- and would drain the ring at each
// phase.  Here each wave waits for exactly the DMA loads the next phase needs
// (wait_vmcnt) before the barrier; LDS reads complete before their MFMA
// consumers inside the phase, and the memory clobber keeps the compiler from
// moving any LDS access across the barrier.
// The scheduling fences on both sides keep each phase's instructions
// (MFMA and exponentials included) inside the phase.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

}  // namespace fa
