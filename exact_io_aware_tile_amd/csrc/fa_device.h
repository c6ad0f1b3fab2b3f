// fa_device.h -- gfx950 device helpers: MFMA wrappers, bf16 packing,
// base-2 transcendental wrappers, wave-level reductions, the LDS-DMA,
// wait and barrier primitives of the prefill pipelines, and the counter-based
// generator and byte threshold of attention dropout.
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

// Race check.  The prefill pipelines order their LDS ring by hand: each wave
// waits for exactly the DMA loads the next phase reads (wait_vmcnt<N>) and
// then meets the others at a fence-free barrier (lds_barrier).  Built with
// FA_SYNC_CHECK defined (a separate checking library, never the product),
// every such wait drains all of the wave's memory operations and every
// barrier is a full __syncthreads; a correct hand ordering gives the same
// bits, so any difference between the two builds exposes a stage read
// before its data landed or overwritten while still being read.
#ifdef FA_SYNC_CHECK
constexpr bool kSyncCheck = true;
#else
constexpr bool kSyncCheck = false;
#endif

// s_waitcnt immediates (gfx9 encoding): vmcnt(N) with expcnt / lgkmcnt left open.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  if (kSyncCheck)
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
  else
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
  if (kSyncCheck) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  } else {
    asm volatile("s_barrier" ::: "memory");
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Philox-4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011), from its published definition: ten rounds on a
// four-word counter; each round takes the 64-bit products of words 0 and 2
// with the two round multipliers, and the new words are, in order, the high
// half of the second product xor word 1 xor key word 0, its low half, the
// high half of the first product xor word 3 xor key word 1, and its low
// half.  The key words grow by the two Weyl constants after every round.
// The key is wave-uniform, so its schedule stays in scalar registers; it is
// rebuilt at each call (two scalar adds per round) instead of being hoisted
// out of the caller's loop as twenty live registers.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
  asm volatile("" : "+s"(k0), "+s"(k1));
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    // 0x96: the three-input exclusive or (one v_bitop3_b32 each)
    c = make_uint4(__builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.y, k0, 0x96), (uint32_t)p1,
                   __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w, k1, 0x96), (uint32_t)p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// Keep mask of two dropout bytes for two bf16 weights packed in one word:
// bytes 2*HALF and 2*HALF + 1 of w (little-endian) go to the low and high
// 16-bit halves; a half is 0xFFFF iff its byte is >= the threshold t, where
// tm1 holds t - 1 (t >= 1) in both halves: (t - 1) - byte is negative as a
// 16-bit integer exactly when byte >= t.
template <int HALF>
__device__ __forceinline__ uint32_t keep_mask16(uint32_t w, uint32_t tm1) {
  const uint32_t x = __builtin_amdgcn_perm(0u, w, HALF ? 0x0c030c02u : 0x0c010c00u);
  const u16x2 d = __builtin_bit_cast(u16x2, tm1) - __builtin_bit_cast(u16x2, x);
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, d) >> (short)15);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

}  // namespace fa
