// fa_decode.hip -- paged single-token decode with grouped-query heads, split
// across workgroups (flash-decoding) and merged by a second kernel.
//
// Sources: "S12 FlashAttention" (llminference.xinbetween.com):
//   * "What this unlocks beyond speed": tiles need not be contiguous -- each
//     can be a block fetched through the block table; with one query the
//     keys are split across thread blocks and the partial (m, l, o) states
//     are combined at the end;
//   * "How this composes with what you already built": one loop over the
//     block table that loads the KV head shared by the query's group and
//     updates (m, l, o);
//   * "Build it / Implementation" (paged excerpt): block i holds
//     min(block, seq_len - i*block) keys and the walk stops when that is <= 0.
// The merge of two partial states is the rule printed on the "FlashAttention"
// page of tachyon.techntrek.in ("For engineers / Show the maths"):
// m = max(m1, m2), l = e^(m1-m) l1 + e^(m2-m) l2, and o rescales the same way.
//
// gfx950 mapping of the split kernel: one wave per (sequence, kv head, split),
// no LDS and no barriers.  A 16-token x 128-dim bf16 block of one kv head is
// 4 KB; every 16-byte load of the wave covers 8 token rows x 128 contiguous
// bytes.  The G query heads of the group share every load (GQA).  q.k uses
// v_dot2_f32_bf16 on the raw bf16 pairs, and a token's partial dot products
// are summed across its 8 lanes with DPP moves.  Split boundaries are
// multiples of the block size and depend only on logical token positions, and
// nothing in the arithmetic depends on where a block sits in the pool, so a
// permuted pool gives bit-identical results.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBlock = 16;
constexpr int kD = 128;

__device__ __forceinline__ void unpack8(const uint4 w, float (&f)[8]) {
  f[0] = bf16_lo(w.x);
  f[1] = bf16_hi(w.x);
  f[2] = bf16_lo(w.y);
  f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z);
  f[5] = bf16_hi(w.z);
  f[6] = bf16_lo(w.w);
  f[7] = bf16_hi(w.w);
}

// Cross-lane moves inside a row of 16 lanes (DPP, no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowRor8 = 0x128;

// Sum over the 8 lanes that share lane bits 3..5 (one token row of a block).
__device__ __forceinline__ float sum8(float x) {
  x += dpp_mov<kQuadXor1>(x);
  x += dpp_mov<kQuadXor2>(x);
  x += dpp_mov<kRowHalfMirror>(x);  // lane i <-> 7 - i: the other quad of the 8
  return x;
}

// 8 bf16 of a and b: acc + sum a_i * b_i (fp32 accumulation, v_dot2_f32_bf16).
__device__ __forceinline__ float dot8(const uint4 a, const uint4 b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x), __builtin_bit_cast(bf16x2, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y), __builtin_bit_cast(bf16x2, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z), __builtin_bit_cast(bf16x2, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w), __builtin_bit_cast(bf16x2, b.w), acc, false);
  return acc;
}

// One block's K and V as this lane holds them: tokens t0 and t0 + 8, dims
// 8c..8c+7 and 64+8c..64+8c+7.
struct KV {
  uint4 k[2][2];
  uint4 v[2][2];
};

// Split kernel.  Lane l = 8*t0 + c owns tokens t0 and t0 + 8 of every block
// and the 16 dims {8c + e, 64 + 8c + e}; the 8 lanes of a token row read its
// 256 bytes with two fully coalesced 128-byte runs.  Each lane runs the
// recurrence on its own token stream (tokens t0, t0 + 8, t0 + 16, ...) with
// its own (m, l, o) per query head -- the keys of the split are split once
// more across the 8 token slots of the wave -- and the 8 slot states are
// merged with the same rule at the end of the split.  Three K/V buffers keep
// two blocks in flight while one is being consumed.
template <int G>
__global__ __launch_bounds__(64) void decode_split_kernel(const DecodeParams p) {
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;

  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
  const int t_begin = split * p.split_tokens;
  if (t_begin >= L) return;  // no keys in this split; the combine skips it
  const int t_end = L < t_begin + p.split_tokens ? L : t_begin + p.split_tokens;
  const int blk0 = t_begin / kBlock;
  const int blk1 = (t_end + kBlock - 1) / kBlock;

  const int c = lane & 7;
  const int t0 = lane >> 3;

  uint4 qv[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      qv[h][i] = *(const uint4*)((const uint16_t*)p.q + (int64_t)b * p.q_bs + (int64_t)(g * G + h) * p.q_hs +
                                 64 * i + 8 * c);

  float o[G][2][8];
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][i][e] = 0.f;
  }

  const uint16_t* __restrict__ kbase = (const uint16_t*)p.k_pool + (int64_t)g * p.p_hs + 8 * c;
  const uint16_t* __restrict__ vbase = (const uint16_t*)p.v_pool + (int64_t)g * p.p_hs + 8 * c;
  const int32_t* __restrict__ bt = p.block_table + (int64_t)b * p.max_blocks;
  const float cs = p.scale_log2;

  // Loads past the split's last block re-read that block (it is in cache);
  // their tokens are masked when processed.
  auto issue = [&](KV& B, int blk) {
    const int bb = blk < blk1 ? blk : blk1 - 1;
    const int64_t base = (int64_t)bt[bb] * p.p_bs;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t off = base + (int64_t)(t0 + 8 * a) * p.p_ts + 64 * i;
        B.k[a][i] = *(const uint4*)(kbase + off);
        B.v[a][i] = *(const uint4*)(vbase + off);
      }
  };

  // One block through the recurrence.  TAIL masks tokens at or past t_end
  // (only the sequence's last block can hold such tokens).
  auto process = [&](const KV& B, int blk, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
    const int tok0 = blk * kBlock;
    const bool ok0 = !TAIL || tok0 + t0 < t_end;
    const bool ok1 = !TAIL || tok0 + t0 + 8 < t_end;
    float s[2][G];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int h = 0; h < G; ++h) s[a][h] = sum8(dot8(qv[h][1], B.k[a][1], dot8(qv[h][0], B.k[a][0], 0.f)));
    float v0[2][8], v1[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      unpack8(B.v[0][i], v0[i]);
      unpack8(B.v[1][i], v1[i]);
      if (TAIL) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v0[i][e] = ok0 ? v0[i][e] : 0.f;
          v1[i][e] = ok1 ? v1[i][e] : 0.f;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float x0 = ok0 ? s[0][h] : -INFINITY;
      const float x1 = ok1 ? s[1][h] : -INFINITY;
      const float m_new = fmaxf(m[h], fmaxf(x0, x1) * cs);
      const float mu = (!TAIL || m_new != -INFINITY) ? m_new : 0.f;
      const float alpha = exp2_fast(m[h] - mu);
      const float p0 = exp2_fast(__builtin_fmaf(x0, cs, -mu));
      const float p1 = exp2_fast(__builtin_fmaf(x1, cs, -mu));
      l[h] = __builtin_fmaf(alpha, l[h], p0 + p1);
      m[h] = m_new;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          o[h][i][e] = __builtin_fmaf(p1, v1[i][e], __builtin_fmaf(p0, v0[i][e], o[h][i][e] * alpha));
    }
  };
  // Blocks wholly inside the split take the unmasked path; blocks past the
  // split's end (the ring's overrun) are skipped.  The branch is uniform.
  auto step = [&](const KV& B, int blk) {
    if (blk * kBlock + kBlock <= t_end) {
      process(B, blk, std::false_type{});
    } else if (blk < blk1) {
      process(B, blk, std::true_type{});
    }
  };

  // The scheduling barriers keep each ring refill where it is written, two
  // blocks ahead of its use, instead of letting the scheduler sink the loads
  // next to their consumers.
  KV A, B, C;
  issue(A, blk0);
  issue(B, blk0 + 1);
  issue(C, blk0 + 2);
  __builtin_amdgcn_sched_barrier(0);
  for (int blk = blk0; blk < blk1; blk += 3) {
    step(A, blk);
    __builtin_amdgcn_sched_barrier(0);
    issue(A, blk + 3);
    __builtin_amdgcn_sched_barrier(0);
    step(B, blk + 1);
    __builtin_amdgcn_sched_barrier(0);
    issue(B, blk + 4);
    __builtin_amdgcn_sched_barrier(0);
    step(C, blk + 2);
    __builtin_amdgcn_sched_barrier(0);
    issue(C, blk + 5);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Merge the 8 token-slot states (lane bits 3..5) pairwise.
#pragma unroll
  for (int st = 0; st < 3; ++st) {
    const int mask = 8 << st;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = st == 0 ? dpp_mov<kRowRor8>(m[h]) : __shfl_xor(m[h], mask, 64);
      const float lo = st == 0 ? dpp_mov<kRowRor8>(l[h]) : __shfl_xor(l[h], mask, 64);
      const float M = fmaxf(m[h], mo);
      const float mu = M == -INFINITY ? 0.f : M;
      const float w = exp2_fast(m[h] - mu);
      const float wo = exp2_fast(mo - mu);
      l[h] = w * l[h] + wo * lo;
      m[h] = M;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float oo = st == 0 ? dpp_mov<kRowRor8>(o[h][i][e]) : __shfl_xor(o[h][i][e], mask, 64);
          o[h][i][e] = w * o[h][i][e] + wo * oo;
        }
    }
  }

  if (t0 == 0) {
    const int64_t row0 = ((int64_t)b * p.heads_q + (int64_t)g * G) * p.num_splits + split;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* dst = p.ws_o + (row0 + (int64_t)h * p.num_splits) * kD + 8 * c;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        *(float4*)(dst + 64 * i) = make_float4(o[h][i][0], o[h][i][1], o[h][i][2], o[h][i][3]);
        *(float4*)(dst + 64 * i + 4) = make_float4(o[h][i][4], o[h][i][5], o[h][i][6], o[h][i][7]);
      }
      if (c == 0) {
        float* ml = p.ws_ml + (row0 + (int64_t)h * p.num_splits) * 2;
        ml[0] = m[h];
        ml[1] = l[h];
      }
    }
  }
}

// One wave per (sequence, query head): merge the sequence's non-empty splits.
__global__ __launch_bounds__(64) void decode_combine_kernel(const DecodeParams p) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
  const int ns = (L + p.split_tokens - 1) / p.split_tokens;
  const int64_t row0 = ((int64_t)b * p.heads_q + h) * p.num_splits;
  const float* ml = p.ws_ml + row0 * 2;

  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
  const float m_use = M == -INFINITY ? 0.f : M;
  float l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = exp2_fast(ml[2 * s] - m_use);
    l = __builtin_fmaf(w, ml[2 * s + 1], l);
    const float2 v = *(const float2*)(p.ws_o + (row0 + s) * kD + 2 * lane);
    o0 = __builtin_fmaf(w, v.x, o0);
    o1 = __builtin_fmaf(w, v.y, o1);
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  uint16_t* orow = (uint16_t*)p.o + (int64_t)b * p.o_bs + (int64_t)h * p.o_hs;
  *(uint32_t*)(orow + 2 * lane) = pack_bf16x2(o0 * inv, o1 * inv);
  if (p.lse && lane == 0)
    p.lse[(int64_t)b * p.heads_q + h] = l > 0.f ? (M + log2_fast(l)) * kLn2 : -INFINITY;
}

template <int G>
hipError_t launch_split(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(decode_split_kernel<G>, dim3(p.num_splits, p.heads_kv, p.batch), dim3(64), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_paged(const DecodeParams& p, hipStream_t stream) {
  hipError_t e;
  switch (p.group) {
    case 1: e = launch_split<1>(p, stream); break;
    case 2: e = launch_split<2>(p, stream); break;
    case 4: e = launch_split<4>(p, stream); break;
    case 8: e = launch_split<8>(p, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(p.heads_q, p.batch), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa
