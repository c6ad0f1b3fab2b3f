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
// gfx950 mapping of the split kernel: one wave per (sequence, kv head, split).
// A 16-token x 128-dim bf16 block is 4 KB; the wave reads it with four
// coalesced 16-byte loads per lane (lane l, load a: token 4a + l/16, dims
// 8*(l%16) .. +7), prefetching the next block's K and V while it computes the
// current one.  The G query heads of the group share every load.  Partial dot
// products are summed over the 16 lanes of a token with a reduce-scatter, so
// afterwards each lane owns the complete score of one (token, head) pair;
// the block's weights are exchanged through a 16 x G LDS table for the P.V
// step.  Split boundaries are multiples of the block size and depend only on
// logical token positions, so the result does not depend on where the blocks
// sit in the pool.
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

template <int G>
__global__ __launch_bounds__(64) void decode_split_kernel(const DecodeParams p) {
  constexpr int HPL = G >= 4 ? G / 4 : 1;  // heads per lane after the reduction
  constexpr int DUP = G >= 4 ? 1 : 4 / G;  // lanes that hold the same (token, head)
  constexpr int NV = 4 * G;                // partial dot products per lane
  __shared__ __attribute__((aligned(16))) float pl[kBlock][G];

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

  const int sub = lane >> 4;
  const int d8 = (lane & 15) * 8;
  const int my_tok = 4 * ((lane >> 2) & 3) + sub;
  const int hb = ((lane & 3) / DUP) * HPL;

  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 w = *(const uint4*)((const uint16_t*)p.q + (int64_t)b * p.q_bs +
                                    (int64_t)(g * G + h) * p.q_hs + d8);
    unpack8(w, qf[h]);
  }

  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  float m_run[HPL], l_run[HPL];
#pragma unroll
  for (int e = 0; e < HPL; ++e) {
    m_run[e] = -INFINITY;
    l_run[e] = 0.f;
  }

  const uint16_t* __restrict__ kpool = (const uint16_t*)p.k_pool + (int64_t)g * p.p_hs + d8;
  const uint16_t* __restrict__ vpool = (const uint16_t*)p.v_pool + (int64_t)g * p.p_hs + d8;
  const int32_t* __restrict__ bt = p.block_table + (int64_t)b * p.max_blocks;
  const float c = p.scale_log2;

  uint4 kc[4], vc[4];
  auto load = [&](int blk, uint4 (&kd)[4], uint4 (&vd)[4]) {
    const int64_t base = (int64_t)bt[blk] * p.p_bs;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int64_t off = base + (int64_t)(4 * a + sub) * p.p_ts;
      kd[a] = *(const uint4*)(kpool + off);
      vd[a] = *(const uint4*)(vpool + off);
    }
  };
  load(blk0, kc, vc);

  for (int blk = blk0; blk < blk1; ++blk) {
    uint4 kn[4], vn[4];
    if (blk + 1 < blk1) load(blk + 1, kn, vn);
    const int tok0 = blk * kBlock;

    // Partial q.k over this lane's 8 dims: x[a*G + h] for token 4a + sub.
    float x[NV];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float kf[8];
      unpack8(kc[a], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = __builtin_fmaf(qf[h][e], kf[e], s);
        x[a * G + h] = s;
      }
    }
    // Reduce-scatter over the 16 lanes of a token row: each stage keeps half
    // of the values (the half picked by one lane bit) and adds the partner's.
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int M = 8 >> st;
      const int cnt = NV >> st;
      if (cnt >= 2) {
        const bool up = (lane & M) != 0;
#pragma unroll
        for (int j = 0; j < cnt / 2; ++j) {
          const float keep = up ? x[cnt / 2 + j] : x[j];
          const float send = up ? x[j] : x[cnt / 2 + j];
          x[j] = keep + __shfl_xor(send, M, 64);
        }
      } else {
        x[0] += __shfl_xor(x[0], M, 64);
      }
    }
    // x[e] is now the full score of (my_tok, hb + e).
    const bool valid = tok0 + my_tok < t_end;
    float alpha[HPL];
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      const float s = valid ? x[e] : -INFINITY;
      float tmax = s;
      tmax = fmaxf(tmax, __shfl_xor(tmax, 4, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 8, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run[e], tmax * c);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      alpha[e] = exp2_fast(m_run[e] - m_use);
      const float pe = exp2_fast(__builtin_fmaf(s, c, -m_use));
      l_run[e] = alpha[e] * l_run[e] + pe;
      m_run[e] = m_new;
      if (lane % DUP == 0) pl[my_tok][hb + e] = pe;
    }
    __syncthreads();
    // Correct the accumulators of every head (alpha is uniform per head).
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float ah = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha[h % HPL]), (h / HPL) * DUP));
      if (ah != 1.f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= ah;
      }
    }
    // P.V for this lane's four tokens and 8 dims.
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int t = 4 * a + sub;
      float vf[8];
      unpack8(vc[a], vf);
      if (tok0 + t >= t_end) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = 0.f;
      }
      float pw[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pw[h] = pl[t][h];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = __builtin_fmaf(pw[h], vf[e], acc[h][e]);
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      kc[a] = kn[a];
      vc[a] = vn[a];
    }
  }

  // Sum l over the 16 tokens of a head and o over the 4 token sub-rows.
#pragma unroll
  for (int e = 0; e < HPL; ++e) {
    float l = l_run[e];
    l += __shfl_xor(l, 4, 64);
    l += __shfl_xor(l, 8, 64);
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    l_run[e] = l;
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[h][e];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      acc[h][e] = v;
    }

  const int64_t row0 = ((int64_t)b * p.heads_q + (int64_t)g * G) * p.num_splits + split;
  if (sub == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* dst = p.ws_o + (row0 + (int64_t)h * p.num_splits) * kD + d8;
      *(float4*)dst = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      *(float4*)(dst + 4) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
  }
  if (lane < 4 && lane % DUP == 0) {
#pragma unroll
    for (int e = 0; e < HPL; ++e) {
      float* ml = p.ws_ml + (row0 + (int64_t)(hb + e) * p.num_splits) * 2;
      ml[0] = m_run[e];
      ml[1] = l_run[e];
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
