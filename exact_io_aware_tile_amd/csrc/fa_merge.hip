// fa_merge.hip -- merge of attention results over disjoint key sets.
//
// Method: the (m, l, o) merge rule of "FlashAttention"
// (tachyon.techntrek.in), "For engineers / Show the maths", taken over P
// states at once.  A state given as a normalised output o_p and its
// log-sum-exp lse_p is (m_p, l_p, o_p) with lse_p = m_p + log l_p; against
// the common reference m = max_p lse_p each state weighs w_p = exp(lse_p - m)
// = l_p exp(m_p - m), so the union has o = sum w_p o_p / sum w_p and
// lse = m + log sum w_p.  "S12 FlashAttention" (llminference.xinbetween.com),
// "What this unlocks beyond speed", applies the same merge to the states of
// one sequence's key shards held on different GPUs (ring attention) and to
// flash-decoding splits.
//
// gfx950 mapping: pure streaming, bound by HBM.  One lane owns 8 consecutive
// elements of one output row (one 16-byte bf16 load per part, two for fp32),
// so a wave covers whole rows with fully coalesced, non-temporal loads (each
// input byte is read once).  The row's P log-sum-exps are read by all of its
// lanes at the same address and served by one cache line.  Parts are
// taken eight at a time in one pass, all eight loads in flight together.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kMergeThreads = 256;
constexpr int kGroup = 8;  // parts whose loads are in flight together
constexpr int64_t kMergeMaxGrid = 65536;  // workgroups; the rest is a grid-stride loop
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool F32>
__device__ __forceinline__ void load8(const void* base, int64_t e, float (&x)[8]) {
  if (F32) {
    const f32x4* s = (const f32x4*)((const float*)base + e);
    const f32x4 a = __builtin_nontemporal_load(s);
    const f32x4 b = __builtin_nontemporal_load(s + 1);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    const u32x4 w = __builtin_nontemporal_load((const u32x4*)((const uint16_t*)base + e));
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(u[i] << 16);
      x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
}

template <int D, bool F32>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeParams p) {
  constexpr int CPR = D / 8;  // lanes per row
  const int64_t n = p.rows * CPR;  // < 2^31
  const float kLog2e = 1.4426950408889634f;
  // Lane indices stay below 2^31 (the host bounds a part below 2^34
  // elements), so a row splits into (batch, seqlen, head) by the divisors
  // the host prepared, without any runtime division.
  for (int64_t i = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kMergeThreads) {
    const int r = (int)i / CPR;  // row (b, s, h) of the [batch, seqlen, heads] order
    const int c = (int)i % CPR;
    const int bs = idiv(r, p.by_heads);
    const int h = r - bs * p.heads;
    const int b = idiv(bs, p.by_seqlen);
    const int s = bs - b * p.seqlen;
    const int64_t li = ((int64_t)b * p.heads + h) * p.seqlen + s;  // [batch, heads, seqlen] order
    const int64_t e = (int64_t)r * D + 8 * c;

    // One pass over the parts in groups of kGroup: a group's loads (its
    // log-sum-exps and output rows) are all issued before any is used, the
    // group's max moves the running reference m, and what was accumulated
    // against the old reference is rescaled by exp(m_old - m_new) -- the
    // pages' own recurrence, with states in place of key tiles.  Past the
    // last part the index is clamped to it (a valid address) and the part
    // counts as empty.
    float m = -INFINITY;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float sw = 0.f;
    for (int q0 = 0; q0 < p.parts; q0 += kGroup) {
      float lq[kGroup];
      float x[kGroup][8];
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        const int64_t q = min(q0 + u, p.parts - 1);
        lq[u] = p.lse_parts[q * p.part_rows + li];
        if (q0 + u >= p.parts) lq[u] = -INFINITY;
        load8<F32>(p.o_parts, q * p.part_elems + e, x[u]);
      }
      float gm = lq[0];
#pragma unroll
      for (int u = 1; u < kGroup; ++u) gm = fmaxf(gm, lq[u]);
      if (gm == -INFINITY) continue;  // no part of the group saw a key of this row
      const float m_new = fmaxf(m, gm);
      const float a = exp2f((m - m_new) * kLog2e);  // 0 while nothing was accumulated (m = -inf)
      sw *= a;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= a;
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        // A part that saw no key (lse -inf) contributes nothing, whatever
        // its output row holds.
        const bool live = lq[u] != -INFINITY;
        const float w = live ? exp2f((lq[u] - m_new) * kLog2e) : 0.f;
        sw += w;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += live ? w * x[u][j] : 0.f;
      }
      m = m_new;
    }
    // sw >= 1: the part that holds the max weighs exactly 1.
    const float inv = m != -INFINITY ? 1.f / sw : 0.f;
    if (F32) {
      float4* d = (float4*)((float*)p.o + e);
      d[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
      d[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    } else {
      uint4 w;
      w.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
      w.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
      w.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
      w.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
      *(uint4*)((uint16_t*)p.o + e) = w;
    }
    if (p.lse && c == 0) p.lse[li] = m != -INFINITY ? m + logf(sw) : -INFINITY;
  }
}

template <int D>
hipError_t launch_merge_d(const MergeParams& p, hipStream_t stream) {
  const int64_t n = p.rows * (D / 8);
  const int64_t blocks = (n + kMergeThreads - 1) / kMergeThreads;
  const unsigned grid = (unsigned)(blocks < kMergeMaxGrid ? blocks : kMergeMaxGrid);
  if (p.f32)
    merge_kernel<D, true><<<grid, kMergeThreads, 0, stream>>>(p);
  else
    merge_kernel<D, false><<<grid, kMergeThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  switch (p.head_dim) {
    case 64: return launch_merge_d<64>(p, stream);
    case 128: return launch_merge_d<128>(p, stream);
    case 256: return launch_merge_d<256>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
