// fa_fwd_f32.hip -- fp32 prefill attention on gfx950 (dense and packed).
//
// Same recurrence and work split as the bf16 kernel ("S12 FlashAttention",
// llminference.xinbetween.com, "Core idea / The solution"), on the fp32
// matrix cores: v_mfma_f32_32x32x2_f32, i.e. full fp32 products with fp32
// accumulation.  Scores are computed transposed (S^T = K Q^T) so a lane owns
// one query row; the second product O^T += V^T P^T takes one score register
// per step as its B operand (contraction slot hi of step (kb, r) is key
// 32*kb + 8*(r/4) + 4*hi + r%4), reading V straight from a row-major LDS tile.
// LDS is single-buffered: this path serves small fp32 problems where the
// tile loads are not the bottleneck.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;
static_assert(kBr == kFwdRowsPerTileF32, "host tiling must match");
constexpr int kBc = 64;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(const FwdParams p) {
  constexpr int kStride = D + 1;  // pad K rows: lanes read 32 different rows per column
  __shared__ float ks[kBc * kStride];
  __shared__ float vs[kBc * D];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int nwg = gridDim.x;
  const int w = blockIdx.x;
  const int lin = (nwg % 8 == 0) ? (w % 8) * (nwg / 8) + (w / 8) : w;
  const int qt = p.num_qtiles - 1 - (lin % p.num_qtiles);
  const int bh = lin / p.num_qtiles;
  const int h = bh % p.heads_q;
  const int b = bh / p.heads_q;

  int nq, nk;
  int64_t q_base, k_base, v_base, o_base, lse_base;
  if (p.cu_seqlens) {
    const int s0 = p.cu_seqlens[b];
    const int s1 = p.cu_seqlens[b + 1];
    nq = nk = s1 - s0;
    q_base = (int64_t)s0 * p.q_ss;
    k_base = (int64_t)s0 * p.k_ss;
    v_base = (int64_t)s0 * p.v_ss;
    o_base = (int64_t)s0 * p.o_ss;
    lse_base = (int64_t)h * p.total_tokens + s0;
  } else {
    nq = p.seqlen_q;
    nk = p.seqlen_k;
    q_base = (int64_t)b * p.q_bs;
    k_base = (int64_t)b * p.k_bs;
    v_base = (int64_t)b * p.v_bs;
    o_base = (int64_t)b * p.o_bs;
    lse_base = ((int64_t)b * p.heads_q + h) * nq;
  }
  const int q0 = qt * kBr;
  if (q0 >= nq) return;
  const int g = h / p.group;
  q_base += (int64_t)h * p.q_hs;
  k_base += (int64_t)g * p.k_hs;
  v_base += (int64_t)g * p.v_hs;
  o_base += (int64_t)h * p.o_hs;
  const int off = nk - nq;

  int ntiles = (nk + kBc - 1) / kBc;
  if (CAUSAL) {
    const int last = q0 + kBr - 1 + off;
    const int lim = last < 0 ? 0 : last / kBc + 1;
    ntiles = ntiles < lim ? ntiles : lim;
  }

  const float* __restrict__ qg = (const float*)p.q + q_base;
  const float* __restrict__ kg = (const float*)p.k + k_base;
  const float* __restrict__ vg = (const float*)p.v + v_base;

  const int rw0 = q0 + wave * 32;
  const int row = rw0 + l32;
  float qf[D / 2];  // Q[row][2*kk + hi]
  {
    const bool ok = row < nq;
    const float* qr = qg + (int64_t)(ok ? row : 0) * p.q_ss;
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) qf[kk] = ok ? qr[2 * kk + hi] : 0.f;
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = zero16();
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c = p.scale_log2;

  for (int j = 0; j < ntiles; ++j) {
    const int k0 = j * kBc;
    // Cooperative tile load, 16 bytes per access.
#pragma unroll
    for (int i = 0; i < kBc * D / 4 / kThreads; ++i) {
      const int cidx = i * kThreads + tid;
      const int r = cidx / (D / 4);
      const int col = (cidx % (D / 4)) * 4;
      const int key = k0 + r;
      float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
      if (key < nk) {
        kx = *(const float4*)(kg + (int64_t)key * p.k_ss + col);
        vx = *(const float4*)(vg + (int64_t)key * p.v_ss + col);
      }
      float* kd = &ks[r * kStride + col];
      kd[0] = kx.x;
      kd[1] = kx.y;
      kd[2] = kx.z;
      kd[3] = kx.w;
      *(float4*)&vs[r * D + col] = vx;
    }
    __syncthreads();

    if (!CAUSAL || k0 <= rw0 + 31 + off) {
      f32x16 sacc[2] = {zero16(), zero16()};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk)
          sacc[kb] = mfma_32x32x2_f32(ks[(kb * 32 + l32) * kStride + 2 * kk + hi], qf[kk], sacc[kb]);

      const bool need_mask = (k0 + kBc > nk) || (CAUSAL && k0 + kBc - 1 > rw0 + off);
      if (need_mask) {
        const int lim = CAUSAL ? row + off : nk - 1;
        const int kend = nk - 1 < lim ? nk - 1 : lim;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key > kend) sacc[kb][r] = -INFINITY;
          }
      }
      float tmax = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[kb][r]);
      tmax = max_halves(tmax);
      const float m_new = fmaxf(m_run, tmax * c);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = exp2_fast(__builtin_fmaf(sacc[kb][r], c, -m_use));
          sacc[kb][r] = pv;
          psum += pv;
        }
      l_run = alpha * l_run + psum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
            oacc[db] = mfma_32x32x2_f32(vs[key * D + db * 32 + l32], sacc[kb][r], oacc[db]);
        }
    }
    __syncthreads();
  }

  const float l_tot = sum_halves(l_run);
  if (row < nq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* orow = (float*)p.o + o_base + (int64_t)row * p.o_ss;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = db * 32 + 8 * gq + 4 * hi;
        *(float4*)(orow + d) = make_float4(oacc[db][4 * gq + 0] * inv, oacc[db][4 * gq + 1] * inv,
                                           oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv);
      }
    if (p.lse && hi == 0)
      p.lse[lse_base + row] = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const int64_t nwg = (int64_t)p.num_qtiles * p.heads_q * p.batch;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
  if (head_dim == 64) return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
