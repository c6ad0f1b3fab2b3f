// fa_fwd_bf16.hip -- bf16 prefill attention on gfx950 (dense and packed).
//
// Method: "S12 FlashAttention" (llminference.xinbetween.com), "Core idea /
// The solution" and "Mechanics / How it works": for each key/value tile, the
// running max moves to m_new, everything accumulated so far is corrected by
// alpha = exp(m_old - m_new), the tile's weights p = exp(s - m_new) are added
// to the running sum l and p.V to the output accumulator o; the output is
// o / l.  Outer loop over query tiles, inner loop over key/value tiles, as in
// "FlashAttention: The Algorithm That Beat the Memory Wall" (repo-explainer.com),
// "A Tile, a Register File, and a Trick Called Online Softmax".
//
// gfx950 mapping
//   * workgroup = 4 waves = 128 query rows of one (sequence, head); each wave
//     owns 32 rows for the whole key loop (Q fragments live in VGPRs).
//   * key/value tiles of 64 rows are staged in LDS, double-buffered: the next
//     tile's global loads are issued before the current tile's MFMAs and
//     written to the other buffer afterwards; one barrier per tile.
//   * scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16,
//     so each lane's accumulator column is ONE query row: the row max and row
//     sum are in-lane reductions plus one exchange with lane l ^ 32, and the
//     correction alpha is a per-lane scalar.
//   * the tile's weights P^T are already in the B-operand layout of the
//     second product O^T += V^T P^T (the contraction index is relabelled to
//     match), so P never leaves registers; V is stored transposed in LDS.
//   * scores are kept in base 2: x = s * scale * log2(e), p = 2^(x - m).
//   * causal tiles above the diagonal are never visited; only tiles that
//     straddle the diagonal or the sequence end are masked; a tile that is
//     fully masked for a wave is skipped by that wave.
//   * the first-tile NaN of "exp(-inf - -inf)" ("S12 FlashAttention", "Build
//     it / Implementation") is avoided by substituting 0 for a -inf running
//     max when forming exponents.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;  // query rows per workgroup
static_assert(kBr == kFwdRowsPerTile, "host tiling must match");
constexpr int kBc = 64;           // keys per tile
constexpr float kLazyLog2 = 8.f;  // max growth (base 2) tolerated before correcting o and l

template <int D>
struct Geometry {
  static constexpr int kStride = D + 8;         // K row in LDS, bf16 elements (16 B pad)
  static constexpr int vStride = kBc + 4;       // V^T row in LDS (8 B pad)
  static constexpr int kElems = kBc * kStride;
  static constexpr int vElems = D * vStride;
  static constexpr int kChunks = kBc * D / 8 / kThreads;  // 16-byte K chunks per thread
  static constexpr int vKeys = kBc * D / 8 / kThreads;    // keys per thread in the V transpose
  static constexpr int vKeyGroups = kBc / vKeys;          // key groups per tile
  // Thread t transposes keys vKeys*(t % vKeyGroups) .. +vKeys-1 of dims
  // 8*(t / vKeyGroups) .. +7.  Consecutive lanes take consecutive key groups
  // of the same V^T rows, so each LDS write instruction covers whole rows
  // (no bank conflicts); the V^T row pitch of 34 dwords keeps the reads of
  // 16 consecutive rows on distinct banks.
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(const FwdParams p) {
  using G = Geometry<D>;
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][G::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][G::vElems];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Work item.  Workgroups are dealt round-robin to the 8 XCDs; renumber so
  // each XCD receives a contiguous run of (sequence, head) pairs (their K/V
  // stay in that XCD's L2), and within a pair the heaviest causal query
  // tiles (the last ones) come first.
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
  if (q0 >= nq) return;  // uniform over the workgroup
  const int g = h / p.group;
  q_base += (int64_t)h * p.q_hs;
  k_base += (int64_t)g * p.k_hs;
  v_base += (int64_t)g * p.v_hs;
  o_base += (int64_t)h * p.o_hs;
  const int off = nk - nq;  // causal: key j visible from row i iff j <= i + off

  int ntiles = (nk + kBc - 1) / kBc;
  if (CAUSAL) {
    const int last = q0 + kBr - 1 + off;
    const int lim = last < 0 ? 0 : last / kBc + 1;
    ntiles = ntiles < lim ? ntiles : lim;
  }

  const uint16_t* __restrict__ qg = (const uint16_t*)p.q + q_base;
  const uint16_t* __restrict__ kg = (const uint16_t*)p.k + k_base;
  const uint16_t* __restrict__ vg = (const uint16_t*)p.v + v_base;

  // Q fragments: lane holds Q[row][16*kk + 8*hi .. +7] for every kk.
  const int rw0 = q0 + wave * 32;
  const int row = rw0 + l32;
  bf16x8 qf[D / 16];
  {
    const bool ok = row < nq;
    const uint16_t* qr = qg + (int64_t)(ok ? row : 0) * p.q_ss + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      uint4 x = ok ? *(const uint4*)(qr + 16 * kk) : make_uint4(0, 0, 0, 0);
      qf[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Global -> register staging of one K/V tile, then register -> LDS.
  uint4 kreg[G::kChunks];
  uint4 vreg[G::vKeys];
  // Rows past the end of the keys are zero-filled, so masked weights never
  // meet stale values; tiles wholly inside the keys take the unguarded path
  // (a uniform branch).
  const int kgrp = tid % G::vKeyGroups;
  const int vcol = (tid / G::vKeyGroups) * 8;
  auto gload = [&](int tile) {
    const int k0 = tile * kBc;
    if (k0 + kBc <= nk) {
#pragma unroll
      for (int i = 0; i < G::kChunks; ++i) {
        const int c = i * kThreads + tid;
        kreg[i] = *(const uint4*)(kg + (int64_t)(k0 + c / (D / 8)) * p.k_ss + (c % (D / 8)) * 8);
      }
#pragma unroll
      for (int i = 0; i < G::vKeys; ++i)
        vreg[i] = *(const uint4*)(vg + (int64_t)(k0 + kgrp * G::vKeys + i) * p.v_ss + vcol);
    } else {
#pragma unroll
      for (int i = 0; i < G::kChunks; ++i) {
        const int c = i * kThreads + tid;
        const int key = k0 + c / (D / 8);
        kreg[i] = key < nk ? *(const uint4*)(kg + (int64_t)key * p.k_ss + (c % (D / 8)) * 8)
                           : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < G::vKeys; ++i) {
        const int key = k0 + kgrp * G::vKeys + i;
        vreg[i] = key < nk ? *(const uint4*)(vg + (int64_t)key * p.v_ss + vcol) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < G::kChunks; ++i) {
      const int c = i * kThreads + tid;
      const int r = c / (D / 8);
      const int col = (c % (D / 8)) * 8;
      *(uint4*)&ks[buf][r * G::kStride + col] = kreg[i];
    }
    // Transpose: thread holds vKeys keys x 8 d; write 8 rows of V^T.
    const uint32_t* w32 = (const uint32_t*)vreg;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t packed[G::vKeys / 2];
#pragma unroll
      for (int i = 0; i < G::vKeys; i += 2) {
        const uint32_t a = w32[i * 4 + (e >> 1)];
        const uint32_t c = w32[(i + 1) * 4 + (e >> 1)];
        packed[i / 2] = (e & 1) ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
      }
      uint16_t* dst = &vt[buf][(vcol + e) * G::vStride + kgrp * G::vKeys];
      if constexpr (G::vKeys == 4) {
        *(uint2*)dst = make_uint2(packed[0], packed[1]);
      } else {
        *(uint32_t*)dst = packed[0];
      }
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = zero16();
  float m_run = -INFINITY;  // base-2 running max of this lane's row
  float l_run = 0.f;        // this half-wave's share of the running sum
  const float c = p.scale_log2;

  // The prologue runs even when no tile is visible (it only reads in-bounds
  // rows): waiting here for the first tile also retires the Q loads on every
  // path into the loop, so the loop never waits on them again.
  gload(0);
  lstore(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) gload(j + 1);
    const int k0 = j * kBc;
    const bool active = !CAUSAL || (k0 <= rw0 + 31 + off);
    if (active) {
      // S^T tile: two 32-key blocks.
      f32x16 sacc[2] = {zero16(), zero16()};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint4 a = *(const uint4*)&ks[buf][(kb * 32 + l32) * G::kStride + 16 * kk + 8 * hi];
          sacc[kb] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[kk], sacc[kb]);
        }
      }
      // Mask keys past the end and, for causal, keys past the row's limit.
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
      // Online softmax update for this lane's row.
      // Row max: a 4-way tree of max3 chains, then the other half-wave.
      float mx[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        mx[t] = fmaxf(sacc[t >> 1][8 * (t & 1)], sacc[t >> 1][8 * (t & 1) + 1]);
#pragma unroll
        for (int r = 2; r < 8; ++r) mx[t] = fmaxf(mx[t], sacc[t >> 1][8 * (t & 1) + r]);
      }
      float tmax = max_halves(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])));
      // Lazy correction: the reference max m_run moves (and o, l are scaled
      // by alpha = 2^(m_run - m_new)) only when some row of the wave sees its
      // max grow by more than kLazyLog2; otherwise the weights are taken
      // against the slightly stale reference, so p <= 2^kLazyLog2.  Any
      // reference gives the same o / l; this one keeps the correction off
      // the common path.
      const float m_new = fmaxf(m_run, tmax * c);
      if (__any(m_new > m_run + kLazyLog2)) {
        const float alpha = m_new == -INFINITY ? 1.f : exp2_fast(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      float ps[4] = {0.f, 0.f, 0.f, 0.f};  // four independent partial sums
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = exp2_fast(__builtin_fmaf(sacc[kb][r], c, -m_use));
          sacc[kb][r] = pv;
          ps[r & 3] += pv;
        }
      l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
      // O^T += V^T P^T over four 16-key chunks.  Contraction slot j of lane
      // half hi is key 16*kc + 4*hi + j (j < 4) or 16*kc + 8 + 4*hi + (j-4):
      // exactly the keys this lane's score registers 8*(kc%2) .. +7 hold.
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const int kb = kc >> 1;
        const int r0 = 8 * (kc & 1);
        uint4 pw;
        pw.x = pack_bf16x2(sacc[kb][r0 + 0], sacc[kb][r0 + 1]);
        pw.y = pack_bf16x2(sacc[kb][r0 + 2], sacc[kb][r0 + 3]);
        pw.z = pack_bf16x2(sacc[kb][r0 + 4], sacc[kb][r0 + 5]);
        pw.w = pack_bf16x2(sacc[kb][r0 + 6], sacc[kb][r0 + 7]);
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const uint16_t* vr = &vt[buf][(db * 32 + l32) * G::vStride + 16 * kc + 4 * hi];
          const uint2 lo = *(const uint2*)vr;
          const uint2 up = *(const uint2*)(vr + 8);
          const uint4 a = make_uint4(lo.x, lo.y, up.x, up.y);
          oacc[db] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pf, oacc[db]);
        }
      }
    }
    if (j + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: O = o / l, LSE = (m + log2 l) * ln 2.
  const float l_tot = sum_halves(l_run);
  if (row < nq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = (uint16_t*)p.o + o_base + (int64_t)row * p.o_ss;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = db * 32 + 8 * gq + 4 * hi;
        uint2 st;
        st.x = pack_bf16x2(oacc[db][4 * gq + 0] * inv, oacc[db][4 * gq + 1] * inv);
        st.y = pack_bf16x2(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv);
        *(uint2*)(orow + d) = st;
      }
    if (p.lse && hi == 0)
      p.lse[lse_base + row] = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const int64_t nwg = (int64_t)p.num_qtiles * p.heads_q * p.batch;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
  if (head_dim == 64) return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
