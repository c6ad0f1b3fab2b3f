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
//   * one workgroup per CU: 8 waves (2 per SIMD) x 32 query rows = 256 rows
//     of one (sequence, head).  Wave w owns rows q0 + w, q0 + w + 8, ...,
//     q0 + w + 248, so under a causal mask every wave sees the same number of
//     key tiles.  Q fragments and the output accumulator stay in registers.
//   * key and value tiles of 64 rows go from global memory straight into LDS
//     (global_load_lds, 16 bytes per lane, no register staging) through a
//     ring of 4 stages.  Rows are stored whole (d contiguous) with the 16-byte
//     chunks of each row XOR-swizzled so that both the score-operand reads and
//     the transposed value reads hit distinct banks.
//   * scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16,
//     so each lane's accumulator column is ONE query row: the row max and row
//     sum are in-lane reductions plus one v_permlane32_swap, and the
//     correction alpha is a per-lane scalar.
//   * the tile's weights P^T are already in the B-operand layout of the
//     second product O^T += V^T P^T (the contraction index is relabelled to
//     match), so P never leaves registers; the V^T operand is read from the
//     row-major V tile with ds_read_b64_tr_b16 (a 4 x 16 transpose of 16-bit
//     elements inside each 16-lane group).
//   * ping-pong: each wave alternates an MFMA phase (P.V of the previous tile
//     and the scores of the next) with a VALU phase (softmax).  Waves 4..7
//     run one phase behind waves 0..3 and every phase ends at a workgroup
//     barrier, so on each SIMD one wave is in its MFMA phase while the other
//     is in its softmax phase and both pipes stay busy.
//   * scores are kept in base 2: x = s * scale * log2(e), p = 2^(x - m).
//   * lazy correction: o and l are rescaled only when some row of the wave
//     sees its max grow by more than 2^8; otherwise the weights are formed
//     against the slightly stale reference (p <= 256).  Any reference gives
//     the same o / l.
//   * causal tiles above the diagonal are never visited; only tiles that
//     straddle the diagonal or the sequence end are masked.
//   * the first-tile NaN of "exp(-inf - -inf)" ("S12 FlashAttention", "Build
//     it / Implementation") is avoided by substituting 0 for a -inf reference
//     when forming exponents.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;   // query rows per workgroup
static_assert(kBr == kFwdRowsPerTileBf16, "host tiling must match");
constexpr int kBc = 64;            // keys per tile
constexpr int kStages = 4;         // LDS ring depth
constexpr float kLazyLog2 = 8.f;   // max growth (base 2) tolerated before correcting o and l

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// LDS swizzles, for 64 banks of 4 bytes.  ch = 16-byte chunks per row (16 or 8).
// Physical chunk of logical chunk c in key row r: the score-operand reads
// (16 lanes, 16 consecutive rows, one chunk) land on 16 distinct bank groups.
__device__ __forceinline__ int swz_k(int ch, int r, int c) {
  return ch == 16 ? c ^ (r & 15) : c ^ ((r >> 1) & 7);
}
// Value rows: the transposed reads (32 lanes, 4 consecutive rows x 4
// half-chunk pairs) land on distinct banks.
__device__ __forceinline__ int swz_v(int ch, int r, int c) {
  return ch == 16 ? c ^ (4 * (r & 3)) : c ^ (4 * ((r >> 1) & 1));
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

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(const FwdParams p) {
  constexpr int CH = D / 8;                // 16-byte chunks per row
  constexpr int TILE = kBc * D;            // elements per K or V tile
  constexpr int RPI = 512 / D;             // rows per 1 KB DMA instruction
  constexpr int IPW = kBc / RPI / kWaves;  // DMA instructions per wave per tile, per operand
  constexpr int IPT = 2 * IPW;             // ... for K and V together
  static_assert(IPW >= 1, "tile too small for the wave count");
  __shared__ __attribute__((aligned(1024))) uint16_t k_s[kStages][TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_s[kStages][TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: leads, 1: one phase behind
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

  // Key tiles the workgroup streams (every wave uses all of them).
  int nt = (nk + kBc - 1) / kBc;
  if (CAUSAL) {
    const int last = q0 + kBr - 1 + off;
    const int lim = last < 0 ? 0 : last / kBc + 1;
    nt = nt < lim ? nt : lim;
  }

  const uint16_t* __restrict__ qg = (const uint16_t*)p.q + q_base;
  const uint16_t* __restrict__ kg = (const uint16_t*)p.k + k_base;
  const uint16_t* __restrict__ vg = (const uint16_t*)p.v + v_base;

  // This lane's query row and its Q fragments Q[row][16*kk + 8*hi .. +7].
  const int row = q0 + 8 * l32 + wave;
  const int wrow0 = q0 + wave;  // the wave's first row
  // A row past the end of the queries (never stored) reads the last valid
  // row instead: each row's scores, max and sum stay in its own lane.
  bf16x8 qf[D / 16];
  {
    const uint16_t* qr = qg + (int64_t)min(row, nq - 1) * p.q_ss + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, *(const uint4*)(qr + 16 * kk));
  }
  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = zero16();
  float m_run = -INFINITY;  // base-2 reference max of this lane's row
  float l_run = 0.f;        // this half-wave's share of the running sum
  const float c = p.scale_log2;

  // DMA of one tile into its LDS stage; wave w covers rows 8w .. 8w+7.
  // Lane l of instruction i writes the 16 bytes at LDS row (8w + i*RPI +
  // l/CH), physical chunk l%CH, so it fetches the logical chunk the swizzle
  // maps there.  The tile's base address is uniform (scalar registers); the
  // per-lane byte offsets within a tile are the same for every full tile
  // (the host keeps them below 2^31).  In a tile that runs past the last key,
  // rows past the end re-read the last key row: their weights are exactly
  // zero and their values finite.
  const int drow = lane / CH;
  const int dpch = lane % CH;
  uint32_t koff[IPW], voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int r = wave * (kBc / kWaves) + i * RPI + drow;
    koff[i] = (uint32_t)(((int64_t)r * p.k_ss + swz_k(CH, r, dpch) * 8) * 2);
    voff[i] = (uint32_t)(((int64_t)r * p.v_ss + swz_v(CH, r, dpch) * 8) * 2);
  }
  auto dma = [&](int tile) {
    const int st = tile % kStages;
    const uint16_t* kt = kg + (int64_t)tile * kBc * p.k_ss;
    const uint16_t* vt = vg + (int64_t)tile * kBc * p.v_ss;
    const int rows_left = nk - tile * kBc;  // uniform
    if (rows_left >= kBc) {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int r0 = wave * (kBc / kWaves) + i * RPI;
        dma_16b(kt, koff[i], __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(&k_s[st][0] + r0 * D)));
        dma_16b(vt, voff[i], __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(&v_s[st][0] + r0 * D)));
      }
    } else {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int r0 = wave * (kBc / kWaves) + i * RPI;
        const int r = r0 + drow;
        const int rk = min(r, rows_left - 1);
        const uint32_t ko = (uint32_t)(((int64_t)rk * p.k_ss + swz_k(CH, r, dpch) * 8) * 2);
        const uint32_t vo = (uint32_t)(((int64_t)rk * p.v_ss + swz_v(CH, r, dpch) * 8) * 2);
        dma_16b(kt, ko, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(&k_s[st][0] + r0 * D)));
        dma_16b(vt, vo, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(&v_s[st][0] + r0 * D)));
      }
    }
  };

  if (nt > 0) dma(0);  // in flight while the Q fragments arrive

  // Scores of one tile (S^T, two 32-key blocks).
  f32x16 sacc[2];
  auto scores = [&](int t) {
    const uint16_t* ks = &k_s[t % kStages][0];
    sacc[0] = zero16();
    sacc[1] = zero16();
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int r = kb * 32 + l32;
        const uint4 a = *(const uint4*)&ks[r * D + swz_k(CH, r, 2 * kk + hi) * 8];
        sacc[kb] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[kk], sacc[kb]);
      }
    }
    // Keep four operand reads in flight ahead of the MFMAs (LDS latency is
    // several MFMAs long).
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < D / 8 - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };

  // Softmax of tile t in place (scores -> weights), producing the bf16 B
  // operands of the P.V product.
  bf16x8 pf[4];
  // The correction of o found by a softmax is applied at the start of the
  // following P.V phase (o is not touched in between); l is corrected at once.
  bool corr = false;   // the reference moved in the last softmax: o must be scaled by alpha
  float alpha = 1.f;
  auto softmax = [&](int t) {
    const int k0 = t * kBc;
    const bool need_mask = (k0 + kBc > nk) || (CAUSAL && k0 + kBc - 1 > wrow0 + off);
    if (need_mask) {
      const int lim = CAUSAL ? row + off : nk - 1;
      const int kend = (nk - 1 < lim ? nk - 1 : lim) - k0 - 4 * hi;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) > kend) sacc[kb][r] = -INFINITY;
    }
    float mx[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      mx[q] = fmaxf(sacc[q >> 1][8 * (q & 1)], sacc[q >> 1][8 * (q & 1) + 1]);
#pragma unroll
      for (int r = 2; r < 8; ++r) mx[q] = fmaxf(mx[q], sacc[q >> 1][8 * (q & 1) + r]);
    }
    const float tmax = max_halves(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]))) * c;
    const float m_new = fmaxf(m_run, tmax);
    corr = __any(m_new > m_run + kLazyLog2);
    if (corr) {
      alpha = m_new == -INFINITY ? 1.f : exp2_fast(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = exp2_fast(__builtin_fmaf(sacc[kb][r], c, -m_use));
        sacc[kb][r] = pv;
        ps[r & 3] += pv;
      }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int kb = kc >> 1;
      const int r0 = 8 * (kc & 1);
      uint4 pw;
      pw.x = pack_bf16x2(sacc[kb][r0 + 0], sacc[kb][r0 + 1]);
      pw.y = pack_bf16x2(sacc[kb][r0 + 2], sacc[kb][r0 + 3]);
      pw.z = pack_bf16x2(sacc[kb][r0 + 4], sacc[kb][r0 + 5]);
      pw.w = pack_bf16x2(sacc[kb][r0 + 6], sacc[kb][r0 + 7]);
      pf[kc] = __builtin_bit_cast(bf16x8, pw);
    }
  };

  // O^T += V^T P^T over four 16-key chunks of tile t.  Contraction slot j of
  // lane half hi is key 16*kc + 4*hi + j (j < 4) or 16*kc + 8 + 4*hi + (j-4):
  // exactly the keys the lane's score registers 8*(kc%2) .. +7 hold.  The two
  // transposed reads return those 8 keys for d = 32*db + l%32: lane (4k + q)
  // of each 16-lane group points at key row (base + k), dims
  // (16-block + 4q .. +3).
  const int g16 = lane >> 4;
  const int tk = (lane >> 2) & 3;
  const int tq = lane & 3;
  auto pv = [&](int t) {
    if (corr) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const uint16_t* vs = &v_s[t % kStages][0];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int dc = 4 * db + 2 * (g16 & 1) + (tq >> 1);  // logical 16-byte chunk
        const int ka = 16 * kc + 4 * hi + tk;
        const int kb2 = ka + 8;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)&vs[ka * D + swz_v(CH, ka, dc) * 8 + 4 * (tq & 1)]);
        const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)&vs[kb2 * D + swz_v(CH, kb2, dc) * 8 + 4 * (tq & 1)]);
        const uint2 l2 = __builtin_bit_cast(uint2, lo);
        const uint2 u2 = __builtin_bit_cast(uint2, up);
        const uint4 a = make_uint4(l2.x, l2.y, u2.x, u2.y);
        oacc[db] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pf[kc], oacc[db]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < D / 8 - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };

  // Phase schedule.  Global phases P = 0 .. 2*nt + 1, each ended by a
  // workgroup barrier.  Group 0 runs the MFMA phase of tile t (the scores of
  // tile t, then P.V of tile t - 1) in phase 2t and the softmax of tile t in
  // phase 2t + 1; group 1 runs the same sequence one phase later.  Scores go
  // first so that the next softmax waits only for them, not for the P.V
  // products queued behind them on the matrix pipe.  Tile t is
  // DMA'd at the start of phase 2t - 4 (prologue: tiles 0, 1) into stage
  // t % 4, whose previous tile t - 4 was last read in phase 2t - 5; each wave
  // waits for its share of tile (P+1)/2 at the end of odd phase P, just
  // before group 0 first reads it.  The two groups' loops are written out
  // separately so every phase is straight-line code.
  auto phase_begin = [&](int P) {
    if ((P & 1) == 0 && P / 2 + 2 < nt) dma(P / 2 + 2);
  };
  auto phase_end = [&](int P) {
    if (P & 1) {
      const int t_need = (P + 1) / 2;
      if (t_need < nt) {
        if (t_need + 1 < nt)
          wait_vmcnt<IPT>();
        else
          wait_vmcnt<0>();
      }
    }
    lds_barrier();
  };
  if (nt > 0) {
    // The Q loads were issued before tile 0's DMA (the DMA asm is a memory
    // barrier for the compiler); wait for both, then let tile 1 fly.
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(qf[kk]));
    wait_vmcnt<0>();
    if (nt > 1) dma(1);
    lds_barrier();
    if (grp == 0) {
      phase_begin(0);
      scores(0);
      phase_end(0);
      for (int t = 0; t < nt; ++t) {
        phase_begin(2 * t + 1);
        softmax(t);
        phase_end(2 * t + 1);
        phase_begin(2 * t + 2);
        if (t + 1 < nt) scores(t + 1);
        pv(t);
        phase_end(2 * t + 2);
      }
      phase_begin(2 * nt + 1);
      phase_end(2 * nt + 1);
    } else {
      phase_begin(0);
      phase_end(0);
      phase_begin(1);
      scores(0);
      phase_end(1);
      for (int t = 0; t < nt; ++t) {
        phase_begin(2 * t + 2);
        softmax(t);
        phase_end(2 * t + 2);
        phase_begin(2 * t + 3);
        if (t + 1 < nt) scores(t + 1);
        pv(t);
        phase_end(2 * t + 3);
      }
    }
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
