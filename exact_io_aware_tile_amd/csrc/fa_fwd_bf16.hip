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
//     of one (sequence, head).  Wave w owns rows q0 + 32 w .. +31, so under a
//     causal mask only the waves at the diagonal mask a tile, and the first
//     four waves (128 rows) stop computing two tiles before the last four.
//     Q fragments and the output accumulator stay in registers.
//   * key and value tiles of 64 rows (128 in the dense and packed head-dim-64
//     instances) go from global memory straight into LDS (global_load_lds,
//     16 bytes per lane, no register staging) through a ring of 4 stages.  Rows are stored whole (d contiguous) with the 16-byte
//     chunks of each row XOR-swizzled so that both the score-operand reads and
//     the transposed value reads hit distinct banks.  The waves in their
//     MFMA phase issue the loads, spread between the products: a load that
//     waits for the CU's vector-memory path delays the next product only by
//     what the matrix pipe has not yet absorbed of the one before it.
//   * scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16,
//     so each lane's accumulator column is ONE query row: the row max and row
//     sum are in-lane reductions plus one v_permlane32_swap, and the
//     correction alpha is a per-lane scalar.
//   * the tile's weights P^T are already in the B-operand layout of the
//     second product O^T += V^T P^T (the contraction index is relabelled to
//     match), so P never leaves registers; the V^T operand is read from the
//     row-major V tile with ds_read_b64_tr_b16 (a 4 x 16 transpose of 16-bit
//     elements inside each 16-lane group).
//   * ping-pong: each wave alternates an MFMA phase (the scores of the next
//     tile and P.V of the previous one) with a VALU phase (softmax).  Waves 4..7
//     run one phase behind waves 0..3 and every phase ends at a workgroup
//     barrier, so on each SIMD one wave is in its MFMA phase while the other
//     is in its softmax phase and both pipes stay busy.  The MFMA-phase wave
//     raises its issue priority (s_setprio), so the matrix pipe is fed first.
//   * scores are kept in base 2: x = s * scale * log2(e), p = 2^(x - m).
//   * lazy correction: a tile's weights are formed against the reference
//     max of an earlier tile, and the row max is not even taken, as long as
//     no weight exceeds 2^16 (checked on each lane's partial sum).  Only
//     then is the tile's max taken, o and l rescaled and the weights
//     recomputed.  Any reference gives the same o / l; fp32 and bf16 carry
//     weights up to 2^16 without loss of relative precision.
//   * o is divided by the sum of the weights as P.V took them (rounded to
//     bf16), so each output row is a convex combination of value rows; the
//     LSE uses the fp32 sum.
//   * causal tiles above the diagonal are never visited; only tiles that
//     straddle the diagonal or the sequence end are masked.
//   * dropout (a compile-time variant, as "FlashAttention: The Algorithm That
//     Beat the Memory Wall", "Why Templates Matter Here", describes the
//     kernel family): each weight is kept or zeroed by one byte of a
//     counter-based generator drawn in registers (in the MFMA phase before
//     the tile's softmax, where the vector ALU is idle), so no mask is
//     stored; the dropped weights still count in l, and O is scaled
//     by 256 / (256 - t) at the end (t the byte threshold).
//   * the first-tile NaN of "exp(-inf - -inf)" ("S12 FlashAttention", "Build
//     it / Implementation") is avoided by substituting 0 for a -inf reference
//     when forming exponents.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;   // query rows per workgroup
static_assert(kBr == kFwdRowsPerTileBf16, "host tiling must match");
constexpr int kBc = 64;            // keys per tile (128 in the plain head-dim-64 instance, see BC below)
constexpr int kStages = 4;         // LDS ring depth
constexpr float kLazyBound = 65536.f;  // largest weight (2^16) formed against a stale reference

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

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

template <int D, bool CAUSAL, bool PAGED, bool DROP>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(const FwdParams p) {
  static_assert(!(PAGED && DROP), "dropout is built for dense and packed prefill");
  // Keys per tile: at head_dim 64 a 64-key tile holds only 16 products per
  // wave and phase against the same per-tile softmax bookkeeping, so the
  // dense and packed instances take 128 keys (the same 16 KB per stage as
  // d = 128).  The paged instance keeps 64 (one 16-token pool block per wave
  // and tile), and so does dropout (128 keys would spill its registers).
  constexpr int BC = (D == 64 && !PAGED && !DROP) ? 128 : kBc;
  constexpr int NKB = BC / 32;             // 32-key score blocks of a tile
  constexpr int NKC = BC / 16;             // 16-key chunks of the P.V contraction
  constexpr int CH = D / 8;                // 16-byte chunks per row
  constexpr int TILE = BC * D;             // elements per K or V tile
  constexpr int RPI = 512 / D;              // rows per 1 KB DMA instruction
  constexpr int RPW = BC / 4;               // rows per wave when one group loads an operand
  constexpr int IPW = RPW / RPI;            // DMA instructions per wave per operand of a tile
  static_assert(IPW >= 1 && IPW <= 4 && RPW % RPI == 0, "DMA split");
  __shared__ __attribute__((aligned(1024))) uint16_t k_s[kStages][TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_s[kStages][TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: leads, 1: one phase behind
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Work item: XCD-balanced, longest first (prefill_work_item).
  int qt, bh;
  prefill_work_item(p.wmap, blockIdx.x, qt, bh);
  const int b = idiv(bh, p.by_heads);
  const int h = bh - b * p.heads_q;

  int nq, nk;
  int64_t q_base, k_base, v_base, o_base, lse_base;
  if (PAGED) {
    // new queries packed by cu_seqlens; keys of the sequence in the pools
    const int s0 = p.cu_seqlens[b];
    nq = p.cu_seqlens[b + 1] - s0;
    nk = min(max(p.seq_lens_k[b], 0), p.seqlen_k);
    q_base = (int64_t)s0 * p.q_ss;
    k_base = 0;
    v_base = 0;
    o_base = (int64_t)s0 * p.o_ss;
    lse_base = (int64_t)h * p.total_tokens + s0;
  } else if (p.cu_seqlens) {
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
  const int g = idiv(h, p.wmap.by_group);
  q_base += (int64_t)h * p.q_hs;
  k_base += (int64_t)g * (PAGED ? p.p_hs : p.k_hs);
  v_base += (int64_t)g * (PAGED ? p.p_hs : p.v_hs);
  o_base += (int64_t)h * p.o_hs;
  const int off = nk - nq;  // causal: key j visible from row i iff j <= i + off

  // Key tiles the workgroup streams.  Under a causal mask the first 128 rows
  // (group 0) see no key of the last tiles: that group computes only its
  // first nt0 tiles and then keeps to the phase barriers (and its load
  // waits) while group 1 finishes alone.  nt0 >= nt - 3 holds by
  // construction, so the keys group 0 loads four tiles ahead are all issued
  // before it stops.
  int nt = (nk + BC - 1) / BC;
  int nt0 = nt;
  if (CAUSAL) {
    const int last = q0 + kBr - 1 + off;
    const int lim = last < 0 ? 0 : last / BC + 1;
    nt = nt < lim ? nt : lim;
    const int last0 = q0 + kBr / 2 - 1 + off;
    const int lim0 = last0 < 0 ? 0 : last0 / BC + 1;
    nt0 = max(min(nt, lim0), max(nt - 3, 1));
  }

  const uint16_t* __restrict__ qg = (const uint16_t*)p.q + q_base;
  const uint16_t* __restrict__ kg = (const uint16_t*)p.k + k_base;
  const uint16_t* __restrict__ vg = (const uint16_t*)p.v + v_base;

  // This lane's query row and its Q fragments Q[row][16*kk + 8*hi .. +7]:
  // wave w owns rows q0 + 32 w .. +31, so group 0 (waves 0-3) holds the
  // first 128 rows of the tile and group 1 the last 128.
  const int row = q0 + 32 * wave + l32;
  const int wrow0 = q0 + 32 * wave;  // the wave's first row
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
  // Dropout: this lane's row id, its index in the LSE layout.
  const uint64_t rid = (uint64_t)(lse_base + row);
  float m_run = -INFINITY;  // base-2 reference max of this lane's row
  float l_run = 0.f;        // this half-wave's share of the running fp32 sum of weights (LSE)
  // ... of the bf16-rounded weights P.V takes (normalises o), as four running
  // partial sums that each tile's v_dot2 chains extend in place.
  float lb4[4] = {0.f, 0.f, 0.f, 0.f};
  const float c = p.scale_log2;

  // DMA of one operand (K or V) of one tile into its LDS stage by the four
  // waves of one group; wave w covers rows 16(w%4) .. 16(w%4)+15.  Lane l of
  // instruction i writes the 16 bytes at LDS row (16(w%4) + i*RPI + l/CH),
  // physical chunk l%CH, so it fetches the logical chunk the swizzle maps
  // there.  The tile's base address is uniform (scalar registers); the
  // per-lane byte offsets within a tile are the same for every full tile
  // (the host keeps them below 2^31).  In a tile that runs past the last
  // key, rows past the end re-read the last key row: their weights are
  // exactly zero and their values finite.
  const int drow = lane / CH;
  const int dpch = lane % CH;
  const int wq = wave & 3;
  // Paged: wave w's rows 16(w%4) .. 16(w%4)+15 of a tile are exactly one
  // 16-token block, fetched from the pool block the table names; the lane
  // offsets are then relative to that block.
  static_assert(!PAGED || RPW == kFwdPagedBlock, "one pool block per wave and tile");
  const int64_t kv_row_k = PAGED ? p.p_ts : p.k_ss;
  const int64_t kv_row_v = PAGED ? p.p_ts : p.v_ss;
  uint32_t koff[IPW], voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int r = wq * RPW + i * RPI + drow;      // row of the tile in LDS
    const int rs = PAGED ? i * RPI + drow : r;    // ... in the source
    koff[i] = (uint32_t)(((int64_t)rs * kv_row_k + swz_k(CH, r, dpch) * 8) * 2);
    voff[i] = (uint32_t)(((int64_t)rs * kv_row_v + swz_v(CH, r, dpch) * 8) * 2);
  }
  // Paged: the wave's block of tile `tile` (a block past the last key is
  // replaced by the last key's block).
  auto wave_block = [&](int tile) {
    return __builtin_amdgcn_readfirstlane(min(tile * (BC / kFwdPagedBlock) + wq, (nk - 1) / kFwdPagedBlock));
  };
  // Its pool block, read from the table through the scalar cache (the table
  // is constant during the launch; a vector load would be counted with the
  // DMA loads in flight and waiting for it would drain them).
  const __attribute__((address_space(4))) int32_t* table =
      (const __attribute__((address_space(4))) int32_t*)(p.block_table + (PAGED ? (int64_t)b * p.max_blocks : 0));
  auto pool_block = [&](int tile) -> int32_t {
    if (!PAGED || tile < 0) return 0;
    return table[wave_block(tile)];
  };
  // Instruction i of this wave's share of operand V_OP (K when false) of a
  // tile; PHYS is pool_block(tile) when paged.
  auto dma_one = [&](int tile, bool v_op, int i, int32_t phys) {
    const int st = tile % kStages;
    const int r0 = wq * RPW + i * RPI;
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)((v_op ? &v_s[st][0] : &k_s[st][0]) + r0 * D));
    const int rows_left = nk - tile * BC;  // uniform
    const uint16_t* base = PAGED ? (v_op ? vg : kg) + (int64_t)phys * p.p_bs
                                 : (v_op ? vg + (int64_t)tile * BC * p.v_ss : kg + (int64_t)tile * BC * p.k_ss);
    // A full tile takes the precomputed offsets as they are (the load of
    // each branch is issued there, so no offset is copied in the common
    // case).  In the last tile rows past the last key re-read that key (in
    // the last key's block when paged).
    if (rows_left >= BC) {
      dma_16b(base, v_op ? voff[i] : koff[i], lds);
    } else {
      const int r = r0 + drow;
      const int64_t row_stride = PAGED ? p.p_ts : (v_op ? p.v_ss : p.k_ss);
      const int rk = PAGED ? tile * BC + min(r, rows_left - 1) - wave_block(tile) * kFwdPagedBlock
                           : min(r, rows_left - 1);
      const uint32_t off = (uint32_t)(((int64_t)rk * row_stride +
                                       (v_op ? swz_v(CH, r, dpch) : swz_k(CH, r, dpch)) * 8) * 2);
      dma_16b(base, off, lds);
    }
  };

  auto dma_op = [&](int tile, bool v_op) {
    const int32_t phys = pool_block(tile);
#pragma unroll
    for (int i = 0; i < IPW; ++i) dma_one(tile, v_op, i, phys);
  };

  // Group 0 loads the key tiles, group 1 the value tiles.  Tile 0 flies
  // while the Q fragments arrive.
  const bool v_loader = grp != 0;
  if (nt > 0) dma_op(0, v_loader);

  f32x16 sacc[NKB];  // S^T of one tile: NKB 32-key blocks

  // Softmax of tile t in place (scores -> weights), producing the bf16 B
  // operands of the P.V product.
  bf16x8 pf[NKC];
  // Dropout bytes of the tile: dw[kc][0] holds the bytes of keys 16kc + 4hi
  // + 0..3 of this lane's row, dw[kc][1] those of keys 16kc + 8 + 4hi + 0..3
  // (words hi and 2 + hi of the generator's output for the 16-key group kc).
  uint32_t dw[NKC][2];
  const uint32_t tm1 = DROP ? (uint32_t)(p.drop_t - 1) * 0x00010001u : 0u;
  // When a softmax moves the reference, o and l are rescaled by alpha right
  // there, in the vector-ALU phase (o was last written by the P.V products
  // of the MFMA phase before it).
  // Weights p = 2^(s*c - m) of the tile for reference m: packed into the
  // bf16 B operands pf of the P.V product; this lane's sum of the fp32
  // weights goes to ps, and the rounded ones (v_dot2 with (1, 1) on the
  // packed pairs, before any dropout) extend the running sums lb4 into pb4.
  const bf16x2 ones2 = __builtin_bit_cast(bf16x2, 0x3F803F80u);
  auto weights = [&](float m, float& ps, float (&pb4)[4]) {
    float ps4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pb4[q] = lb4[q];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int kb = kc >> 1;
      const int r0 = 8 * (kc & 1);
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pv[j] = exp2_fast(__builtin_fmaf(sacc[kb][r0 + j], c, -m));
        if (kc == 0 && j < 4)
          ps4[j] = pv[j];
        else
          ps4[j & 3] += pv[j];
      }
      uint4 pw;
      pw.x = pack_bf16x2(pv[0], pv[1]);
      pw.y = pack_bf16x2(pv[2], pv[3]);
      pw.z = pack_bf16x2(pv[4], pv[5]);
      pw.w = pack_bf16x2(pv[6], pv[7]);
      pb4[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.x), ones2, pb4[0], false);
      pb4[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.y), ones2, pb4[1], false);
      pb4[2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.z), ones2, pb4[2], false);
      pb4[3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.w), ones2, pb4[3], false);
      if (DROP) {
        // Dropped weights become zero in P.V only; the sum keeps them.
        pw.x &= keep_mask16<0>(dw[kc][0], tm1);
        pw.y &= keep_mask16<1>(dw[kc][0], tm1);
        pw.z &= keep_mask16<0>(dw[kc][1], tm1);
        pw.w &= keep_mask16<1>(dw[kc][1], tm1);
      }
      pf[kc] = __builtin_bit_cast(bf16x8, pw);
    }
    ps = (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
  };

  // Dropout bytes of tile t into dw.  Both halves of the wave hold the same
  // row: lane half hi draws the 16-key groups 2u + hi, and one swap across
  // the halves hands each lane the words it needs from the other half's draw
  // (lanes 0..31 keep words 0 and 2, lanes 32..63 words 1 and 3, of every
  // group).  A tile's draw runs in the MFMA phase before its softmax, where
  // the vector ALU is otherwise idle, and the softmax only applies it.
  auto draw = [&](int t) {
#pragma unroll
    for (int u = 0; u < NKC / 2; ++u) {
      const uint4 r = philox4x32_10(
          make_uint4((uint32_t)(NKC * t + 2 * u + hi), (uint32_t)rid, (uint32_t)(rid >> 32), p.drop_offset),
          p.drop_seed_lo, p.drop_seed_hi);
      const auto w01 = __builtin_amdgcn_permlane32_swap(r.x, r.y, false, false);
      const auto w23 = __builtin_amdgcn_permlane32_swap(r.z, r.w, false, false);
      dw[2 * u][0] = w01[0];
      dw[2 * u + 1][0] = w01[1];
      dw[2 * u][1] = w23[0];
      dw[2 * u + 1][1] = w23[1];
    }
  };

  auto softmax = [&](int t) {
    const int k0 = t * BC;
    const bool need_mask = (k0 + BC > nk) || (CAUSAL && k0 + BC - 1 > wrow0 + off);
    if (need_mask) {
      const int lim = CAUSAL ? row + off : nk - 1;
      const int kend = (nk - 1 < lim ? nk - 1 : lim) - k0 - 4 * hi;
      // One compare and one select per score (a key past kend is masked).
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = sacc[kb][r];
          sacc[kb][r] = kb * 32 + 8 * (r >> 2) + (r & 3) <= kend ? x : -INFINITY;
        }
    }
    // Fast path: weights against the current reference m_run, without the
    // tile's row max.  Every weight is at most this lane's partial sum, so a
    // partial sum <= kLazyBound bounds them all; a larger, infinite or NaN
    // sum (a large jump of the max, or no reference yet) sends the whole wave
    // to the exact step, which takes the row max, moves the reference and
    // recomputes the weights.
    float ps, pb4[4];
    weights(m_run, ps, pb4);
    if (__any(!(ps <= kLazyBound))) {
      float mx[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        mx[q] = fmaxf(sacc[q >> 1][8 * (q & 1)], sacc[q >> 1][8 * (q & 1) + 1]);
#pragma unroll
        for (int r = 2; r < 8; ++r) mx[q] = fmaxf(mx[q], sacc[q >> 1][8 * (q & 1) + r]);
      }
#pragma unroll
      for (int q = 4; q < NKC; ++q)
#pragma unroll
        for (int r = 0; r < 8; ++r) mx[q & 3] = fmaxf(mx[q & 3], sacc[q >> 1][8 * (q & 1) + r]);
      const float tmax = max_halves(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]))) * c;
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = m_new == -INFINITY ? 1.f : exp2_fast(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int q = 0; q < 4; ++q) lb4[q] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
      weights(m_new == -INFINITY ? 0.f : m_new, ps, pb4);
    }
    l_run += ps;
#pragma unroll
    for (int q = 0; q < 4; ++q) lb4[q] = pb4[q];
  };

  // The MFMA phase of tile t is one stream of products: the NPV products
  // O^T += V^T P^T of tile t, then (when tile t + 1 exists) the NSC score
  // products S^T = K Q^T of tile t + 1.  Product i's LDS operand reads are
  // issued kPre products ahead of it, and the reads of the first kPre
  // products (values of tile t, visible since two phases) are issued at the
  // end of the softmax phase before, so the phase opens on a product instead
  // of on the LDS latency, and no latency gap opens between the two halves.
  //
  // O^T += V^T P^T over four 16-key chunks of tile t.  Contraction slot j of
  // lane half hi is key 16*kc + 4*hi + j (j < 4) or 16*kc + 8 + 4*hi + (j-4):
  // exactly the keys the lane's score registers 8*(kc%2) .. +7 hold.  The two
  // transposed reads return those 8 keys for d = 32*db + l%32: lane (4k + q)
  // of each 16-lane group points at key row (base + k), dims
  // (16-block + 4q .. +3).  Score product j = 2 kk + kb reads key rows
  // 32 kb + l%32, head dims 16 kk + 8 hi .. +7 of tile t + 1.
  constexpr int NPV = NKC * (D / 32);
  constexpr int NSC = NKB * (D / 16);
  constexpr int kPre = 6;  // products whose operand reads are in flight ahead
  const int g16 = lane >> 4;
  const int tk = (lane >> 2) & 3;
  const int tq = lane & 3;
  uint4 opa[NPV + NSC];
  // Value reads: the swizzle of key rows 16 kc + 4 hi + tk (+ 8) depends on
  // tk only, so each 32-dim block db has one per-lane LDS address for stage
  // 0; chunk kc, the upper 8 keys and the stage add uniform offsets.
  uint32_t vbt[D / 32];  // value reads of the current tile's stage
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int dc = 4 * db + 2 * (g16 & 1) + (tq >> 1);  // logical 16-byte chunk
    const int ka = 4 * hi + tk;
    vbt[db] = (uint32_t)(uintptr_t)&v_s[0][0] + 2u * (uint32_t)(ka * D + swz_v(CH, ka, dc) * 8 + 4 * (tq & 1));
  }
  // Key reads: key row l32 (+32 for the second block, an immediate: the
  // swizzle of row r depends on r mod 32 only), chunk 2kk + hi.
  uint32_t kbt[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    kbt[kk] = (uint32_t)(uintptr_t)&k_s[0][0] + 2u * (uint32_t)(l32 * D + swz_k(CH, l32, 2 * kk + hi) * 8);
  // The per-lane bases follow the ring one stage per tile: tile j lives in
  // stage j % kStages.  Each wave moves its value bases once per tile (in the
  // prefetch) and its key bases once per tile read (in the MFMA phase), in
  // tile order, so a read adds only an immediate.
  auto stage_step = [&](int j) {  // byte step from the stage of tile j - 1 to that of tile j
    return (j % kStages == 0) ? (uint32_t)(-(int)(2 * (kStages - 1) * TILE)) : (uint32_t)(2 * TILE);
  };
  auto advance_v = [&](int t) {
    if (t > 0) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) vbt[db] += stage_step(t);
    }
  };
  auto advance_k = [&](int j) {
    if (j > 0) {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) kbt[kk] += stage_step(j);
    }
  };
  auto read_op = [&](int i, int t) {
    if (i < NPV) {
      const int kc = i / (D / 32), db = i % (D / 32);
      const uint32_t a = vbt[db] + 2u * (uint32_t)(16 * kc * D);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a);
      const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(a + 2u * 8u * D));
      const uint2 l2 = __builtin_bit_cast(uint2, lo);
      const uint2 u2 = __builtin_bit_cast(uint2, up);
      opa[i] = make_uint4(l2.x, l2.y, u2.x, u2.y);
    } else {
      const int kk = (i - NPV) / NKB, kb = (i - NPV) % NKB;
      const uint32_t a = kbt[kk] + 2u * (uint32_t)(kb * 32 * D);
      const u32x4_t v = *(const lds_u32x4*)(uintptr_t)a;
      opa[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
  };
  auto mfma_op = [&](int i) {
    if (i < NPV) {
      const int kc = i / (D / 32), db = i % (D / 32);
      oacc[db] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8, opa[i]), pf[kc], oacc[db]);
    } else {
      const int kk = (i - NPV) / NKB, kb = (i - NPV) % NKB;
      sacc[kb] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8, opa[i]), qf[kk], kk == 0 ? zero16() : sacc[kb]);
    }
  };
  // Reads of the first kPre products of tile t's phase, at the end of the
  // softmax phase before it (only the value tile, already visible, is read).
  auto prefetch = [&](int t) {
    advance_v(t);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kPre; ++i) read_op(i, t);
    __builtin_amdgcn_sched_barrier(0);
  };
  // The products of tile t (and the scores of tile t + 1 when NEXT).  When
  // dma_tile >= 0, this wave's share of that tile's operand (values for
  // group 1, keys for group 0) is issued along the way, one LDS-DMA
  // instruction after every N / IPW products: the CU's vector-memory path
  // takes a 1 KB instruction every ~16 cycles, so an instruction may wait
  // to issue while the matrix pipe works through the product before it.
  auto mfma_phase = [&](int t, auto next, int dma_tile, int32_t dma_phys) {
    constexpr int N = decltype(next)::value ? NPV + NSC : NPV;
    constexpr int DSTEP = N / IPW;
    if (decltype(next)::value) advance_k(t + 1);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      mfma_op(i);
      if (i + kPre < N) read_op(i + kPre, t);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + kPre < NPV)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two transposed value reads
      else if (i + kPre < N)
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one key read
      if (i % DSTEP == DSTEP / 2 && dma_tile >= 0) dma_one(dma_tile, v_loader, i / DSTEP, dma_phys);
    }
  };
  // The scores of tile 0 (the first MFMA phase), kPre reads ahead.
  auto scores0 = [&]() {
#pragma unroll
    for (int i = NPV; i < NPV + NSC; ++i) {
      if (i == NPV) {
#pragma unroll
        for (int j = 0; j < kPre; ++j) read_op(NPV + j, -1);
      }
      mfma_op(i);
      if (i + kPre < NPV + NSC) read_op(i + kPre, -1);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
    for (int i = NPV; i < NPV + NSC; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + kPre < NPV + NSC) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  const std::integral_constant<bool, true> with_next{};
  const std::integral_constant<bool, false> last{};

  // Phase schedule.  Global phases P = 0 .. 2*nt + 1, each ended by a
  // workgroup barrier.  Group 0 runs the scores of tile 0 in phase 0, then
  // for each tile t the softmax of tile t in phase 2t + 1 (closing with the
  // prefetch of tile t's first value operands) and the MFMA phase of tile t
  // (P.V of tile t, scores of tile t + 1) in phase 2t + 2; group 1 runs the
  // same sequence one phase later.  So K of tile t is read in phases 2t and
  // 2t + 1, V of tile t in phases 2t + 1 .. 2t + 3.
  //
  // Loads into stage t % 4, from the group in its MFMA phase (whose matrix
  // pipe hides the issue cost): K of tile t + 4 by group 0 in phase 2t + 2
  // (K of tile t was last read in phase 2t + 1), V of tile t + 3 by group 1
  // in phase 2t + 3 (V of tile t - 1 was last read in phase 2t + 1).  The
  // prologue loads K of tiles 0 .. 3 and V of tiles 0 .. 2.  At the end of odd
  // phase 2s - 1 each wave waits for its share of tile s, which group 0 reads
  // next: of its own later loads, K of tiles s + 1 and s + 2 (group 0) or V
  // of tile s + 1 (group 1) may still be in flight.  The two groups' loops
  // are written out separately so every phase is straight-line code.
  auto wait_tiles_in_flight = [&](int n) {  // n later tiles of this wave may fly
    if (n <= 0)
      wait_vmcnt<0>();
    else if (n == 1)
      wait_vmcnt<IPW>();
    else
      wait_vmcnt<2 * IPW>();
  };
  auto phase_end = [&](int P) {
    if (P & 1) {
      const int s_need = (P + 1) / 2;
      if (s_need < nt) {
        const int last_issued = v_loader ? min(s_need + 1, nt - 1) : min(s_need + 2, nt - 1);
        wait_tiles_in_flight(last_issued - s_need);
      }
    }
    lds_barrier();
  };
  if (nt > 0) {
    // The Q loads were issued before tile 0's DMA (the DMA asm is a memory
    // barrier for the compiler); wait for both, then let the next tiles fly.
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(qf[kk]));
    wait_vmcnt<0>();
    for (int j = 1; j < (v_loader ? 3 : 4) && j < nt; ++j) dma_op(j, v_loader);
    lds_barrier();
    // Paged: the table entry for the next MFMA phase's DMA is read through
    // the scalar cache at the start of the softmax phase before it, when no
    // LDS read is pending (both count on the same counter), and is waited
    // for before that phase's prefetch reads are issued.
    auto table_entry = [&](int tile) {
      const int32_t e = pool_block(tile);
      return e;
    };
    auto settle = [&](int32_t& e) {
      if (PAGED) asm volatile("" : "+s"(e));
    };
    // The last tile's MFMA phase has no scores of a next tile; it is peeled
    // off the loop so that the loop body is one straight stream.
    if (grp == 0) {
      scores0();
      if (DROP) draw(0);
      phase_end(0);
      for (int t = 0; t < nt0 - 1; ++t) {
        int32_t ph = table_entry(t + 4 < nt ? t + 4 : -1);
        softmax(t);
        settle(ph);
        prefetch(t);
        phase_end(2 * t + 1);
        __builtin_amdgcn_s_setprio(1);
        if (DROP) draw(t + 1);
        mfma_phase(t, with_next, t + 4 < nt ? t + 4 : -1, ph);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        phase_end(2 * t + 2);
      }
      softmax(nt0 - 1);
      prefetch(nt0 - 1);
      phase_end(2 * nt0 - 1);
      __builtin_amdgcn_s_setprio(1);
      mfma_phase(nt0 - 1, last, -1, 0);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      phase_end(2 * nt0);
      for (int P = 2 * nt0 + 1; P <= 2 * nt + 1; ++P) phase_end(P);
    } else if (q0 + kBr / 2 >= nq) {
      // No row of group 1 exists in this tile (the last, ragged tile of a
      // sequence): it only loads its value tiles, three ahead in what would
      // be its MFMA phases, and keeps to the barriers and its load waits
      // while group 0 computes alone.
      phase_end(0);
      phase_end(1);
      for (int t = 0; t < nt; ++t) {
        phase_end(2 * t + 2);
        if (t + 3 < nt) dma_op(t + 3, true);
        phase_end(2 * t + 3);
      }
    } else {
      phase_end(0);
      scores0();
      if (DROP) draw(0);
      phase_end(1);
      for (int t = 0; t < nt - 1; ++t) {
        int32_t ph = table_entry(t + 3 < nt ? t + 3 : -1);
        softmax(t);
        settle(ph);
        prefetch(t);
        phase_end(2 * t + 2);
        __builtin_amdgcn_s_setprio(1);
        if (DROP) draw(t + 1);
        mfma_phase(t, with_next, t + 3 < nt ? t + 3 : -1, ph);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        phase_end(2 * t + 3);
      }
      softmax(nt - 1);
      prefetch(nt - 1);
      phase_end(2 * nt);
      __builtin_amdgcn_s_setprio(1);
      mfma_phase(nt - 1, last, -1, 0);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      phase_end(2 * nt + 1);
    }
  }

  // Epilogue: O = o / lb with lb the sum of the bf16-rounded weights P.V
  // took, so each row is a convex combination of value rows up to fp32
  // rounding (dividing by the fp32 sum instead would carry the rounding of
  // a dominant weight, up to 2^-9 relative, into O); LSE = (m + log2 l) *
  // ln 2 with the fp32 sum l.
  const float l_tot = sum_halves(l_run);
  const float lb_tot = sum_halves((lb4[0] + lb4[1]) + (lb4[2] + lb4[3]));
  const float inv = (lb_tot > 0.f ? 1.f / lb_tot : 0.f) * (DROP ? p.drop_scale : 1.f);
  // The wave's 32 output rows go through LDS (the tile ring is idle: every
  // tile has been consumed behind the last barrier) so that global stores
  // write whole rows, 16 bytes per lane, instead of 8-byte pieces of 64
  // rows.  Staging rows are 16-byte-chunk swizzled like the key tiles.
  uint16_t* stage = &k_s[0][0] + wave * (32 * D);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      uint2 st;
      st.x = pack_bf16x2(oacc[db][4 * gq + 0] * inv, oacc[db][4 * gq + 1] * inv);
      st.y = pack_bf16x2(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv);
      *(uint2*)&stage[l32 * D + ((4 * db + gq) ^ (l32 & (CH - 1))) * 8 + 4 * hi] = st;
    }
  constexpr int RPS = 64 / CH;  // rows per store instruction
  uint16_t* __restrict__ og = (uint16_t*)p.o + o_base;
#pragma unroll
  for (int s = 0; s < 32 / RPS; ++s) {
    const int r = s * RPS + lane / CH;
    const int cc = lane % CH;
    const uint4 v = *(const uint4*)&stage[r * D + (cc ^ (r & (CH - 1))) * 8];
    const int orow = q0 + 32 * wave + r;
    if (orow < nq) *(uint4*)(og + (int64_t)orow * p.o_ss + cc * 8) = v;
  }
  if (row < nq && p.lse && hi == 0)
    p.lse[lse_base + row] = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : -INFINITY;
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const int64_t nwg = (int64_t)p.num_qtiles * p.heads_q * p.batch;
  if (p.paged)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, true, false>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                       p);
  else if (p.drop_t > 0)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, false, true>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                       p);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, false, false>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                       p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
  if (head_dim == 64) return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  if (head_dim == 256) return launch_fwd_bf16_d256(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
