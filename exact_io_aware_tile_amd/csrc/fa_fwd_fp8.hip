// fa_fwd_fp8.hip -- FP8 (E4M3) prefill attention on gfx950, head_dim 128.
//
// Method: the same online-softmax recurrence as the bf16 prefill ("S12
// FlashAttention", llminference.xinbetween.com, "Core idea / The solution"
// and "Mechanics / How it works"), with the FP8 inputs that section
// "Production notes / In production" credits to FlashAttention-3.  Q, K and V
// are E4M3 codes standing for descale * value(code), one descale factor per
// tensor; both products run on the FP8 matrix cores with fp32 accumulation.
//
// gfx950 mapping (the bf16 kernel's pipeline, with FP8 operands)
//   * one workgroup per CU: 8 waves (2 per SIMD) x 32 query rows = 256 rows
//     of one (sequence, head); wave w owns rows q0 + 32 w .. +31, and under a
//     causal mask the first four waves stop two tiles before the last four.
//   * 64-key tiles of K and V (8 KB each: 64 rows of 128 bytes) go from
//     global memory straight into LDS (global_load_lds) through a 4-stage
//     ring, 16-byte chunks XOR-swizzled per row pair so that both the score
//     operand reads and the transposed value reads spread over the banks.
//   * scores S^T = K Q^T on v_mfma_scale_f32_32x32x64_f8f6f4 (unit block
//     scales): lane l supplies key (or query) l % 32 and the 32 head-dim
//     bytes 64 kk + 32 (l / 32) .. +31; the product only pairs equal
//     contraction slots of the two operands, so any slot numbering shared by
//     both works.  Scores come out one query row per lane, as in bf16.
//   * the weights are rounded to E4M3 (v_cvt_pk_fp8_f32, nearest-even) into
//     the B operand of O^T += V^T P^T, slot j of lane half h holding the key
//     of score register j (key 32 (j/16) + 8 ((j%16)/4) + 4 h + j % 4); the
//     V^T operand is read with ds_read_b64_tr_b8, which hands lane i of each
//     16-lane group byte i % 8 of the 8-byte rows 2b + i / 8 (b = 0..7):
//     rows 2b and 2b+1 address the same key, head-dim bytes 8 apart.
//   * O is normalised by the sum of the rounded weights, which one more
//     MFMA per tile accumulates (all-ones A operand), so O is an exact
//     convex combination of V rows under the weights P.V used; LSE uses the
//     fp32 sum of the unrounded weights.
//   * the lazy correction bounds every weight by 2^8 (E4M3 reaches 448).
//   * base-2 scores with scale * log2(e) * q_descale * k_descale folded into
//     one constant; O is multiplied by v_descale / sum in the epilogue.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int D = 128;             // head dim = bytes per K/V row
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;   // query rows per workgroup
static_assert(kBr == kFwdRowsPerTileFp8, "host tiling must match");
constexpr int kBc = 64;            // keys per tile
constexpr int kStages = 4;         // LDS ring depth
constexpr int CH = D / 16;         // 16-byte chunks per row (8)
constexpr float kLazyBound = 256.f;  // largest weight (2^8) formed against a stale reference
constexpr uint32_t kOnesE4M3 = 0x38383838u;  // four E4M3 1.0

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

// D(32x32 fp32) += A(32x64 E4M3) * B(64x32 E4M3), unit block scales.
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Physical 16-byte chunk of logical chunk c in row r (128-byte rows): rows
// r and r + 2 land in different chunks, so 8 consecutive same-parity rows
// cover all 8 chunk positions.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// Four weights -> four E4M3 bytes (nearest-even), a first.
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  // The first conversion writes the low half of a's register in place (its
  // upper half, a's old bits, is overwritten by the second), so no register
  // is cleared for it.
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

template <bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(kThreads) void fwd_fp8_kernel(const FwdParams p) {
  constexpr int TILE = kBc * D;          // bytes per K or V tile
  constexpr int RPI = 1024 / D;          // rows per 1 KB DMA instruction (8)
  constexpr int RPW = kBc / 4;           // rows per wave when one group loads an operand (16)
  constexpr int IPW = RPW / RPI;         // DMA instructions per wave per operand of a tile (2)
  static_assert(IPW == 2, "DMA split");
  __shared__ __attribute__((aligned(1024))) uint8_t k_s[kStages][TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t v_s[kStages][TILE];

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
    nq = nk = p.cu_seqlens[b + 1] - s0;
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

  // Key tiles the workgroup streams; under a causal mask the first 128 rows
  // (group 0) need only the first nt0 of them (as in the bf16 prefill; nt0 >=
  // nt - 3, so group 0 has issued every key load by the time it stops).
  int nt = (nk + kBc - 1) / kBc;
  int nt0 = nt;
  if (CAUSAL) {
    const int last = q0 + kBr - 1 + off;
    const int lim = last < 0 ? 0 : last / kBc + 1;
    nt = nt < lim ? nt : lim;
    const int last0 = q0 + kBr / 2 - 1 + off;
    const int lim0 = last0 < 0 ? 0 : last0 / kBc + 1;
    nt0 = max(min(nt, lim0), max(nt - 3, 1));
  }

  const uint8_t* __restrict__ qg = (const uint8_t*)p.q + q_base;
  const uint8_t* __restrict__ kg = (const uint8_t*)p.k + k_base;
  const uint8_t* __restrict__ vg = (const uint8_t*)p.v + v_base;

  // This lane's query row and its Q fragments: qf[kk] = Q[row][64 kk + 32 hi
  // .. +31]; wave w owns rows q0 + 32 w .. +31.  A row past the end (never
  // stored) reads the last valid row.
  const int row = q0 + 32 * wave + l32;
  const int wrow0 = q0 + 32 * wave;
  i32x8 qf[2];
  {
    const uint8_t* qr = qg + (int64_t)min(row, nq - 1) * p.q_ss + 32 * hi;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint4 lo = *(const uint4*)(qr + 64 * kk);
      const uint4 up = *(const uint4*)(qr + 64 * kk + 16);
      qf[kk] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)up.x, (int)up.y, (int)up.z, (int)up.w};
    }
  }
  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = zero16();
  f32x16 lsum = zero16();   // every register: the sum of this row's rounded weights
  i32x8 ones = {(int)kOnesE4M3, (int)kOnesE4M3, (int)kOnesE4M3, (int)kOnesE4M3,
                (int)kOnesE4M3, (int)kOnesE4M3, (int)kOnesE4M3, (int)kOnesE4M3};
  asm volatile("" : "+v"(ones));  // opaque: kept in registers, not rebuilt every tile
  float m_run = -INFINITY;  // base-2 reference max of this lane's row
  float l_run = 0.f;        // this half-wave's share of the fp32 sum of weights
  const float c = p.scale_log2;

  // DMA of one operand of one tile by the four waves of one group; wave w
  // covers rows 16(w%4) .. +15, two 1 KB instructions of 8 rows.  Lane l of
  // instruction i writes LDS row 16(w%4) + 8i + l/8, physical chunk l%8, so it
  // fetches the logical chunk the swizzle maps there.  Rows past the last
  // key re-read the last key row (their weights are exactly zero).
  const int drow = lane / CH;
  const int dpch = lane % CH;
  const int wq = wave & 3;
  // Paged (an FP8 KV cache): wave w's 16 rows of a tile are exactly one
  // 16-token pool block, fetched from the block the table names, as in the
  // bf16 paged instance; the lane offsets are then relative to that block.
  static_assert(!PAGED || RPW == kFwdPagedBlock, "one pool block per wave and tile");
  const int64_t kv_row_k = PAGED ? p.p_ts : p.k_ss;
  const int64_t kv_row_v = PAGED ? p.p_ts : p.v_ss;
  uint32_t koff[IPW], voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int r = wq * RPW + i * RPI + drow;
    const int rs = PAGED ? i * RPI + drow : r;
    koff[i] = (uint32_t)((int64_t)rs * kv_row_k + swz(r, dpch) * 16);
    voff[i] = (uint32_t)((int64_t)rs * kv_row_v + swz(r, dpch) * 16);
  }
  auto wave_block = [&](int tile) {
    return __builtin_amdgcn_readfirstlane(min(tile * (kBc / kFwdPagedBlock) + wq, (nk - 1) / kFwdPagedBlock));
  };
  const __attribute__((address_space(4))) int32_t* table =
      (const __attribute__((address_space(4))) int32_t*)(p.block_table + (PAGED ? (int64_t)b * p.max_blocks : 0));
  auto pool_block = [&](int tile) -> int32_t {
    if (!PAGED || tile < 0) return 0;
    return table[wave_block(tile)];
  };
  auto dma_one = [&](int tile, bool v_op, int i, int32_t phys) {
    const int st = tile % kStages;
    const int r0 = wq * RPW + i * RPI;
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)((v_op ? &v_s[st][0] : &k_s[st][0]) + r0 * D));
    const int rows_left = nk - tile * kBc;  // uniform
    const uint8_t* base = PAGED ? (v_op ? vg : kg) + (int64_t)phys * p.p_bs
                                : (v_op ? vg + (int64_t)tile * kBc * p.v_ss : kg + (int64_t)tile * kBc * p.k_ss);
    // A full tile takes the precomputed offsets as they are (each branch
    // issues its own load, so no offset is copied in the common case); in
    // the last tile rows past the last key re-read that key (in the last
    // key's block when paged).
    if (rows_left >= kBc) {
      dma_16b(base, v_op ? voff[i] : koff[i], lds);
    } else {
      const int r = r0 + drow;
      const int64_t row_stride = PAGED ? p.p_ts : (v_op ? p.v_ss : p.k_ss);
      const int rk = PAGED ? tile * kBc + min(r, rows_left - 1) - wave_block(tile) * kFwdPagedBlock
                           : min(r, rows_left - 1);
      dma_16b(base, (uint32_t)((int64_t)rk * row_stride + swz(r, dpch) * 16), lds);
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

  // Scores of one tile: two 32-key blocks, two 64-byte halves of the head dim.
  f32x16 sacc[2];
  // Per-lane LDS operand addresses in stage 0, moved one stage per tile
  // (tile j lives in stage j % kStages) by the wave that reads them, in tile
  // order, so each read adds only an immediate.  Keys: row l32 (+32 rows
  // for the second block: the swizzle of row r depends on r mod 32 only),
  // chunk 4kk + 2hi + u.  Values: key rows tkey (+16 q rows), chunk
  // 2db + tchunk.
  uint32_t kaddr[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      kaddr[kk][u] = (uint32_t)(uintptr_t)&k_s[0][0] + (uint32_t)(l32 * D + swz(l32, 4 * kk + 2 * hi + u) * 16);
  auto stage_step = [&](int t) {  // bytes from the stage of tile t - 1 to that of tile t
    return (t % kStages == 0) ? (uint32_t)(-(int)((kStages - 1) * TILE)) : (uint32_t)TILE;
  };
  auto scores = [&](int t) {
    if (t > 0) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int u = 0; u < 2; ++u) kaddr[kk][u] += stage_step(t);
    }
    uint4 a[2][2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x4_t v = *(const lds_u32x4*)(uintptr_t)(kaddr[kk][u] + (uint32_t)(32 * kb * D));
          a[kk][kb][u] = make_uint4(v.x, v.y, v.z, v.w);
        }
      }
    sacc[0] = zero16();
    sacc[1] = zero16();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint4 lo = a[kk][kb][0], up = a[kk][kb][1];
        const i32x8 av = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)up.x, (int)up.y, (int)up.z, (int)up.w};
        sacc[kb] = mfma_fp8(av, qf[kk], sacc[kb]);
      }
  };

  // Softmax of tile t in place, producing the E4M3 B operand pf of P.V.
  i32x8 pf;
  bool corr = false;
  float alpha = 1.f;
  auto weights = [&](float m, float& ps) {
    float ps4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int kb = kc >> 1;
      const int r0 = 8 * (kc & 1);
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pv[j] = exp2_fast(__builtin_fmaf(sacc[kb][r0 + j], c, -m));
        ps4[j & 3] += pv[j];
      }
      // score registers 16 kb + r0 .. +7 are contraction slots 8 kc .. +7
      pf[2 * kc] = pack_fp8x4(pv[0], pv[1], pv[2], pv[3]);
      pf[2 * kc + 1] = pack_fp8x4(pv[4], pv[5], pv[6], pv[7]);
    }
    ps = (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
  };

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
    // Weights against the current reference; a lane sum above 2^8 (or not
    // finite) sends the wave to the exact step (see the bf16 kernel).
    float ps;
    weights(m_run, ps);
    corr = __any(!(ps <= kLazyBound));
    if (corr) {
      float mx[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        mx[q] = fmaxf(sacc[q >> 1][8 * (q & 1)], sacc[q >> 1][8 * (q & 1) + 1]);
#pragma unroll
        for (int r = 2; r < 8; ++r) mx[q] = fmaxf(mx[q], sacc[q >> 1][8 * (q & 1) + r]);
      }
      const float tmax = max_halves(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]))) * c;
      const float m_new = fmaxf(m_run, tmax);
      alpha = m_new == -INFINITY ? 1.f : exp2_fast(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      weights(m_new == -INFINITY ? 0.f : m_new, ps);
    }
    l_run += ps;
  };

  // O^T += V^T P^T for tile t, and the sum of the rounded weights.  Read q
  // (q = 0..3) of the V^T operand fills contraction slots 8q .. 8q+7: in the
  // 16-lane group gg of lane l, lane 16 gg + r addresses key 16q + 8 (r/8) +
  // 4 hi + (r/2) % 4 at head-dim bytes 32 db + 16 (gg % 2) + 8 (r % 2).
  const int gg = lane >> 4;
  const int rr = lane & 15;
  const int tkey = 8 * (rr >> 3) + 4 * hi + ((rr >> 1) & 3);  // + 16 q
  const int tchunk = gg & 1;                                     // + 2 db
  const int tbyte = 8 * (rr & 1);
  uint32_t vaddr[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
    vaddr[db] = (uint32_t)(uintptr_t)&v_s[0][0] + (uint32_t)(tkey * D + swz(tkey, 2 * db + tchunk) * 16 + tbyte);
  auto pv = [&](int t, int dma_tile, int32_t dma_phys) {
    if (t > 0) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) vaddr[db] += stage_step(t);
    }
    if (corr) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      lsum[0] *= alpha;  // the only register of lsum that is read
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      i32x2 pieces[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        pieces[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(uintptr_t)(vaddr[db] + (uint32_t)(16 * q * D)));
      const i32x8 av = {pieces[0][0], pieces[0][1], pieces[1][0], pieces[1][1],
                        pieces[2][0], pieces[2][1], pieces[3][0], pieces[3][1]};
      oacc[db] = mfma_fp8(av, pf, oacc[db]);
      if (db == 1 && dma_tile >= 0) {
        __builtin_amdgcn_sched_barrier(0);
        dma_one(dma_tile, v_loader, 1, dma_phys);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lsum = mfma_fp8(ones, pf, lsum);
  };
  // The MFMA phase of tile t: the scores of tile t + 1 (when it exists), then
  // P.V of tile t.  When dma_tile >= 0, this wave's two LDS-DMA instructions
  // for that tile's operand (keys for group 0, values for group 1) go out
  // between the products, where the matrix pipe hides their issue.
  auto mfma_phase = [&](int t, int dma_tile, int32_t dma_phys, int ntg) {
    if (t + 1 < ntg) scores(t + 1);
    if (dma_tile >= 0) {
      __builtin_amdgcn_sched_barrier(0);
      dma_one(dma_tile, v_loader, 0, dma_phys);
      __builtin_amdgcn_sched_barrier(0);
    }
    pv(t, dma_tile, dma_phys);
  };

  // Phase schedule (as in the bf16 prefill): global phases P = 0 .. 2 nt + 1,
  // each ended by a workgroup barrier.  Group 0 runs the scores of tile 0 in
  // phase 0, the softmax of tile t in phase 2t + 1 and the MFMA phase of tile
  // t (scores of t + 1, P.V of t) in phase 2t + 2; group 1 runs the same one
  // phase later.  So K of tile t is read in phases 2t and 2t + 1, V of tile t
  // in phases 2t + 2 and 2t + 3.
  //
  // Loads into stage t % 4 from the MFMA phases: K of tile t + 3 by group 0
  // in phase 2t + 2 (K of tile t - 1, in that stage, was last read in phase
  // 2t - 1), V of tile t + 3 by group 1 in phase 2t + 3 (V of tile t - 1 was
  // last read in phase 2t + 1).  The prologue loads tiles 0 .. 2 of each
  // operand.  At the end of odd phase 2s - 1 each wave waits for its share of
  // tile s (read from phase 2s on); of its later loads, tile s + 1 may still
  // be in flight.
  auto phase_end = [&](int P) {
    if (P & 1) {
      const int s_need = (P + 1) / 2;
      if (s_need < nt) {
        if (s_need + 1 < nt)
          wait_vmcnt<IPW>();
        else
          wait_vmcnt<0>();
      }
    }
    lds_barrier();
  };
  if (nt > 0) {
    // The Q loads were issued before tile 0's DMA; wait for both, then let
    // the next tiles fly.
    asm volatile("" : "+v"(qf[0]), "+v"(qf[1]));
    wait_vmcnt<0>();
    for (int j = 1; j < 3 && j < nt; ++j) dma_op(j, v_loader);
    lds_barrier();
    // Paged: the table entry for the next MFMA phase's DMA is read through
    // the scalar cache at the start of the softmax phase before it (no LDS
    // read is pending there: both count on one counter) and waited for at its
    // end.
    auto settle = [&](int32_t& e) {
      if (PAGED) asm volatile("" : "+s"(e));
    };
    if (grp == 0) {
      scores(0);
      phase_end(0);
      for (int t = 0; t < nt0; ++t) {
        const int dt = t + 3 < nt ? t + 3 : -1;
        int32_t ph = pool_block(dt);
        softmax(t);
        settle(ph);
        phase_end(2 * t + 1);
        __builtin_amdgcn_s_setprio(1);
        mfma_phase(t, dt, ph, nt0);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        phase_end(2 * t + 2);
      }
      // past its last tile: the barriers and load waits only, while group 1
      // finishes alone
      for (int P = 2 * nt0 + 1; P <= 2 * nt + 1; ++P) phase_end(P);
    } else {
      phase_end(0);
      scores(0);
      phase_end(1);
      for (int t = 0; t < nt; ++t) {
        const int dt = t + 3 < nt ? t + 3 : -1;
        int32_t ph = pool_block(dt);
        softmax(t);
        settle(ph);
        phase_end(2 * t + 2);
        __builtin_amdgcn_s_setprio(1);
        mfma_phase(t, dt, ph, nt);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        phase_end(2 * t + 3);
      }
    }
  }

  // Epilogue: O = v_descale * o / (sum of the rounded weights), LSE = (m +
  // log2 l) * ln 2 with l the fp32 sum.  Rows go through LDS (the ring is
  // idle: waves 0-3 stage in the K stages, 4-7 in the V stages) so that
  // stores write whole 256-byte rows.
  const float l_tot = sum_halves(l_run);
  const float lhat = lsum[0];
  const float inv = lhat > 0.f ? p.o_scale / lhat : 0.f;
  uint16_t* stage = (uint16_t*)(grp == 0 ? &k_s[0][0] : &v_s[0][0]) + wq * (32 * D);
  constexpr int OCH = D / 8;  // 16-byte chunks of a bf16 output row (16)
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      uint2 st;
      st.x = pack_bf16x2(oacc[db][4 * gq + 0] * inv, oacc[db][4 * gq + 1] * inv);
      st.y = pack_bf16x2(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv);
      *(uint2*)&stage[l32 * D + ((4 * db + gq) ^ (l32 & (OCH - 1))) * 8 + 4 * hi] = st;
    }
  constexpr int RPS = 64 / OCH;  // rows per store instruction (4)
  uint16_t* __restrict__ og = (uint16_t*)p.o + o_base;
#pragma unroll
  for (int s = 0; s < 32 / RPS; ++s) {
    const int r = s * RPS + lane / OCH;
    const int cc = lane % OCH;
    const uint4 v = *(const uint4*)&stage[r * D + (cc ^ (r & (OCH - 1))) * 8];
    const int orow = q0 + 32 * wave + r;
    if (orow < nq) *(uint4*)(og + (int64_t)orow * p.o_ss + cc * 8) = v;
  }
  if (row < nq && p.lse && hi == 0)
    p.lse[lse_base + row] = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : -INFINITY;
}

template <bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const int64_t nwg = (int64_t)p.num_qtiles * p.heads_q * p.batch;
  if (p.paged)
    hipLaunchKernelGGL((fwd_fp8_kernel<CAUSAL, true>), dim3((unsigned)nwg), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<CAUSAL, false>), dim3((unsigned)nwg), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdParams& p, int head_dim, hipStream_t stream) {
  if (head_dim != D) return hipErrorInvalidValue;
  return p.causal ? launch<true>(p, stream) : launch<false>(p, stream);
}

}  // namespace fa
