// fa_fwd_bf16_d256.hip -- bf16 prefill attention at head_dim 256 on gfx950
// (dense and packed sequences, optional dropout; chunked prefill over a
// paged KV pool).
//
// Method: the online-softmax recurrence of "S12 FlashAttention"
// (llminference.xinbetween.com), "Core idea / The solution" and "Mechanics /
// How it works", with the loop order of "FlashAttention: The Algorithm That
// Beat the Memory Wall" (repo-explainer.com), "A Tile, a Register File, and a
// Trick Called Online Softmax"; a separate kernel for one head size, as that
// page's "Why Templates Matter Here" describes the kernel family.
//
// gfx950 mapping.  The pipeline of the head_dim 64 / 128 kernel (8 waves in
// two ping-pong groups, K/V tiles fetched by LDS DMA into a 4-stage ring,
// XCD-aware longest-first work order, lazy correction, output staged through
// LDS) with a smaller tile per wave:
//   * 16 query rows per wave, 128 per workgroup.  At head_dim 256 the Q
//     fragments and the output accumulator of 32 rows would take 192 of the
//     256 registers a wave has at two waves per SIMD; 16 rows take 96.
//   * scores S^T[16 keys x 16 rows] = K Q^T on v_mfma_f32_16x16x32_bf16: lane
//     l supplies key row l%16 and Q row l%16, head dims 32s + 8(l/16) .. +7;
//     the accumulator leaves lane l with keys 4(l/16) .. +3 of the block for
//     row l%16;
//   * O^T += V^T P^T also on v_mfma_f32_16x16x32_bf16 (16x16x16 runs at half
//     its rate), over both 16-key blocks of a tile: contraction slot
//     8(l/16) + e is key 4(l/16) + e of block 0 for e < 4 and key
//     4(l/16) + e - 4 of block 1 otherwise -- exactly the weights lane l holds
//     for row l%16, so they stay in their lanes; the matching V^T operand is
//     two ds_read_b64_tr_b16 reads (four keys of one head dim each);
//   * 32-key tiles: a K or V tile is 16 KB and the two 4-stage rings 128 KB;
//   * a row's 32 scores of a tile sit in the four lanes l%16 + 16g; the row
//     max (taken only when the reference must move) and the final sum reduce
//     over those four lanes;
//   * paged pools: a 32-key tile is two 16-token pool blocks and each wave of
//     the loading group covers 8 rows, half a block; only its DMA base
//     changes, to the pool block the table names ("S12 FlashAttention",
//     "What this unlocks beyond speed": tiles fetched through a block table).
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int D = 256;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 16;                // query rows per wave
constexpr int kBr = kRows * kWaves;      // query rows per workgroup
static_assert(kBr == kFwdRowsPerTileBf16D256, "host tiling must match");
constexpr int kBc = 32;                  // keys per tile
constexpr int kStages = 4;               // LDS ring depth
constexpr int CH = D / 8;                // 16-byte chunks per row
constexpr int TILE = kBc * D;            // elements per K or V tile
constexpr int RPI = 512 / D;             // rows per 1 KB DMA instruction
constexpr int RPW = kBc / 4;             // rows per wave when one group loads an operand
constexpr int IPW = RPW / RPI;           // DMA instructions per wave per operand of a tile
constexpr int kKAhead = 4;               // score-operand reads issued ahead of their MFMA
constexpr int kVAhead = 4;               // P.V operand reads issued ahead of their MFMA
constexpr float kLazyBound = 65536.f;    // largest weight (2^16) formed against a stale reference
static_assert(IPW == 4 && RPW % RPI == 0, "DMA split");

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// LDS swizzles of the 32 16-byte chunks of a row, for 64 banks of 4 bytes
// (chunk c of any row sits on banks 4(c mod 16) .. +3).  Key rows: the
// score-operand reads of a 16-lane group (16 consecutive rows, one logical
// chunk) get 16 distinct chunks mod 16.  Value rows: the transposed reads of
// a half-wave touch 8 consecutive rows, two adjacent chunks 2db and 2db + 1
// and both 8-byte halves of each; xor-ing bits 1..3 of the chunk with the
// row keeps bit 0 and gives the 16 (row, chunk) pairs distinct chunks mod 16.
__device__ __forceinline__ int swz_k(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int swz_v(int r, int c) { return c ^ (2 * (r & 7)); }

template <bool CAUSAL, bool PAGED, bool DROP>
__global__ __launch_bounds__(kThreads) void fwd_bf16_d256_kernel(const FwdParams p) {
  static_assert(!(PAGED && DROP), "dropout is built for dense and packed prefill");
  __shared__ __attribute__((aligned(1024))) uint16_t k_s[kStages][TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_s[kStages][TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: leads, 1: one phase behind
  const int lane = tid & 63;
  const int n = lane & 15;    // the lane's query row (product column)
  const int j = lane >> 4;    // its key group: keys 4j .. 4j+3 of each 16-key block

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
  const int off = nk - nq;  // causal: key i visible from row r iff i <= r + off

  // Key tiles the workgroup streams; under a causal mask the first 64 rows
  // (group 0) need only the first nt0 of them and then keep to the barriers
  // and their load waits while group 1 finishes alone.  Group 0 loads the
  // values two tiles ahead, so nt0 >= nt - 2 (which the 64-row offset of the
  // groups gives anyway) keeps every value load issued before it stops.
  int nt = (nk + kBc - 1) / kBc;
  int nt0 = nt;
  if (CAUSAL) {
    const int last = q0 + kBr - 1 + off;
    const int lim = last < 0 ? 0 : last / kBc + 1;
    nt = nt < lim ? nt : lim;
    const int last0 = q0 + kBr / 2 - 1 + off;
    const int lim0 = last0 < 0 ? 0 : last0 / kBc + 1;
    nt0 = max(min(nt, lim0), max(nt - 2, 1));
  }

  const uint16_t* __restrict__ qg = (const uint16_t*)p.q + q_base;
  const uint16_t* __restrict__ kg = (const uint16_t*)p.k + k_base;
  const uint16_t* __restrict__ vg = (const uint16_t*)p.v + v_base;

  // Wave w owns rows q0 + 16 w .. +15; lane l holds row q0 + 16 w + l%16.
  // Rows past the end read the last valid row (never stored).
  const int row = q0 + 16 * wave + n;
  const int wrow0 = q0 + 16 * wave;
  bf16x8 qf[D / 32];  // Q[row][32s + 8j .. +7]
  {
    const uint16_t* qr = qg + (int64_t)min(row, nq - 1) * p.q_ss + 8 * j;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qf[s] = __builtin_bit_cast(bf16x8, *(const uint4*)(qr + 32 * s));
  }
  f32x4 oacc[D / 16];  // O^T[16db + 4j + r][row]
#pragma unroll
  for (int i = 0; i < D / 16; ++i) oacc[i] = zero4();
  const uint64_t rid = (uint64_t)(lse_base + row);  // dropout row id (LSE layout)
  float m_run = -INFINITY;  // base-2 reference max of this lane's row
  float l_run = 0.f;        // this lane's share of the running fp32 sum of weights (LSE)
  float lb_run = 0.f;       // ... of the bf16-rounded weights P.V takes (normalises o)
  const float c = p.scale_log2;

  // DMA: wave w of the loading group covers rows 8(w%4) .. +7 of a tile,
  // four 1 KB instructions of two rows each; lane l writes row (.. + l/32),
  // physical chunk l%32, fetching the logical chunk the swizzle maps there.
  // In a tile past the last key, rows past the end re-read the last key row.
  const int drow = lane / CH;
  const int dpch = lane % CH;
  const int wq = wave & 3;
  // Paged: wave w's rows 8(w%4) .. +7 of a tile are half of pool block
  // 2t + (w%4)/2 (rows (w%4 odd) 8 .. 15 or 0 .. 7 of it); the lane offsets
  // are then relative to that block.
  const int64_t kv_row_k = PAGED ? p.p_ts : p.k_ss;
  const int64_t kv_row_v = PAGED ? p.p_ts : p.v_ss;
  uint32_t koff[IPW], voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int r = wq * RPW + i * RPI + drow;  // row of the tile in LDS
    const int rs = PAGED ? r & (kFwdPagedBlock - 1) : r;  // ... in the source
    koff[i] = (uint32_t)(((int64_t)rs * kv_row_k + swz_k(r, dpch) * 8) * 2);
    voff[i] = (uint32_t)(((int64_t)rs * kv_row_v + swz_v(r, dpch) * 8) * 2);
  }
  // Paged: the block holding the wave's rows of tile `tile` (a block past
  // the last key is replaced by the last key's block), and its pool block,
  // read through the scalar cache as in the head_dim 64 / 128 kernel.
  auto wave_block = [&](int tile) {
    return __builtin_amdgcn_readfirstlane(
        min(tile * (kBc / kFwdPagedBlock) + wq * RPW / kFwdPagedBlock, (nk - 1) / kFwdPagedBlock));
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
    const uint16_t* base = PAGED ? (v_op ? vg : kg) + (int64_t)phys * p.p_bs
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
      dma_16b(base, (uint32_t)(((int64_t)rk * row_stride + (v_op ? swz_v(r, dpch) : swz_k(r, dpch)) * 8) * 2), lds);
    }
  };

  auto dma_op = [&](int tile, bool v_op) {
    const int32_t phys = pool_block(tile);
#pragma unroll
    for (int i = 0; i < IPW; ++i) dma_one(tile, v_op, i, phys);
  };

  if (nt > 0) dma_op(0, grp != 0);

  // Per-lane LDS operand addresses in stage 0, moved one stage per tile
  // (tile j lives in stage j % kStages) by the wave that reads them, in tile
  // order, so each read adds only an immediate.  Keys: row n (+16 rows for
  // the second block), chunk 4s + j; the swizzle leaves bit 4 of the chunk,
  // so s and s + 4 differ by 16 chunks.  Values: rows 4j + tk (+16 rows),
  // chunk 2db + (tq >> 1), db and db + 8 likewise 16 chunks apart.
  uint32_t kaddr[4], vaddr[8];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    kaddr[s] = (uint32_t)(uintptr_t)&k_s[0][0] + 2u * (uint32_t)(n * D + swz_k(n, 4 * s + j) * 8);
  auto stage_step = [&](int t) {  // bytes from the stage of tile t - 1 to that of tile t
    return (t % kStages == 0) ? (uint32_t)(-(int)(2 * (kStages - 1) * TILE)) : (uint32_t)(2 * TILE);
  };

  // Scores of one tile: two 16-key blocks, sacc[kb][r] = S[key 16kb + 4j + r][row].
  f32x4 sacc[2];
  auto scores = [&](int t) {
    if (t > 0) {
#pragma unroll
      for (int s = 0; s < 4; ++s) kaddr[s] += stage_step(t);
    }
    sacc[0] = zero4();
    sacc[1] = zero4();
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t ad = kaddr[s & 3] + 2u * (uint32_t)(16 * (s >> 2) * 8 + 16 * kb * D);
        const u32x4_t av = *(const lds_u32x4*)(uintptr_t)ad;
        const uint4 a = make_uint4(av.x, av.y, av.z, av.w);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), qf[s], sacc[kb], 0, 0,
                                                           0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kKAhead, 0);
#pragma unroll
    for (int i = 0; i < D / 16 - kKAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kKAhead, 0);
  };

  // Weights p = 2^(s*c - m) of the tile as the bf16 B operands of P.V; this
  // lane's fp32 sum goes to ps.  DMA of the next tiles is spread over it.
  i16x4 pf[2];
  uint32_t dw[2];  // dropout bytes of keys 4j .. 4j+3 of each block (word j of its draw)
  const uint32_t tm1 = DROP ? (uint32_t)(p.drop_t - 1) * 0x00010001u : 0u;
  bool corr = false;
  float alpha = 1.f;
  const bf16x2 ones2 = __builtin_bit_cast(bf16x2, 0x3F803F80u);
  auto weights = [&](float m, float& ps, float& pb, int dma_tile, bool dma_v, int32_t dma_phys) {
    float ps2[2] = {0.f, 0.f};
    float pb2 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (dma_tile >= 0) {
        __builtin_amdgcn_sched_barrier(0);
        dma_one(dma_tile, dma_v, 2 * kb, dma_phys);
        dma_one(dma_tile, dma_v, 2 * kb + 1, dma_phys);
        __builtin_amdgcn_sched_barrier(0);
      }
      float pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[r] = exp2_fast(__builtin_fmaf(sacc[kb][r], c, -m));
        ps2[r & 1] += pv[r];
      }
      uint32_t w01 = pack_bf16x2(pv[0], pv[1]);
      uint32_t w23 = pack_bf16x2(pv[2], pv[3]);
      pb2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w01), ones2, pb2, false);
      pb2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w23), ones2, pb2, false);
      if (DROP) {
        w01 &= keep_mask16<0>(dw[kb], tm1);
        w23 &= keep_mask16<1>(dw[kb], tm1);
      }
      pf[kb] = __builtin_bit_cast(i16x4, make_uint2(w01, w23));
    }
    ps = ps2[0] + ps2[1];
    pb = pb2;
  };

  auto softmax = [&](int t, int dma_tile, bool dma_v, int32_t dma_phys) {
    const int k0 = t * kBc;
    const bool need_mask = (k0 + kBc > nk) || (CAUSAL && k0 + kBc - 1 > wrow0 + off);
    if (need_mask) {
      const int lim = CAUSAL ? row + off : nk - 1;
      const int kend = (nk - 1 < lim ? nk - 1 : lim) - k0 - 4 * j;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * kb + r > kend) sacc[kb][r] = -INFINITY;
    }
    if (DROP) {
      // The four lanes of a row need word j of the draws of both 16-key
      // blocks.  Lanes with j even draw block 0, j odd block 1; each keeps
      // word j of its own draw and hands word j ^ 1 to the lane 16 away,
      // which draws the other block and needs exactly that word.
      const int kb = j & 1;
      const uint4 r = philox4x32_10(
          make_uint4((uint32_t)(2 * t + kb), (uint32_t)rid, (uint32_t)(rid >> 32), p.drop_offset),
          p.drop_seed_lo, p.drop_seed_hi);
      const uint32_t mine = j == 0 ? r.x : j == 1 ? r.y : j == 2 ? r.z : r.w;
      const uint32_t send = j == 0 ? r.y : j == 1 ? r.x : j == 2 ? r.w : r.z;
      const uint32_t recv = (uint32_t)__shfl_xor((int)send, 16, 64);
      dw[0] = kb ? recv : mine;
      dw[1] = kb ? mine : recv;
    }
    // Fast path against the current reference (see the head_dim 64 / 128
    // kernel): a lane partial sum above the bound, infinite or NaN sends the
    // wave to the exact step.
    float ps, pb;
    weights(m_run, ps, pb, dma_tile, dma_v, dma_phys);
    corr = __any(!(ps <= kLazyBound));
    if (corr) {
      float mx = fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3]));
      mx = fmaxf(mx, fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      const float tmax = max_halves(mx) * c;
      const float m_new = fmaxf(m_run, tmax);
      alpha = m_new == -INFINITY ? 1.f : exp2_fast(m_run - m_new);
      l_run *= alpha;
      lb_run *= alpha;
      m_run = m_new;
      weights(m_new == -INFINITY ? 0.f : m_new, ps, pb, -1, false, 0);
    }
    l_run += ps;
    lb_run += pb;
  };

  // O^T += V^T P^T over both 16-key blocks of tile t in one product per
  // 16 head dims: lane 4k + q of group j reads key rows 4j + k (block 0)
  // and 16 + 4j + k (block 1), head dims 16db + 4q .. +3; each transposed
  // read leaves lane n with dim 16db + n of four keys of its block.
  const int tk = n >> 2;
  const int tq = n & 3;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const int va = 4 * j + tk;
    vaddr[d] = (uint32_t)(uintptr_t)&v_s[0][0] +
               2u * (uint32_t)(va * D + swz_v(va, 2 * d + (tq >> 1)) * 8 + 4 * (tq & 1));
  }
  auto pv = [&](int t) {
    if (t > 0) {
#pragma unroll
      for (int d = 0; d < 8; ++d) vaddr[d] += stage_step(t);
    }
    if (corr) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[db][r] *= alpha;
    }
    const uint2 p0 = __builtin_bit_cast(uint2, pf[0]);
    const uint2 p1 = __builtin_bit_cast(uint2, pf[1]);
    const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(p0.x, p0.y, p1.x, p1.y));
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const uint32_t ad = vaddr[db & 7] + 2u * (uint32_t)(16 * (db >> 3) * 8);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)ad);
      const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(ad + 2u * 16u * D));
      const uint2 l2 = __builtin_bit_cast(uint2, lo);
      const uint2 u2 = __builtin_bit_cast(uint2, up);
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, u2.x, u2.y)), pb, oacc[db], 0, 0, 0);
    }
    // Two transposed reads per MFMA; kVAhead MFMAs' worth in flight.
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVAhead, 0);
#pragma unroll
    for (int i = 0; i < D / 16 - kVAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kVAhead, 0);
  };

  // Phase schedule and loads: as in the head_dim 64 / 128 kernel (group 0
  // runs the MFMA phase of tile t in phase 2t and its softmax in 2t + 1,
  // group 1 one phase later; K of tile t is loaded in phase 2t - 4 by group
  // 1, V of tile t in phase 2t - 3 by group 0, into stage t % 4).
  auto phase_end = [&](int P) {
    if (P & 1) {
      const int t_need = (P + 1) / 2;
      if (t_need < nt) {
        if (t_need + 1 < nt)
          wait_vmcnt<IPW>();
        else
          wait_vmcnt<0>();
      }
    }
    lds_barrier();
  };
  if (nt > 0) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) asm volatile("" : "+v"(qf[s]));
    wait_vmcnt<0>();
    if (nt > 1) dma_op(1, grp != 0);
    lds_barrier();
    // Paged: the table entry for the DMA of the next softmax phase is read
    // at the end of the MFMA phase before it (see the head_dim 64 / 128
    // kernel).
    if (grp == 0) {
      scores(0);
      int32_t ph = pool_block(2 < nt ? 2 : -1);
      phase_end(0);
      for (int t = 0; t < nt0; ++t) {
        softmax(t, t + 2 < nt ? t + 2 : -1, true, ph);
        phase_end(2 * t + 1);
        __builtin_amdgcn_s_setprio(1);
        if (t + 1 < nt0) scores(t + 1);
        pv(t);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        ph = pool_block(t + 3 < nt ? t + 3 : -1);
        phase_end(2 * t + 2);
      }
      for (int P = 2 * nt0 + 1; P <= 2 * nt + 1; ++P) phase_end(P);
    } else {
      if (2 < nt) dma_op(2, false);
      int32_t ph = pool_block(3 < nt ? 3 : -1);
      phase_end(0);
      scores(0);
      phase_end(1);
      for (int t = 0; t < nt; ++t) {
        softmax(t, t + 3 < nt ? t + 3 : -1, false, ph);
        phase_end(2 * t + 2);
        __builtin_amdgcn_s_setprio(1);
        if (t + 1 < nt) scores(t + 1);
        pv(t);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        ph = pool_block(t + 4 < nt ? t + 4 : -1);
        phase_end(2 * t + 3);
      }
    }
  }

  // Epilogue: O = o / lb (times the dropout keep scale), LSE = (m + log2 l)
  // ln 2, with l and lb summed over the row's four lanes.
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot = sum_halves(l_tot);
  // o is divided by the sum of the weights as P.V took them (bf16): each row
  // is a convex combination of value rows; the LSE uses the fp32 sum.
  float lb_tot = lb_run + __shfl_xor(lb_run, 16, 64);
  lb_tot = sum_halves(lb_tot);
  const float inv = (lb_tot > 0.f ? 1.f / lb_tot : 0.f) * (DROP ? p.drop_scale : 1.f);
  // The wave's 16 output rows go through its 8 KB share of the idle K ring
  // (16-byte chunks of each row swizzled by the row) so that global stores
  // write whole rows.
  uint16_t* stage = &k_s[0][0] + wave * (kRows * D);
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    uint2 st;
    st.x = pack_bf16x2(oacc[db][0] * inv, oacc[db][1] * inv);
    st.y = pack_bf16x2(oacc[db][2] * inv, oacc[db][3] * inv);
    *(uint2*)&stage[n * D + ((2 * db + (j >> 1)) ^ n) * 8 + 4 * (j & 1)] = st;
  }
  constexpr int RPS = 64 / CH;  // rows per store instruction
  uint16_t* __restrict__ og = (uint16_t*)p.o + o_base;
#pragma unroll
  for (int s = 0; s < kRows / RPS; ++s) {
    const int r = s * RPS + lane / CH;
    const int cc = lane % CH;
    const uint4 v = *(const uint4*)&stage[r * D + (cc ^ r) * 8];
    const int orow = q0 + 16 * wave + r;
    if (orow < nq) *(uint4*)(og + (int64_t)orow * p.o_ss + cc * 8) = v;
  }
  if (row < nq && p.lse && j == 0)
    p.lse[lse_base + row] = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : -INFINITY;
}

template <bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const int64_t nwg = (int64_t)p.num_qtiles * p.heads_q * p.batch;
  if (p.paged)
    hipLaunchKernelGGL((fwd_bf16_d256_kernel<CAUSAL, true, false>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                       p);
  else if (p.drop_t > 0)
    hipLaunchKernelGGL((fwd_bf16_d256_kernel<CAUSAL, false, true>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                       p);
  else
    hipLaunchKernelGGL((fwd_bf16_d256_kernel<CAUSAL, false, false>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                       p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16_d256(const FwdParams& p, hipStream_t stream) {
  return p.causal ? launch<true>(p, stream) : launch<false>(p, stream);
}

}  // namespace fa
