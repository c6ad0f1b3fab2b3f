/*
 * fa.h -- C ABI of libfa_gfx950.so: exact attention on MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention as a stream over
 * key/value tiles with the online-softmax recurrence -- a running row max m,
 * a running sum l, the correction alpha = exp(m_old - m_new) applied to the
 * output accumulator o, and a final o / l -- so the N x N score matrix never
 * reaches device memory.  Sources (page titles and sections):
 *   - "S12 FlashAttention" (llminference.xinbetween.com): "Core idea / The
 *     solution" (the recurrence), "Mechanics / How it works" (tiles in fast
 *     on-chip memory), "What this unlocks beyond speed" (paged tiles,
 *     flash-decoding split and combine), "How this composes with what you
 *     already built" (block table + GQA in one decode loop), "Build it /
 *     Implementation" (paged excerpt; the fully masked tile NaN guard);
 *   - "FlashAttention" (tachyon.techntrek.in/learn/flash-attention), "For
 *     engineers / Show the maths": the (m, l) merge rule;
 *   - "FlashAttention: The Algorithm That Beat the Memory Wall"
 *     (repo-explainer.com/hillfate/flash-attention): "A Tile, a Register
 *     File, and a Trick Called Online Softmax" (outer loop over query tiles,
 *     inner loop over key/value tiles), "How the Repo Connects Python to
 *     Bare-Metal CUDA" (strides, dtypes, masking mode and sequence layout
 *     carried in a parameter struct), "Varlen Is the Quiet Superpower"
 *     (packed sequences, no padding).
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or retains them, and keeps no state
 *     between calls (fa_decode_paged_noalloc's fixed per-device workspace
 *     holds only intermediate values of one call).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on that stream and returns; nothing
 *     synchronises.  Faults during execution surface at the caller's next
 *     synchronisation.
 *   - Strides are in ELEMENTS; the head dimension d must be contiguous.
 *   - Scores are s = scale * q . k with `scale` given by the caller (1/sqrt(d)
 *     is the usual choice).  LSE is the natural log of the sum over visible
 *     keys of exp(s), in fp32.  A query with no visible key gets O = 0 and
 *     LSE = -inf.
 *   - Causal masking is aligned to the END of the keys: key j is visible
 *     from query i iff j <= i + (Nk - Nq)  (plain j <= i when Nq == Nk).
 *   - GQA: heads_q must be a multiple of heads_kv; query head h reads key /
 *     value head h / (heads_q / heads_kv).
 *   - Validation runs on the host before any launch.  On any error nothing
 *     is launched, no output is written, and fa_last_error() describes it.
 *     No C++ exception crosses this interface.  Calls are re-entrant on
 *     distinct streams.
 */
#ifndef FA_GFX950_H
#define FA_GFX950_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 10

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL_POINTER = 1,       /* a required pointer is NULL */
  FA_ERR_BAD_SHAPE = 2,          /* negative size, heads_q % heads_kv != 0, bad stride ... */
  FA_ERR_UNSUPPORTED = 3,        /* valid but not built: dtype / head_dim / block_size */
  FA_ERR_WORKSPACE_TOO_SMALL = 4,
  FA_ERR_HIP = 5                 /* the HIP runtime reported an error at launch */
} fa_status;

typedef enum { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

/*
 * fa_fwd -- dense batched attention (MHA or GQA), optional causal mask,
 * optional LSE output.
 *
 *   q  [batch, seqlen_q, heads_q,  head_dim]   strides q_stride  = {batch, seq, head}
 *   k  [batch, seqlen_k, heads_kv, head_dim]   strides k_stride
 *   v  [batch, seqlen_k, heads_kv, head_dim]   strides v_stride
 *   o  [batch, seqlen_q, heads_q,  head_dim]   strides o_stride  (written)
 *   lse [batch, heads_q, seqlen_q] fp32, contiguous (written; may be NULL)
 *
 * dtype FA_F32 (fp32 in, fp32 out, fp32 MFMA) or FA_BF16 (bf16 in, bf16 out
 * rounded to nearest-even, fp32 accumulation); head_dim 64 or 128, and 256
 * for FA_BF16 (FA_ERR_UNSUPPORTED otherwise).
 * seqlen_q == 0 or batch == 0 is a no-op; seqlen_k == 0 writes O = 0 and
 * LSE = -inf (k and v may then be NULL).  Strides are in elements,
 * non-negative multiples of 16 bytes; for FA_BF16 the k and v sequence
 * strides are at most 2^24 elements (FA_ERR_UNSUPPORTED otherwise).
 */
typedef struct {
  const void *q, *k, *v;
  void *o;
  float *lse;
  int32_t batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
  fa_dtype dtype;
  float scale;
  int32_t causal;
} fa_fwd_args;

fa_status fa_fwd(const fa_fwd_args *args, void *stream);

/*
 * fa_fwd_fp8 -- dense attention (MHA or GQA) over FP8 E4M3 inputs with
 * per-tensor descale factors, the FP8 mode "S12 FlashAttention"
 * (llminference.xinbetween.com), "Production notes / In production",
 * credits to FlashAttention-3.
 *
 *   q  [batch, seqlen_q, heads_q,  head_dim] E4M3 codes (one byte each),
 *      strides q_stride = {batch, seq, head}
 *   k  [batch, seqlen_k, heads_kv, head_dim] E4M3, strides k_stride
 *   v  [batch, seqlen_k, heads_kv, head_dim] E4M3, strides v_stride
 *   o  [batch, seqlen_q, heads_q,  head_dim] bf16, strides o_stride (written)
 *   lse [batch, heads_q, seqlen_q] fp32, contiguous (written; may be NULL)
 *
 * The inputs stand for q_descale * value(q), k_descale * value(k) and
 * v_descale * value(v) (E4M3: sign, 4-bit exponent with bias 7, 3-bit
 * mantissa, subnormals, no infinities); scores are scale * q . k over those
 * tensors, with the causal and GQA conventions above.  Both products run on
 * the FP8 matrix cores with fp32 accumulation; the softmax weights are
 * rounded to E4M3 for the second product and O is normalised by the sum of
 * the rounded weights, LSE by the fp32 sum.  head_dim 128; strides are in
 * elements (bytes for the inputs) and multiples of 16 bytes; k and v
 * sequence strides at most 2^24.  Descale factors must be positive and
 * finite.  seqlen_q == 0 or batch == 0 is a no-op; seqlen_k == 0 writes
 * O = 0 and LSE = -inf.
 */
typedef struct {
  const void *q, *k, *v;
  void *o;
  float *lse;
  int32_t batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
  float q_descale, k_descale, v_descale;
  float scale;
  int32_t causal;
} fa_fwd_fp8_args;

fa_status fa_fwd_fp8(const fa_fwd_fp8_args *args, void *stream);

/*
 * fa_fwd_varlen -- packed variable-length sequences, no padding tokens.
 *
 *   q  [total_tokens, heads_q,  head_dim]   strides q_stride = {token, head}
 *   k,v[total_tokens, heads_kv, head_dim]
 *   o  [total_tokens, heads_q,  head_dim]   (written)
 *   lse [heads_q, total_tokens] fp32 contiguous (written; may be NULL)
 *   cu_seqlens: DEVICE int32 [num_seqs + 1], cu[0] = 0, non-decreasing,
 *     cu[num_seqs] = total_tokens; sequence s owns tokens [cu[s], cu[s+1]).
 *   max_seqlen: a HOST-side upper bound on every sequence length (it sizes
 *     the grid; the library never reads cu_seqlens on the host).  A sequence
 *     longer than max_seqlen is processed only up to max_seqlen queries.
 *
 * A query sees only keys of its own sequence (causal in local positions
 * when causal != 0); an empty sequence writes nothing.  dtype FA_BF16 or
 * FA_F32; head_dim 64 or 128, and 256 for FA_BF16.  For FA_BF16 the k and
 * v token strides are at most 2^24 elements (FA_ERR_UNSUPPORTED otherwise).
 */
typedef struct {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const int32_t *cu_seqlens;
  int32_t num_seqs, total_tokens, max_seqlen, heads_q, heads_kv, head_dim;
  int64_t q_stride[2], k_stride[2], v_stride[2], o_stride[2];
  fa_dtype dtype;
  float scale;
  int32_t causal;
} fa_fwd_varlen_args;

fa_status fa_fwd_varlen(const fa_fwd_varlen_args *args, void *stream);

/*
 * fa_fwd_varlen_fp8 -- packed variable-length sequences (as fa_fwd_varlen)
 * over FP8 E4M3 inputs with per-tensor descale factors (as fa_fwd_fp8).
 *
 *   q  [total_tokens, heads_q,  head_dim] E4M3 codes, strides q_stride = {token, head}
 *   k,v[total_tokens, heads_kv, head_dim] E4M3
 *   o  [total_tokens, heads_q,  head_dim] bf16 (written)
 *   lse [heads_q, total_tokens] fp32 contiguous (written; may be NULL)
 *   cu_seqlens, max_seqlen: as for fa_fwd_varlen.
 *
 * Arithmetic, rounding, head_dim (128), stride and descale rules are those
 * of fa_fwd_fp8; sequence rules those of fa_fwd_varlen.
 */
typedef struct {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const int32_t *cu_seqlens;
  int32_t num_seqs, total_tokens, max_seqlen, heads_q, heads_kv, head_dim;
  int64_t q_stride[2], k_stride[2], v_stride[2], o_stride[2];
  float q_descale, k_descale, v_descale;
  float scale;
  int32_t causal;
} fa_fwd_varlen_fp8_args;

fa_status fa_fwd_varlen_fp8(const fa_fwd_varlen_fp8_args *args, void *stream);

/*
 * fa_fwd_dropout / fa_fwd_varlen_dropout -- fa_fwd and fa_fwd_varlen with
 * dropout of the normalised attention weights, the dropout variant
 * "FlashAttention: The Algorithm That Beat the Memory Wall"
 * (repo-explainer.com), "How the Repo Connects Python to Bare-Metal CUDA"
 * and "Why Templates Matter Here", lists among the kernel's parameters and
 * specialisations.
 *
 * With t = the nearest integer to 256 * p (ties to even), each weight
 * P[r][j] = exp(s_rj - LSE_r) is kept with probability (256 - t) / 256 and
 * scaled by 256 / (256 - t), or replaced by 0:
 *     O[r] = sum_j keep(r, j) * 256 / (256 - t) * P[r][j] * v_j.
 * LSE is that of the weights before dropout (the same as without it).  The
 * mask is a function of (seed, offset, row, key) only, so it can be
 * regenerated exactly: row r is the row's index in the LSE layout
 * ((b * heads_q + h) * seqlen_q + i for fa_fwd_dropout, h * total_tokens +
 * token for fa_fwd_varlen_dropout), j is the key's position in its sequence,
 * and keep(r, j) holds iff byte (j mod 16) (little-endian) of
 * Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011) at counter
 * {j / 16, r mod 2^32, r / 2^32, offset} under key {seed mod 2^32,
 * seed / 2^32} is >= t.  Callers advance `offset` (or the seed) between
 * calls that need independent masks.
 *
 * p must be in [0, 1) and round to t <= 255 (FA_ERR_BAD_SHAPE otherwise);
 * t = 0 runs the plain kernel.  Dropout is built for FA_BF16
 * (FA_ERR_UNSUPPORTED for FA_F32 with t > 0); all other arguments and
 * limits are those of fa_fwd / fa_fwd_varlen.
 */
typedef struct {
  double p;        /* dropout probability */
  uint64_t seed;   /* generator key */
  uint32_t offset; /* counter word 3 */
} fa_dropout_args;

fa_status fa_fwd_dropout(const fa_fwd_args *args, const fa_dropout_args *dropout, void *stream);
fa_status fa_fwd_varlen_dropout(const fa_fwd_varlen_args *args, const fa_dropout_args *dropout, void *stream);

/*
 * fa_fwd_paged -- chunked prefill over a paged KV pool: every sequence
 * brings a chunk of new queries that attends to all of the sequence's keys
 * in the pool (the cached prefix and the chunk's own keys, which the caller
 * has already written there).  The tiles of keys and values are fetched
 * through the block table, as "S12 FlashAttention"
 * (llminference.xinbetween.com), "What this unlocks beyond speed", has the
 * tiled loop do for paged memory; queries are packed without padding as in
 * "Varlen Is the Quiet Superpower" (repo-explainer.com).
 *
 *   q   [total_q, heads_q, head_dim] bf16, strides q_stride = {token, head};
 *       sequence s owns query rows [cu_seqlens_q[s], cu_seqlens_q[s+1]).
 *   k_pool, v_pool, pool_stride, block_table, num_blocks: as for
 *       fa_decode_paged; the token stride is at most 2^24 elements.
 *   cu_seqlens_q: DEVICE int32 [num_seqs + 1], cu[0] = 0, non-decreasing,
 *       cu[num_seqs] = total_q.
 *   seq_lens_k: DEVICE int32 [num_seqs]: keys of sequence s, the chunk's
 *       own included; values outside [0, max_seqlen_k] are clamped to it.
 *   o   [total_q, heads_q, head_dim] bf16, strides o_stride (written)
 *   lse [heads_q, total_q] fp32 contiguous (written; may be NULL)
 *   max_seqlen_q: HOST-side upper bound on every chunk length (it sizes the
 *       grid; a longer chunk is processed only up to max_seqlen_q queries).
 *   max_seqlen_k: HOST-side upper bound on seq_lens_k, at most
 *       max_blocks_per_seq * block_size.
 *
 * With causal != 0 query i of a chunk of n_q queries over n_k keys sees
 * keys j <= i + n_k - n_q: the chunk is the last n_q positions of the
 * sequence.  A query that sees no key (a chunk longer than its keys, or
 * n_k = 0) gets o = 0 and lse = -inf.  A chunk of one query is a decode
 * step.  Supported: bf16, head_dim 64, 128 or 256, block_size 16.
 */
typedef struct {
  const void *q;
  const void *k_pool, *v_pool;
  int64_t pool_stride[3];
  const int32_t *block_table;
  const int32_t *cu_seqlens_q;
  const int32_t *seq_lens_k;
  void *o;
  float *lse;
  int64_t q_stride[2], o_stride[2];
  int32_t num_seqs, total_q, max_seqlen_q, max_seqlen_k, heads_q, heads_kv, head_dim, block_size,
      max_blocks_per_seq, num_blocks;
  float scale;
  int32_t causal;
} fa_fwd_paged_args;

fa_status fa_fwd_paged(const fa_fwd_paged_args *args, void *stream);

/*
 * fa_fwd_paged_fp8 -- fa_fwd_paged with FP8 E4M3 queries and pools (an FP8
 * KV cache) and per-tensor descale factors, computed as fa_fwd_fp8 computes
 * (both products on the FP8 matrix cores, O normalised by the sum of the
 * E4M3-rounded weights, LSE by the fp32 sum).  `base` is read as for
 * fa_fwd_paged with q and the pools as E4M3 codes: their strides count
 * bytes and are multiples of 16 (o stays bf16, strides in elements).
 * head_dim 128, block_size 16; descale factors positive and finite.
 */
typedef struct {
  fa_fwd_paged_args base;
  float q_descale, k_descale, v_descale;
} fa_fwd_paged_fp8_args;

fa_status fa_fwd_paged_fp8(const fa_fwd_paged_fp8_args *args, void *stream);

/*
 * fa_decode_paged -- one query token per sequence over a paged KV pool
 * (flash-decoding: the keys are split across waves and the partial
 * (m, l, o) states are merged by a second kernel).
 * "S12 FlashAttention" (llminference.xinbetween.com): "What this unlocks
 * beyond speed" (tiles fetched through a block table; keys split across
 * thread blocks, partial states combined), "How this composes with what
 * you already built" (one loop with the block-table indirection and the
 * group's shared KV head), "Build it / Implementation" (the paged loop).
 *
 *   q   [batch, heads_q, head_dim] bf16, strides q_stride = {batch, head}
 *   k_pool, v_pool: bf16 block pools addressed with element strides
 *       pool_stride = {block, head, token}; the default layout is
 *       [num_blocks, heads_kv, block_size, head_dim].  Both pools share the
 *       strides; the token stride is at most 2^26 elements.
 *   block_table: DEVICE int32 [batch, max_blocks_per_seq] (row stride
 *       max_blocks_per_seq); logical key t of sequence b lives in block
 *       block_table[b][t / block_size], slot t % block_size.  Entries past
 *       ceil(seq_lens[b] / block_size) are never read.  Entries that are read
 *       must lie in [0, num_blocks): the kernel does not check them.
 *   seq_lens: DEVICE int32 [batch], each in [0, max_seq_len].
 *   o   [batch, heads_q, head_dim] bf16, strides o_stride (written)
 *   lse [batch, heads_q] fp32 contiguous (written; may be NULL).  A sequence
 *       with no keys gets o = 0 and lse = -inf.
 *   max_seq_len: HOST-side upper bound on seq_lens, at most
 *       max_blocks_per_seq * block_size; batch * ceil(max_seq_len /
 *       block_size) must stay below 2^31.
 *   num_splits: the key blocks of all sequences of one KV head, taken in
 *       batch order, are cut into num_splits equal parts, one wave each
 *       (0 = library choice: one part per wave slot of the device, at most
 *       about one per four blocks).  The cut depends only on logical
 *       positions, so a permuted pool gives bit-identical results.
 *   workspace: DEVICE scratch of at least fa_decode_paged_workspace_size()
 *       bytes, owned by the caller, 16-byte aligned; contents on entry are
 *       ignored.  Holds heads_q * (parts + batch) partial states of
 *       head_dim + 4 floats.
 *
 * Supported: bf16, head_dim 64, 128 or 256, block_size 16,
 * heads_q / heads_kv <= 16.
 */
typedef struct {
  const void *q;
  const void *k_pool, *v_pool;
  int64_t pool_stride[3];
  const int32_t *block_table;
  const int32_t *seq_lens;
  void *o;
  float *lse;
  int64_t q_stride[2], o_stride[2];
  int32_t batch, heads_q, heads_kv, head_dim, block_size, max_blocks_per_seq, num_blocks,
      max_seq_len;
  float scale;
  int32_t num_splits;
  void *workspace;
  size_t workspace_bytes;
} fa_decode_paged_args;

/* Bytes of workspace fa_decode_paged needs for these arguments (0 on invalid
 * arguments).  Depends on batch, heads_q, heads_kv, max_seq_len, num_splits
 * and, when num_splits is 0, the current device's compute-unit count. */
size_t fa_decode_paged_workspace_size(const fa_decode_paged_args *args);

fa_status fa_decode_paged(const fa_decode_paged_args *args, void *stream);

/* The number of parts fa_decode_paged will cut each KV head's key blocks
 * into for these arguments (0 on invalid arguments). */
int32_t fa_decode_paged_num_splits(const fa_decode_paged_args *args);

/*
 * fa_decode_paged_noalloc -- fa_decode_paged for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and results (bit for
 * bit, for the same arguments and split count), with the partial states kept
 * in a workspace the library itself holds instead of the caller's.
 *
 *   args: as for fa_decode_paged; `workspace` and `workspace_bytes` are
 *       ignored.  Inputs and outputs are still the caller's.
 *   The library's workspace is a fixed array of
 *       fa_decode_paged_noalloc_max_bytes() bytes (16 MiB) in device memory,
 *       one per GPU the library runs on, held until the process ends.  Its
 *       address is looked up on the first call on each device (the current
 *       device; `stream` must belong to it).  Arguments whose
 *       fa_decode_paged_workspace_size() exceeds it are rejected with
 *       FA_ERR_WORKSPACE_TOO_SMALL before any launch (lower num_splits or
 *       the batch, or call fa_decode_paged with a workspace).
 *   Nothing is allocated or freed: no hipMalloc, hipFree or allocating
 *       library call.  Nothing needs clearing between calls (the kernels
 *       write every partial state they read).
 *   Every call on one GPU shares that GPU's array: calls that overlap in
 *       time on one GPU (different streams without ordering between them,
 *       or different host threads) race and give undefined results.
 *       Calls ordered on one stream are safe.
 */
fa_status fa_decode_paged_noalloc(const fa_decode_paged_args *args, void *stream);

/* Bytes of the library-held workspace of fa_decode_paged_noalloc. */
size_t fa_decode_paged_noalloc_max_bytes(void);

/*
 * fa_decode_paged_fp8 -- fa_decode_paged over an FP8 KV cache: k_pool and
 * v_pool hold E4M3 codes (one byte each; the OCP format of fa_fwd_fp8)
 * standing for k_descale * value(code) and v_descale * value(code); q and o
 * stay bf16.  `base` is read as for fa_decode_paged, with pool_stride in
 * bytes (multiples of 16, token stride at most 2^26); the workspace size and
 * split count are reported by fa_decode_paged_fp8_workspace_size() and
 * fa_decode_paged_fp8_num_splits() (the automatic split count follows this
 * kernel's occupancy, four waves per SIMD below head_dim 256).  The codes are widened to
 * bf16 exactly in registers and the products and softmax are those of
 * fa_decode_paged; K's descale scales the scores and V's the output.
 * Descale factors must be positive and finite.
 */
typedef struct {
  fa_decode_paged_args base;
  float k_descale, v_descale;
} fa_decode_paged_fp8_args;

fa_status fa_decode_paged_fp8(const fa_decode_paged_fp8_args *args, void *stream);
size_t fa_decode_paged_fp8_workspace_size(const fa_decode_paged_fp8_args *args);
int32_t fa_decode_paged_fp8_num_splits(const fa_decode_paged_fp8_args *args);

/*
 * fa_merge_states -- merge the results of attention of the same queries
 * over P disjoint key sets into the result over their union.  Each part p
 * gives, per query row, its normalised output o_p and its log-sum-exp
 * lse_p (the forms every entry point above writes); with m = max_p lse_p
 * and w_p = exp(lse_p - m), the union has
 *     o = sum_p w_p o_p / sum_p w_p,   lse = m + log(sum_p w_p).
 * This is the (m, l, o) merge rule of "FlashAttention"
 * (tachyon.techntrek.in), "For engineers / Show the maths", applied once
 * to P states; "S12 FlashAttention" (llminference.xinbetween.com), "What
 * this unlocks beyond speed", uses it to pass one sequence's keys around a
 * ring of GPUs and to combine flash-decoding splits across processors.
 * The key sets may live on other devices: gather their (o_p, lse_p) here
 * and merge once.
 *
 *   num_parts P >= 1; batch, seqlen, heads >= 0; head_dim in {64, 128, 256}.
 *   dtype: FA_BF16 or FA_F32, for o_parts and o alike.
 *   o_parts: DEVICE [P, batch, seqlen, heads, head_dim] contiguous (part p
 *       starts at element p * batch * seqlen * heads * head_dim).
 *   lse_parts: DEVICE fp32 [P, batch, heads, seqlen] contiguous, natural
 *       log.  -inf marks a row for which part p saw no key: its o_p row is
 *       then ignored (it may hold anything, NaN included).  Values must not
 *       be NaN or +inf.
 *   o: DEVICE [batch, seqlen, heads, head_dim] contiguous (written); must not
 *       overlap the inputs.
 *   lse: DEVICE fp32 [batch, heads, seqlen] (written; may be NULL).
 * A row with lse_p = -inf in every part gets o = 0 and lse = -inf.  The
 * dense (seqlen = N), packed (batch = 1, seqlen = total tokens) and decode
 * (seqlen = 1) outputs all have this layout.  All pointers 16-byte
 * aligned; P * batch * seqlen * heads * head_dim below 2^40 and
 * batch * seqlen * heads * head_dim below 2^34 (FA_ERR_UNSUPPORTED
 * otherwise).
 */
typedef struct {
  int32_t num_parts, batch, seqlen, heads, head_dim;
  fa_dtype dtype;
  const void *o_parts;
  const float *lse_parts;
  void *o;
  float *lse;
} fa_merge_states_args;

fa_status fa_merge_states(const fa_merge_states_args *args, void *stream);

/* Static text for a status code. */
const char *fa_status_string(fa_status status);

/* Detail of the last error on the calling thread ("" if none). */
const char *fa_last_error(void);

/* FA_ABI_VERSION of the loaded library. */
int32_t fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_GFX950_H */
