/*
 * ssa.h -- Skip-Softmax sparse attention for AMD MI355X (gfx950), C ABI.
 *
 * The operation (TRT-LLM "Skip Softmax" page, the three-step algorithm;
 * SpargeAttn page, stage two of the online filter): FlashAttention-style
 * tiled attention in which, for each query tile and key tile, the kernel
 * computes S = Q K^T / sqrt(d), takes each row's maximum over the tile
 * (m_loc) and compares it with the row's running maximum over the tiles
 * visited before (m_prev). If for EVERY row of the tile m_loc - m_prev is
 * below lambda (< 0), the tile is skipped: no exponentials, no row-sum
 * update, no P.V product and no load of the V tile.
 *
 *  - gap per row: -inf if the row has no allowed key in the tile, +inf if the
 *    row has no earlier score (first tile), else m_loc - m_prev; tile margin
 *    g = max over rows; skip iff g < lambda (strict). lambda <= 0 in natural
 *    log units of the scaled score; lambda = -INFINITY means dense.
 *  - key tiles are visited in ascending order (list order with a block list).
 *  - the output is softmax attention renormalised over the kept tiles;
 *    lse = ln(sum over kept entries of exp(s)).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers to caller-owned memory; the
 *    library never allocates or frees device memory and keeps no state.
 *  - Tensors are dense row-major (innermost dimension contiguous) in the
 *    layouts given per argument. bf16 = IEEE bfloat16.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    legacy default stream). Outputs are valid once the stream reaches it.
 *  - Every argument is validated on the host before any HIP call; a failed
 *    check returns a negative status and enqueues nothing.
 *  - Thread safety: entry points may be called concurrently from several
 *    host threads; calls whose output buffers overlap race.
 */
#ifndef SSA_H
#define SSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SSA_OK 0
#define SSA_ERR_INVALID_ARG (-1) /* null required pointer, bad size, lambda NaN or > 0, ... */
#define SSA_ERR_UNSUPPORTED (-2) /* valid but not built: head dim, tile sizes, group size */
#define SSA_ERR_WORKSPACE (-3)   /* workspace null or smaller than the *_workspace_size value */
#define SSA_ERR_HIP (-4)         /* the HIP runtime reported an error at launch */
#define SSA_ERR_SCRATCH (-5)     /* needs more than the static scratch of ssa_decode_noalloc */

/* Values written into the optional per-tile decision arrays. */
#define SSA_TILE_KEPT 1
#define SSA_TILE_SKIPPED 2

/*
 * ssa_prefill -- causal or full Skip-Softmax prefill with grouped-query heads,
 * optionally restricted to a per-query-tile list of key tiles (block-sparse
 * prefill: MInference page, block-sparse pattern).
 *
 *  q        [B, Hq, L, d]  bf16, required.
 *  k, v     [B, Hkv, L, d] bf16, required. Query head h reads KV head
 *           h / (Hq / Hkv).
 *  out      [B, Hq, L, d]  bf16, required: the renormalised attention output.
 *  lse      [B, Hq, L]     fp32, nullable: natural-log log-sum-exp of the
 *           kept scaled scores (-inf for a row with no kept key).
 *  skip_counts [B, Hq, nQ] int32, nullable: skipped tiles per query tile,
 *           nQ = ceil(L / Br).
 *  tile_state  [B, Hq, nQ, nK] uint8, nullable: SSA_TILE_KEPT or
 *           SSA_TILE_SKIPPED for each visited tile, nK = ceil(L / Bc);
 *           entries of tiles that are not visited are left untouched.
 *  tile_margin [B, Hq, nQ, nK] fp32, nullable: the tile margin g (natural
 *           log units, may be +-inf) of each visited tile; others untouched.
 *           Margins do not depend on lambda, so one call yields the skip
 *           ratio of every threshold.
 *  d in {64, 128}; Br in {32, 64, 128}; Bc = 64. causal: key c is allowed
 *  for row r iff c <= r (L_q = L_k). Br is the decision unit: Br = 32 is the
 *  warp-granular variant of the SpargeAttn page (stage two, "sparse warp
 *  online softmax"): every 32-row group decides alone, while 128-row
 *  workgroups share the K and V tiles (block lists need Br >= 64).
 *  lambda   <= 0 or -INFINITY; NaN or > 0 is rejected.
 *  block_idx [B, Hq, nQ, max_blocks] int32, nullable: for query tile i the
 *           first block_cnt[b,h,i] entries are the key tiles to visit, in
 *           visit order (ascending expected). Entries < 0, >= nK or above the
 *           causal limit are ignored. Entries should be unique: a repeated
 *           entry is visited again, so its keys count twice in the softmax
 *           (the mask builders of this library never repeat one).
 *           block_cnt [B, Hq, nQ] int32 is required with block_idx; counts
 *           are clamped to [0, max_blocks]. With Br = 64 two query tiles
 *           share a workgroup: when both lists are ascending they are merged
 *           (a tile on both is loaded once), otherwise visited one after the
 *           other; either way each tile keeps its own list order.
 *
 * Returns SSA_OK or a negative status.
 */
int ssa_prefill(const void* q, const void* k, const void* v, void* out, float* lse,
                int32_t* skip_counts, uint8_t* tile_state, float* tile_margin,
                int B, int Hq, int Hkv, int L, int d, int Br, int Bc, float lambda,
                int causal, const int32_t* block_idx, const int32_t* block_cnt,
                int max_blocks, void* stream);

/*
 * ssa_prefill_nm -- ssa_prefill with N:M sparse softmax applied to the scores
 * before the tile rule (Model Optimizer attention-sparsity tutorial, step 2:
 * in every M consecutive key positions only the top-N scores are kept and
 * the others set to -inf, a prefill-only method; its FAQ: keep sink tokens
 * and a recent-token window dense).
 *
 * Same arguments as ssa_prefill (without a block list), plus:
 *  nm_n, nm_m  keep the nm_n highest allowed scores in every aligned group of
 *              nm_m keys (key c is in group c / nm_m; ties: lower key first).
 *              nm_m in {2, 4}; 1 <= nm_n <= nm_m (nm_n == nm_m is dense).
 *  dense_sink_tokens    keys c < this are always kept (>= 0).
 *  dense_recent_tokens  keys with row - this < c <= row are always kept (>= 0).
 * lambda = -INFINITY gives N:M sparse softmax alone; a finite lambda applies
 * the Skip-Softmax rule to the N:M-masked scores.
 */
int ssa_prefill_nm(const void* q, const void* k, const void* v, void* out, float* lse,
                   int32_t* skip_counts, uint8_t* tile_state, float* tile_margin,
                   int B, int Hq, int Hkv, int L, int d, int Br, int Bc, float lambda,
                   int causal, int nm_n, int nm_m, int dense_sink_tokens,
                   int dense_recent_tokens, void* stream);

/*
 * ssa_decode_workspace_size -- bytes of device workspace ssa_decode needs:
 * per (sequence, query head, split) one fp32 partial output of d values plus
 * its running max and row-sum, then a 256-byte block holding the split
 * kernel's work counter. Returns 0 for invalid sizes.
 */
size_t ssa_decode_workspace_size(int B, int Hq, int S_max, int d, int Bc, int split_tiles);

/*
 * ssa_decode -- one new query token per sequence against a KV cache, split-K
 * over the cache with a log-sum-exp combine (TRT-LLM Skip Softmax page: the
 * decode phase is memory-bound and the skip avoids loading V tiles).
 *
 *  q        [B, Hq, d] bf16, required.
 *  k_cache, v_cache [B, Hkv, S_max, d] bf16, required; rows [0, seqlens[b])
 *           of sequence b are valid and no other row is read.
 *  seqlens  [B] int32 device array, required; each value is clamped to
 *           [0, S_max]. A length of 0 gives out = 0 and lse = -inf.
 *  out      [B, Hq, d] bf16, required.  lse [B, Hq] fp32, nullable.
 *  skip_counts [B, Hkv, nS] int32, nullable, nS = ceil(ceil(S_max/Bc) /
 *           split_tiles): skipped tiles per split (0 for splits past the end).
 *  tile_state, tile_margin [B, Hkv, nT] uint8 / fp32, nullable,
 *           nT = ceil(S_max / Bc): per visited key tile, as in ssa_prefill.
 *  The decision unit is (sequence, KV head, split): the G = Hq/Hkv query
 *  heads sharing a KV head form the rows of a tile, so a V tile is loaded
 *  unless every one of them can skip it. Each split of split_tiles key tiles
 *  restarts the running max, so its first tile is always kept.
 *  d in {64, 128}; Bc = 64; G in {1, 2, 4, 8, 16}; split_tiles >= 1.
 *  workspace: device buffer of at least ssa_decode_workspace_size(...) bytes,
 *           16-byte aligned; its contents on entry are ignored (the call
 *           sets the work counter itself, with a kernel, before the split
 *           kernel runs).
 *  Calls with B * Hkv * nS >= 2^31 return SSA_ERR_UNSUPPORTED.
 */
int ssa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens,
               void* out, float* lse, int32_t* skip_counts, uint8_t* tile_state,
               float* tile_margin, int B, int Hq, int Hkv, int S_max, int d, int Bc,
               int split_tiles, float lambda, void* workspace, size_t workspace_bytes,
               void* stream);

/* Size of the static device scratch behind ssa_decode_noalloc (32 MiB). */
#define SSA_DECODE_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * ssa_decode_noalloc -- ssa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. Same arguments, results and errors as ssa_decode,
 * without the workspace: the split partials live in a static device array
 * of SSA_DECODE_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends (its address is looked up once per device, on
 * that device's first call). Nothing is allocated or freed, by the library
 * or by any routine it calls.
 *  - Calls whose ssa_decode_workspace_size(...) exceeds
 *    SSA_DECODE_SCRATCH_BYTES return SSA_ERR_SCRATCH and enqueue nothing
 *    (for example B = 32, Hq = 32, S_max = 32768, d = 128, split_tiles = 16
 *    needs 17.0 MB and fits).
 *  - All calls on one GPU share that GPU's scratch: calls that overlap on a
 *    GPU (different streams, or host threads without ordering) race. Calls
 *    ordered on one stream are safe. No scratch content needs to start at
 *    zero: every partial the combine reads is written by the same call, and
 *    the call sets the work counter (with a kernel) before it is used.
 */
int ssa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens,
                       void* out, float* lse, int32_t* skip_counts, uint8_t* tile_state,
                       float* tile_margin, int B, int Hq, int Hkv, int S_max, int d, int Bc,
                       int split_tiles, float lambda, void* stream);

/*
 * ssa_block_mask_max_blocks -- length of the kept-block list per query block
 * that ssa_block_mask can produce: min(nB, topk + sink_blocks + W) with
 * nB = ceil(L / pool) and W = ceil(window_tokens / pool). Returns -1 for
 * invalid sizes.
 */
int ssa_block_mask_max_blocks(int L, int pool, int topk, int sink_blocks, int window_tokens);

/*
 * ssa_block_mask_workspace_size -- bytes of device workspace ssa_block_mask
 * needs (the pooled Q and K, fp32 [B, H, nB, d] each).
 */
size_t ssa_block_mask_workspace_size(int B, int H, int L, int d, int pool);

/*
 * ssa_block_mask -- predicted block-sparse mask from mean-pooled Q and K
 * (MInference page, block-sparse pattern: mean pooling commutes with the
 * matrix product, so pooled scores estimate block importance; its
 * block_sparse_attention(q, k, v, topk=64); NOSA page, section 3: always keep
 * init_blocks leading block(s) and a local window of window_size tokens).
 *
 *  q, k     [B, H, L, d] bf16, required (one KV head per query head).
 *  For query block b (pool tokens): q_bar, k_bar = fp32 means over the rows
 *  of each block (the last block may be short); score(b, c) =
 *  q_bar[b] . k_bar[c] / sqrt(d) for c <= b. Kept: the topk highest-scoring
 *  candidates (ties: lower c first), plus blocks 0..sink_blocks-1, plus
 *  blocks b-W+1..b with W = ceil(window_tokens / pool), all within [0, b].
 *  block_idx [B, H, nB, max_blocks] int32, required: kept blocks in
 *           ascending order, padded with -1. max_blocks must be at least
 *           ssa_block_mask_max_blocks(...).
 *  block_cnt [B, H, nB] int32, required: number of kept blocks.
 *  block_scores [B, H, nB, nB] fp32, nullable: the pooled scores (entries
 *           above the diagonal are -inf).
 *  Only causal masks are built (causal must be 1). d in {64, 128};
 *  pool = 64; nB <= 4096. The result feeds ssa_prefill with Br = Bc = pool.
 *  workspace: at least ssa_block_mask_workspace_size(...) bytes, 16-byte
 *           aligned.
 */
int ssa_block_mask(const void* q, const void* k, int B, int H, int L, int d, int pool,
                   int topk, int sink_blocks, int window_tokens, int causal,
                   int32_t* block_idx, int32_t* block_cnt, int max_blocks,
                   float* block_scores, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * ssa_block_mask_compressed_workspace_size -- bytes of device workspace
 * ssa_block_mask_compressed needs (pooled Q, fp32 [B, H, nB, d], then the
 * compressed keys, fp32 [B, H, ceil(L / stride), d]).
 */
size_t ssa_block_mask_compressed_workspace_size(int B, int H, int L, int d, int pool);

/*
 * ssa_block_mask_compressed -- ssa_block_mask with the keys compressed by
 * overlapping means (NOSA page, section 1: the CompressK module averages
 * kernel_size=32 keys every stride=16 tokens; section 3: attention over the
 * compressed keys picks the blocks, with init_blocks=1, window_size=1024,
 * topk=64 kept as in ssa_block_mask).
 *
 *  Compressed key m = mean of keys [m*stride, min(L, m*stride + kernel_size)),
 *  for every m with m*stride < L (fp32). Key block c is represented by the
 *  windows that start in it (m in [c*pool/stride, (c+1)*pool/stride)), and
 *  score(b, c) = max over those m of q_bar[b] . k_tilde[m] / sqrt(d), c <= b.
 *  Selection, outputs, limits and errors as ssa_block_mask; in addition
 *  kernel_size or stride <= 0 is SSA_ERR_INVALID_ARG, and only
 *  kernel_size = 32, stride = 16 are built (else SSA_ERR_UNSUPPORTED).
 *  workspace: at least ssa_block_mask_compressed_workspace_size(...) bytes,
 *           16-byte aligned.
 */
int ssa_block_mask_compressed(const void* q, const void* k, int B, int H, int L, int d, int pool,
                              int kernel_size, int stride, int topk, int sink_blocks,
                              int window_tokens, int causal, int32_t* block_idx, int32_t* block_cnt,
                              int max_blocks, float* block_scores, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Top-tau selection modes of ssa_sparge_mask. */
#define SSA_TAU_MASS 0
#define SSA_TAU_COUNT 1

/*
 * ssa_sparge_mask_workspace_size -- bytes of device workspace ssa_sparge_mask
 * needs (pooled Q and K, fp32 [B, H, nB, d] each, then the self-similarity
 * of every Q and K block, fp32 [B, H, nB] each).
 */
size_t ssa_sparge_mask_workspace_size(int B, int H, int L, int d, int pool);

/*
 * ssa_sparge_mask -- SpargeAttn stage-one block mask (SpargeAttn page,
 * two-stage online filter, stage one "sparse block online prediction":
 * blocks whose tokens are similar are compressed to their mean token, a
 * compressed attention map P_hat is built, and its Top-tau blocks are
 * kept). Stage two is ssa_prefill's skip rule run over the returned lists.
 *
 *  q, k     [B, H, L, d] bf16, required (one KV head per query head).
 *  Per block of pool tokens (the last may be short): self-similarity =
 *  mean cosine similarity over all ordered token pairs of the block, self
 *  pairs included (= squared norm of the mean unit row; a zero row counts
 *  as a zero vector). A block is compressed iff its self-similarity > theta.
 *  For a compressed query block b: P_hat[b, c] = softmax over the
 *  compressed key blocks c <= b of q_bar[b] . k_bar[c] / sqrt(d) (fp32 block
 *  means). Selection over those candidates, ranked by P_hat (ties: lower c
 *  first):
 *    tau_mode = SSA_TAU_MASS:  the smallest top set whose P_hat mass >= tau;
 *    tau_mode = SSA_TAU_COUNT: the ceil(tau * n) best of the n candidates
 *                              (the product and ceil in fp64).
 *  Kept = the selection plus every uncompressed key block c <= b; an
 *  uncompressed query block keeps every c <= b.
 *  theta    any non-NaN float (> 1: nothing compressed, dense mask).
 *  tau      in (0, 1].
 *  block_idx [B, H, nB, max_blocks] int32, required: kept blocks ascending,
 *           padded with -1; max_blocks >= nB = ceil(L / pool).
 *  block_cnt [B, H, nB] int32, required.
 *  block_sim [B, H, 2, nB] fp32, nullable: self-similarity of the Q blocks
 *           (index 0) and K blocks (index 1).
 *  block_scores [B, H, nB, nB] fp32, nullable: the pooled scores of every
 *           causal pair (entries above the diagonal are -inf).
 *  Only causal masks (causal = 1); d in {64, 128}; pool = 64; nB <= 4096.
 *  The lists feed ssa_prefill with Br = Bc = pool.
 *  workspace: at least ssa_sparge_mask_workspace_size(...) bytes, 16-byte
 *           aligned; its contents on entry are ignored.
 *  Errors: SSA_ERR_INVALID_ARG for missing pointers, bad sizes, theta NaN,
 *  tau outside (0, 1], an unknown tau_mode or max_blocks < nB;
 *  SSA_ERR_UNSUPPORTED for other d, pool or causal = 0.
 */
int ssa_sparge_mask(const void* q, const void* k, int B, int H, int L, int d, int pool,
                    float theta, double tau, int tau_mode, int causal, int32_t* block_idx,
                    int32_t* block_cnt, int max_blocks, float* block_sim, float* block_scores,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssa_vertical_slash_workspace_size -- bytes of device workspace
 * ssa_vertical_slash_mask needs (row statistics, column and diagonal scores
 * and their partials, tile flags and prefix counts).
 */
size_t ssa_vertical_slash_workspace_size(int B, int H, int L);

/*
 * ssa_vertical_slash_mask -- vertical-slash block estimator (MInference
 * page: the vertical-slash pattern is estimated by attending from the last
 * query vector(s) to every key, which picks the best vertical lines and
 * slash lines; its vertical_slash_sparse_attention(vertical_topk, slash)).
 *
 *  q, k     [B, H, L, d] bf16, required (one KV head per query head).
 *  The last last_q query rows i (positions p_i = L - last_q + i) attend
 *  causally: A[i, j] = softmax over j <= p_i of q_i . k_j / sqrt(d), fp32.
 *  Vertical score v[j] = sum_i A[i, j]; slash score s[o] = sum_i A[i, p_i - o]
 *  (o = 0 is the main diagonal). The n_vertical keys and n_slash offsets
 *  with the highest scores are chosen (ties: lower index first; a count of
 *  L or more takes all).
 *  Tiles of pool x pool: tile (b, c), c <= b, is listed iff it holds an
 *  entry (r, j), j <= r, with j a chosen vertical or r - j a chosen slash.
 *  The prefill then computes every listed tile in full (a superset of the
 *  line pattern at tile granularity).
 *  block_idx [B, H, nB, max_blocks] int32, required: ascending, -1 padded;
 *           max_blocks >= nB = ceil(L / pool).
 *  block_cnt [B, H, nB] int32, required.
 *  vertical_idx [B, H, n_vertical] int32, nullable: chosen keys, ascending
 *           (-1 padded when n_vertical > L). slash_idx likewise for offsets.
 *  vertical_scores, slash_scores [B, H, L] fp32, nullable: v and s.
 *  1 <= last_q <= min(L, 64); n_vertical, n_slash >= 0; causal = 1;
 *  d in {64, 128}; pool = 64; nB <= 4096.
 *  workspace: at least ssa_vertical_slash_workspace_size(B, H, L) bytes,
 *           256-byte aligned; contents on entry are ignored.
 *  Errors: SSA_ERR_INVALID_ARG for missing pointers, bad sizes, last_q
 *  outside [1, L], negative counts or max_blocks < nB; SSA_ERR_UNSUPPORTED
 *  for causal = 0, other d or pool, or last_q > 64.
 */
int ssa_vertical_slash_mask(const void* q, const void* k, int B, int H, int L, int d, int last_q,
                            int n_vertical, int n_slash, int pool, int causal, int32_t* block_idx,
                            int32_t* block_cnt, int max_blocks, int32_t* vertical_idx,
                            int32_t* slash_idx, float* vertical_scores, float* slash_scores,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssa_calibrate_workspace_size -- bytes of device workspace that
 * ssa_lambda_for_ratio needs for n_margins margins and the given rank
 * window. Returns 0 for n_margins > 2^40 or window outside [0, 0.5].
 */
size_t ssa_calibrate_workspace_size(size_t n_margins, double window);

/*
 * ssa_lambda_for_ratio -- the threshold that skips a target share of the
 * visited tiles, computed on the device from per-tile margins (TRT-LLM
 * Skip Softmax page, efficiency and accuracy: an automatic calibration
 * program finds the threshold for a target sparsity; Model Optimizer
 * tutorial, step 4: calibrate the threshold to a target sparsity ratio).
 *
 * A tile's margin does not depend on lambda, so the skip set at lambda is
 * {margin < lambda}. With g the sorted non-NaN margins (n of them; NaN marks
 * a tile that was not visited), want = round-half-even(target * n),
 * lo = max(1, floor((target - window) * n)), hi = min(n - 1,
 * ceil((target + window) * n)), then lo = min(lo, max(1, want)) and
 * hi = max(hi, min(n - 1, want)) (all in fp64): among the pairs
 * (g[r-1], g[r]), lo <= r <= hi, with both values finite, the first one with
 * the largest difference g[r] - g[r-1] gives lambda = (g[r-1] + g[r]) / 2;
 * with no such pair, lambda = g[min(max(want, 0), n - 1)] if finite, else 0;
 * n < 2 gives 0. Finally lambda = min(lambda, 0). Differences and the
 * midpoint are taken in fp64 of the fp32 margins.
 *
 *  margins  device fp32 array of n_margins values (for instance the
 *           tile_margin output of ssa_prefill or ssa_decode, initialised to
 *           NaN); nullable only when n_margins = 0; 4-byte aligned.
 *  target   in [0, 1]; window in [0, 0.5] (the rule above uses 0.01).
 *  result   device array of 4 doubles, 8-byte aligned, written on the
 *           stream: lambda, the achieved ratio (margins below lambda / n, 0
 *           when n = 0), n, and the count of margins below lambda. lambda is
 *           NaN only if the workspace bound was exceeded (not expected).
 *  workspace at least ssa_calibrate_workspace_size(n_margins, window) bytes,
 *           256-byte aligned; contents on entry are ignored.
 *  Errors: SSA_ERR_INVALID_ARG (null pointers, target / window out of range,
 *  misalignment), SSA_ERR_WORKSPACE.
 */
int ssa_lambda_for_ratio(const float* margins, size_t n_margins, double target, double window,
                         double* result, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssa_lambda_from_scale_factor -- threshold from a context-length scale
 * factor (TRT-LLM page: the configured threshold_scale_factor is divided by
 * the context length to give the actual threshold, so longer contexts skip
 * more). Read here as a threshold on the softmax value ratio
 * exp(m_loc - m_prev) < scale_factor / L, i.e. lambda = ln(scale_factor / L),
 * clamped to <= 0. Returns NaN for scale_factor <= 0 or L <= 0.
 */
float ssa_lambda_from_scale_factor(float scale_factor, int L);

/* Human-readable name of a status code (static string). */
const char* ssa_status_string(int status);

/* ABI version of this header (major * 100 + minor). */
int ssa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSA_H */
