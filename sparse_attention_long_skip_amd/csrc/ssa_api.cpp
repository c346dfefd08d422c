// C ABI of the Skip-Softmax library: argument validation, workspace sizing,
// and dispatch to the HIP launchers. Every check runs before any HIP call.
#include "../../include/ssa.h"

#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "launch.h"

static_assert(ssa::kDecodeScratchBytes == SSA_DECODE_SCRATCH_BYTES, "scratch size");

namespace {

constexpr int kBc = 64;
constexpr int kMaxMaskBlocks = 4096;
constexpr size_t kMaxMargins = (size_t)1 << 40;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool bad_lambda(float lam) { return isnan(lam) || lam > 0.f; }

// Product of positive ints fits in size_t and the element count stays below 2^62.
bool sizes_ok(std::initializer_list<long long> dims) {
  unsigned long long n = 1;
  for (long long d : dims) {
    if (d <= 0) return false;
    if (n > (1ull << 62) / (unsigned long long)d) return false;
    n *= (unsigned long long)d;
  }
  return true;
}

int check_prefill(const void* q, const void* k, const void* v, const void* out, int B, int Hq,
                  int Hkv, int L, int d, int Br, int Bc, float lambda, int causal,
                  const int32_t* block_idx, const int32_t* block_cnt, int max_blocks) {
  if (!q || !k || !v || !out) return SSA_ERR_INVALID_ARG;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || d <= 0 || Br <= 0 || Bc <= 0)
    return SSA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return SSA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return SSA_ERR_INVALID_ARG;
  if (bad_lambda(lambda)) return SSA_ERR_INVALID_ARG;
  if ((block_idx == nullptr) != (block_cnt == nullptr)) return SSA_ERR_INVALID_ARG;
  if (block_idx && max_blocks <= 0) return SSA_ERR_INVALID_ARG;
  if (!sizes_ok({B, Hq, L, d})) return SSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return SSA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return SSA_ERR_UNSUPPORTED;
  if (Br != 32 && Br != 64 && Br != 128) return SSA_ERR_UNSUPPORTED;
  if (Br == 32 && block_idx) return SSA_ERR_UNSUPPORTED;
  if (Bc != kBc) return SSA_ERR_UNSUPPORTED;
  const long long nQ = ((long long)L + Br - 1) / Br;
  if ((long long)B * Hq * nQ >= (1ll << 31)) return SSA_ERR_UNSUPPORTED;
  return SSA_OK;
}

int check_decode(const void* q, const void* kc, const void* vc, const int32_t* seqlens,
                 const void* out, int B, int Hq, int Hkv, int S_max, int d, int Bc,
                 int split_tiles, float lambda, const void* ws, size_t ws_bytes) {
  if (!q || !kc || !vc || !seqlens || !out) return SSA_ERR_INVALID_ARG;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S_max <= 0 || d <= 0 || Bc <= 0 || split_tiles <= 0)
    return SSA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return SSA_ERR_INVALID_ARG;
  if (bad_lambda(lambda)) return SSA_ERR_INVALID_ARG;
  if (!sizes_ok({B, Hkv, S_max, d})) return SSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16) || !aligned(out, 2))
    return SSA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return SSA_ERR_UNSUPPORTED;
  if (Bc != kBc) return SSA_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return SSA_ERR_UNSUPPORTED;
  const size_t nS = ssa::decode_num_splits(S_max, Bc, split_tiles);
  if (nS > 65535 || Hkv > 65535 || B > 65535 || Hq > 65535) return SSA_ERR_UNSUPPORTED;
  // splits are numbered by a 32-bit work counter
  if ((long long)B * Hkv * (long long)nS >= (1ll << 31)) return SSA_ERR_UNSUPPORTED;
  if (!ws || !aligned(ws, 16)) return SSA_ERR_WORKSPACE;
  if (ws_bytes < ssa::decode_workspace_bytes(B, Hq, S_max, d, Bc, split_tiles))
    return SSA_ERR_WORKSPACE;
  return SSA_OK;
}

int mask_max_blocks(int L, int pool, int topk, int sink, int window) {
  if (L <= 0 || pool <= 0 || topk < 0 || sink < 0 || window < 0) return -1;
  const long long nB = ((long long)L + pool - 1) / pool;
  const long long W = window > 0 ? ((long long)window + pool - 1) / pool : 0;
  long long m = (long long)topk + sink + W;
  if (m > nB) m = nB;
  if (m < 1) m = 1;
  return (int)m;
}

int check_mask(const void* q, const void* k, int B, int H, int L, int d, int pool, int topk,
               int sink, int window, int causal, const int32_t* block_idx,
               const int32_t* block_cnt, int max_blocks, const void* ws, size_t ws_bytes,
               bool compressed = false) {
  if (!q || !k || !block_idx || !block_cnt) return SSA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || L <= 0 || d <= 0 || pool <= 0) return SSA_ERR_INVALID_ARG;
  if (topk < 0 || sink < 0 || window < 0) return SSA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return SSA_ERR_INVALID_ARG;
  if (!sizes_ok({B, H, L, d})) return SSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(block_idx, 4) || !aligned(block_cnt, 4))
    return SSA_ERR_INVALID_ARG;
  if (max_blocks < mask_max_blocks(L, pool, topk, sink, window)) return SSA_ERR_INVALID_ARG;
  if (!causal) return SSA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return SSA_ERR_UNSUPPORTED;
  if (pool != 64) return SSA_ERR_UNSUPPORTED;
  const long long nB = ((long long)L + pool - 1) / pool;
  if (nB > kMaxMaskBlocks || (long long)B * H > 65535) return SSA_ERR_UNSUPPORTED;
  if (!ws || !aligned(ws, 16)) return SSA_ERR_WORKSPACE;
  const size_t need = compressed ? ssa::compressed_mask_workspace_bytes(B, H, L, d, pool)
                                 : ssa::mask_workspace_bytes(B, H, L, d, pool);
  if (ws_bytes < need) return SSA_ERR_WORKSPACE;
  return SSA_OK;
}

int check_sparge(const void* q, const void* k, int B, int H, int L, int d, int pool, float theta,
                 double tau, int tau_mode, int causal, const int32_t* block_idx,
                 const int32_t* block_cnt, int max_blocks, const void* ws, size_t ws_bytes) {
  if (!q || !k || !block_idx || !block_cnt) return SSA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || L <= 0 || d <= 0 || pool <= 0) return SSA_ERR_INVALID_ARG;
  if (isnan(theta) || !(tau > 0.0 && tau <= 1.0)) return SSA_ERR_INVALID_ARG;
  if (tau_mode != SSA_TAU_MASS && tau_mode != SSA_TAU_COUNT) return SSA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return SSA_ERR_INVALID_ARG;
  if (!sizes_ok({B, H, L, d})) return SSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(block_idx, 4) || !aligned(block_cnt, 4))
    return SSA_ERR_INVALID_ARG;
  const long long nB = ((long long)L + pool - 1) / pool;
  if (max_blocks < nB) return SSA_ERR_INVALID_ARG;
  if (!causal) return SSA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return SSA_ERR_UNSUPPORTED;
  if (pool != 64) return SSA_ERR_UNSUPPORTED;
  if (nB > kMaxMaskBlocks || (long long)B * H > 65535) return SSA_ERR_UNSUPPORTED;
  if (!ws || !aligned(ws, 16)) return SSA_ERR_WORKSPACE;
  if (ws_bytes < ssa::sparge_workspace_bytes(B, H, L, d, pool)) return SSA_ERR_WORKSPACE;
  return SSA_OK;
}

int check_vslash(const void* q, const void* k, int B, int H, int L, int d, int last_q, int n_vertical,
                 int n_slash, int pool, int causal, const int32_t* block_idx,
                 const int32_t* block_cnt, int max_blocks, const void* ws, size_t ws_bytes) {
  if (!q || !k || !block_idx || !block_cnt) return SSA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || L <= 0 || d <= 0 || pool <= 0) return SSA_ERR_INVALID_ARG;
  if (last_q < 1 || last_q > L || n_vertical < 0 || n_slash < 0) return SSA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return SSA_ERR_INVALID_ARG;
  if (!sizes_ok({B, H, L, d})) return SSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(block_idx, 4) || !aligned(block_cnt, 4))
    return SSA_ERR_INVALID_ARG;
  const long long nB = ((long long)L + pool - 1) / pool;
  if (max_blocks < nB) return SSA_ERR_INVALID_ARG;
  if (!causal) return SSA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return SSA_ERR_UNSUPPORTED;
  if (pool != 64 || last_q > 64) return SSA_ERR_UNSUPPORTED;
  if (nB > kMaxMaskBlocks || (long long)B * H > 65535) return SSA_ERR_UNSUPPORTED;
  if (!ws || !aligned(ws, 256)) return SSA_ERR_WORKSPACE;
  if (ws_bytes < ssa::VsWorkspace(B, H, L).total) return SSA_ERR_WORKSPACE;
  return SSA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SSA_OK : SSA_ERR_HIP; }

}  // namespace

extern "C" {

int ssa_prefill(const void* q, const void* k, const void* v, void* out, float* lse,
                int32_t* skip_counts, uint8_t* tile_state, float* tile_margin, int B, int Hq,
                int Hkv, int L, int d, int Br, int Bc, float lambda, int causal,
                const int32_t* block_idx, const int32_t* block_cnt, int max_blocks,
                void* stream) {
  const int st = check_prefill(q, k, v, out, B, Hq, Hkv, L, d, Br, Bc, lambda, causal,
                               block_idx, block_cnt, max_blocks);
  if (st != SSA_OK) return st;
  ssa::PrefillParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.skip_counts = skip_counts;
  p.tile_state = tile_state;
  p.tile_margin = tile_margin;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.L = L;
  p.d = d;
  p.Br = Br;
  p.Bc = Bc;
  p.lambda = lambda;
  p.causal = causal;
  p.block_idx = block_idx;
  p.block_cnt = block_cnt;
  p.max_blocks = max_blocks;
  return hip_status(ssa::launch_prefill(p, static_cast<hipStream_t>(stream)));
}

int ssa_prefill_nm(const void* q, const void* k, const void* v, void* out, float* lse,
                   int32_t* skip_counts, uint8_t* tile_state, float* tile_margin, int B, int Hq,
                   int Hkv, int L, int d, int Br, int Bc, float lambda, int causal, int nm_n, int nm_m,
                   int dense_sink_tokens, int dense_recent_tokens, void* stream) {
  const int st = check_prefill(q, k, v, out, B, Hq, Hkv, L, d, Br, Bc, lambda, causal, nullptr,
                               nullptr, 0);
  if (st != SSA_OK) return st;
  if (nm_m <= 0 || nm_n <= 0 || nm_n > nm_m || dense_sink_tokens < 0 || dense_recent_tokens < 0)
    return SSA_ERR_INVALID_ARG;
  if (nm_m != 2 && nm_m != 4) return SSA_ERR_UNSUPPORTED;
  ssa::PrefillParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.skip_counts = skip_counts;
  p.tile_state = tile_state;
  p.tile_margin = tile_margin;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.L = L;
  p.d = d;
  p.Br = Br;
  p.Bc = Bc;
  p.lambda = lambda;
  p.causal = causal;
  p.block_idx = nullptr;
  p.block_cnt = nullptr;
  p.max_blocks = 0;
  p.nm_n = nm_n;
  p.nm_m = nm_m;
  p.dense_sink = dense_sink_tokens;
  p.dense_recent = dense_recent_tokens;
  return hip_status(ssa::launch_prefill(p, static_cast<hipStream_t>(stream)));
}

size_t ssa_decode_workspace_size(int B, int Hq, int S_max, int d, int Bc, int split_tiles) {
  if (B <= 0 || Hq <= 0 || S_max <= 0 || d <= 0 || Bc <= 0 || split_tiles <= 0) return 0;
  return ssa::decode_workspace_bytes(B, Hq, S_max, d, Bc, split_tiles);
}

int ssa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens,
               void* out, float* lse, int32_t* skip_counts, uint8_t* tile_state,
               float* tile_margin, int B, int Hq, int Hkv, int S_max, int d, int Bc,
               int split_tiles, float lambda, void* workspace, size_t workspace_bytes,
               void* stream) {
  const int st = check_decode(q, k_cache, v_cache, seqlens, out, B, Hq, Hkv, S_max, d, Bc,
                              split_tiles, lambda, workspace, workspace_bytes);
  if (st != SSA_OK) return st;
  ssa::DecodeParams p;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.seqlens = seqlens;
  p.out = out;
  p.lse = lse;
  p.skip_counts = skip_counts;
  p.tile_state = tile_state;
  p.tile_margin = tile_margin;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.S_max = S_max;
  p.d = d;
  p.Bc = Bc;
  p.split_tiles = split_tiles;
  p.lambda = lambda;
  p.workspace = workspace;
  return hip_status(ssa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

int ssa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens,
                       void* out, float* lse, int32_t* skip_counts, uint8_t* tile_state,
                       float* tile_margin, int B, int Hq, int Hkv, int S_max, int d, int Bc,
                       int split_tiles, float lambda, void* stream) {
  // Validate as ssa_decode, with a stand-in workspace that passes its checks;
  // then the size against the static scratch.
  const size_t need_ok = (size_t)1 << 62;
  int st = check_decode(q, k_cache, v_cache, seqlens, out, B, Hq, Hkv, S_max, d, Bc, split_tiles, lambda,
                        reinterpret_cast<void*>(uintptr_t(256)), need_ok);
  if (st != SSA_OK) return st;
  if (ssa::decode_workspace_bytes(B, Hq, S_max, d, Bc, split_tiles) > SSA_DECODE_SCRATCH_BYTES)
    return SSA_ERR_SCRATCH;
  void* ws = nullptr;
  if (ssa::decode_scratch(&ws) != hipSuccess) return SSA_ERR_HIP;
  ssa::DecodeParams p;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.seqlens = seqlens;
  p.out = out;
  p.lse = lse;
  p.skip_counts = skip_counts;
  p.tile_state = tile_state;
  p.tile_margin = tile_margin;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.S_max = S_max;
  p.d = d;
  p.Bc = Bc;
  p.split_tiles = split_tiles;
  p.lambda = lambda;
  p.workspace = ws;
  return hip_status(ssa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

int ssa_block_mask_max_blocks(int L, int pool, int topk, int sink_blocks, int window_tokens) {
  return mask_max_blocks(L, pool, topk, sink_blocks, window_tokens);
}

size_t ssa_block_mask_workspace_size(int B, int H, int L, int d, int pool) {
  if (B <= 0 || H <= 0 || L <= 0 || d <= 0 || pool <= 0) return 0;
  return ssa::mask_workspace_bytes(B, H, L, d, pool);
}

int ssa_block_mask(const void* q, const void* k, int B, int H, int L, int d, int pool, int topk,
                   int sink_blocks, int window_tokens, int causal, int32_t* block_idx,
                   int32_t* block_cnt, int max_blocks, float* block_scores, void* workspace,
                   size_t workspace_bytes, void* stream) {
  const int st = check_mask(q, k, B, H, L, d, pool, topk, sink_blocks, window_tokens, causal,
                            block_idx, block_cnt, max_blocks, workspace, workspace_bytes);
  if (st != SSA_OK) return st;
  ssa::MaskParams p;
  p.q = q;
  p.k = k;
  p.B = B;
  p.H = H;
  p.L = L;
  p.d = d;
  p.pool = pool;
  p.topk = topk;
  p.sink_blocks = sink_blocks;
  p.window_tokens = window_tokens;
  p.block_idx = block_idx;
  p.block_cnt = block_cnt;
  p.max_blocks = max_blocks;
  p.block_scores = block_scores;
  p.workspace = workspace;
  return hip_status(ssa::launch_block_mask(p, static_cast<hipStream_t>(stream)));
}

size_t ssa_sparge_mask_workspace_size(int B, int H, int L, int d, int pool) {
  if (B <= 0 || H <= 0 || L <= 0 || d <= 0 || pool <= 0) return 0;
  return ssa::sparge_workspace_bytes(B, H, L, d, pool);
}

int ssa_sparge_mask(const void* q, const void* k, int B, int H, int L, int d, int pool,
                    float theta, double tau, int tau_mode, int causal, int32_t* block_idx,
                    int32_t* block_cnt, int max_blocks, float* block_sim, float* block_scores,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_sparge(q, k, B, H, L, d, pool, theta, tau, tau_mode, causal, block_idx,
                              block_cnt, max_blocks, workspace, workspace_bytes);
  if (st != SSA_OK) return st;
  ssa::SpargeParams p = {};
  p.m.q = q;
  p.m.k = k;
  p.m.B = B;
  p.m.H = H;
  p.m.L = L;
  p.m.d = d;
  p.m.pool = pool;
  p.m.block_idx = block_idx;
  p.m.block_cnt = block_cnt;
  p.m.max_blocks = max_blocks;
  p.m.block_scores = block_scores;
  p.m.workspace = workspace;
  p.theta = theta;
  p.tau = tau;
  p.tau_mode = tau_mode;
  p.block_sim = block_sim;
  return hip_status(ssa::launch_sparge_mask(p, static_cast<hipStream_t>(stream)));
}

size_t ssa_block_mask_compressed_workspace_size(int B, int H, int L, int d, int pool) {
  if (B <= 0 || H <= 0 || L <= 0 || d <= 0 || pool <= 0) return 0;
  return ssa::compressed_mask_workspace_bytes(B, H, L, d, pool);
}

int ssa_block_mask_compressed(const void* q, const void* k, int B, int H, int L, int d, int pool,
                              int kernel_size, int stride, int topk, int sink_blocks,
                              int window_tokens, int causal, int32_t* block_idx, int32_t* block_cnt,
                              int max_blocks, float* block_scores, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (kernel_size <= 0 || stride <= 0) return SSA_ERR_INVALID_ARG;
  const int st = check_mask(q, k, B, H, L, d, pool, topk, sink_blocks, window_tokens, causal,
                            block_idx, block_cnt, max_blocks, workspace, workspace_bytes, true);
  if (st != SSA_OK) return st;
  if (kernel_size != 32 || stride != 16) return SSA_ERR_UNSUPPORTED;
  ssa::MaskParams p;
  p.q = q;
  p.k = k;
  p.B = B;
  p.H = H;
  p.L = L;
  p.d = d;
  p.pool = pool;
  p.topk = topk;
  p.sink_blocks = sink_blocks;
  p.window_tokens = window_tokens;
  p.block_idx = block_idx;
  p.block_cnt = block_cnt;
  p.max_blocks = max_blocks;
  p.block_scores = block_scores;
  p.workspace = workspace;
  p.compressed = 1;
  return hip_status(ssa::launch_block_mask(p, static_cast<hipStream_t>(stream)));
}

size_t ssa_vertical_slash_workspace_size(int B, int H, int L) {
  if (B <= 0 || H <= 0 || L <= 0) return 0;
  return ssa::VsWorkspace(B, H, L).total;
}

int ssa_vertical_slash_mask(const void* q, const void* k, int B, int H, int L, int d, int last_q,
                            int n_vertical, int n_slash, int pool, int causal, int32_t* block_idx,
                            int32_t* block_cnt, int max_blocks, int32_t* vertical_idx,
                            int32_t* slash_idx, float* vertical_scores, float* slash_scores,
                            void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_vslash(q, k, B, H, L, d, last_q, n_vertical, n_slash, pool, causal,
                              block_idx, block_cnt, max_blocks, workspace, workspace_bytes);
  if (st != SSA_OK) return st;
  ssa::VsParams p = {};
  p.q = q;
  p.k = k;
  p.B = B;
  p.H = H;
  p.L = L;
  p.d = d;
  p.last_q = last_q;
  p.n_vertical = n_vertical;
  p.n_slash = n_slash;
  p.block_idx = block_idx;
  p.block_cnt = block_cnt;
  p.max_blocks = max_blocks;
  p.vertical_idx = vertical_idx;
  p.slash_idx = slash_idx;
  p.vertical_scores = vertical_scores;
  p.slash_scores = slash_scores;
  p.workspace = workspace;
  return hip_status(ssa::launch_vertical_slash(p, static_cast<hipStream_t>(stream)));
}

size_t ssa_calibrate_workspace_size(size_t n_margins, double window) {
  if (n_margins > kMaxMargins || !(window >= 0.0 && window <= 0.5)) return 0;
  return ssa::CalWorkspace((long long)n_margins, window).total;
}

int ssa_lambda_for_ratio(const float* margins, size_t n_margins, double target, double window,
                         double* result, void* workspace, size_t workspace_bytes, void* stream) {
  if ((n_margins > 0 && !margins) || !result) return SSA_ERR_INVALID_ARG;
  if (n_margins > kMaxMargins) return SSA_ERR_INVALID_ARG;
  if (!(target >= 0.0 && target <= 1.0) || !(window >= 0.0 && window <= 0.5)) return SSA_ERR_INVALID_ARG;
  if (!aligned(margins, 4) || !aligned(result, 8)) return SSA_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 256)) return SSA_ERR_WORKSPACE;
  if (workspace_bytes < ssa::CalWorkspace((long long)n_margins, window).total) return SSA_ERR_WORKSPACE;
  return hip_status(ssa::launch_lambda_for_ratio(margins, (long long)n_margins, target, window, result,
                                                 workspace, static_cast<hipStream_t>(stream)));
}

float ssa_lambda_from_scale_factor(float scale_factor, int L) {
  if (!(scale_factor > 0.f) || L <= 0) return NAN;
  const float lam = logf(scale_factor / (float)L);
  return lam > 0.f ? 0.f : lam;
}

const char* ssa_status_string(int status) {
  switch (status) {
    case SSA_OK: return "SSA_OK";
    case SSA_ERR_INVALID_ARG: return "SSA_ERR_INVALID_ARG: invalid argument";
    case SSA_ERR_UNSUPPORTED: return "SSA_ERR_UNSUPPORTED: configuration not built";
    case SSA_ERR_WORKSPACE: return "SSA_ERR_WORKSPACE: workspace missing or too small";
    case SSA_ERR_HIP: return "SSA_ERR_HIP: HIP launch error";
    case SSA_ERR_SCRATCH:
      return "SSA_ERR_SCRATCH: the call needs more than the library's static scratch "
             "(SSA_DECODE_SCRATCH_BYTES); use the entry point that takes a workspace";
    default: return "SSA: unknown status";
  }
}

int ssa_abi_version(void) { return 101; }

}  // extern "C"
