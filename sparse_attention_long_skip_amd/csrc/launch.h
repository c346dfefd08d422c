// Host-side launch interface between the C ABI (ssa_api.cpp) and the kernels.
// Arguments reaching these functions have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssa {

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  int32_t* skip_counts;
  uint8_t* tile_state;
  float* tile_margin;
  int B, Hq, Hkv, L, d, Br, Bc;
  float lambda;
  int causal;
  const int32_t* block_idx;
  const int32_t* block_cnt;
  int max_blocks;
  int nm_n = 0, nm_m = 0, dense_sink = 0, dense_recent = 0;  // N:M sparse softmax (0: off)
};

struct DecodeParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* seqlens;
  void* out;
  float* lse;
  int32_t* skip_counts;
  uint8_t* tile_state;
  float* tile_margin;
  int B, Hq, Hkv, S_max, d, Bc, split_tiles;
  float lambda;
  void* workspace;
};

struct MaskParams {
  const void* q;
  const void* k;
  int B, H, L, d, pool, topk, sink_blocks, window_tokens;
  int32_t* block_idx;
  int32_t* block_cnt;
  int max_blocks;
  float* block_scores;
  void* workspace;
  int compressed = 0;  // 1: key blocks scored by overlapping 32-token windows, stride 16
};

// SpargeAttn stage-one mask: m carries the shapes and outputs (topk, sink
// and window unused); the workspace holds the pooled Q and K, then the
// self-similarities of the Q and K blocks.
struct SpargeParams {
  MaskParams m;
  float theta;
  double tau;
  int tau_mode;  // 0: P_hat mass, 1: count
  float* block_sim;
};

// Vertical-slash estimator: scores of the last last_q (<= 64) query rows,
// top vertical keys and slash offsets, and the 64 x 64 tiles covering them.
struct VsParams {
  const void* q;
  const void* k;
  int B, H, L, d, last_q, n_vertical, n_slash;
  int32_t* block_idx;
  int32_t* block_cnt;
  int max_blocks;
  int32_t* vertical_idx;
  int32_t* slash_idx;
  float* vertical_scores;
  float* slash_scores;
  void* workspace;
};

constexpr int kVsChunk = 256;           // keys per workgroup in the scoring passes
constexpr int kVsSpw = kVsChunk + 64;   // per-chunk diagonal partials (chunk + last_q - 1)

// Workspace of the vertical-slash estimator: byte offsets of each array,
// every one 256-byte aligned.
struct VsWorkspace {
  size_t part, stats, v, s, spart, vt, P, total;
  VsWorkspace(int B, int H, int L) {
    const size_t BH = (size_t)B * H;
    const size_t nchunk = ((size_t)L + kVsChunk - 1) / kVsChunk;
    const size_t nB = ((size_t)L + 63) / 64;
    size_t off = 0;
    auto take = [&](size_t bytes) {
      const size_t o = off;
      off += (bytes + 255) & ~(size_t)255;
      return o;
    };
    part = take(BH * nchunk * 64 * 2 * sizeof(float));
    stats = take(BH * 64 * 2 * sizeof(float));
    v = take(BH * L * sizeof(float));
    s = take(BH * L * sizeof(float));
    spart = take(BH * nchunk * kVsSpw * sizeof(float));
    vt = take(BH * nB * sizeof(int32_t));
    P = take(BH * ((size_t)L + 1) * sizeof(int32_t));
    total = off;
  }
};

// Workspace of the device threshold calibration for n margins and a rank
// window: byte offsets (256-byte aligned) of the state, the radix
// histograms, the bucket minima and maxima (nb_max each) and the per-chunk
// gap summaries.
struct CalWorkspace {
  long long nb_max;
  size_t state, hist, bmin, bmax, sums, total;
  CalWorkspace(long long n, double window);
};

// Each returns hipSuccess or the launch error.
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
hipError_t launch_block_mask(const MaskParams& p, hipStream_t stream);
hipError_t launch_sparge_mask(const SpargeParams& p, hipStream_t stream);
hipError_t launch_vertical_slash(const VsParams& p, hipStream_t stream);
// The allocation-free decode entry point's static scratch: its size, and
// its device address on the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch(void** ptr);
hipError_t launch_lambda_for_ratio(const float* margins, long long n, double target, double window,
                                   double* result, void* workspace, hipStream_t stream);

// Decode workspace layout: partial o [B, Hq, nS, d] fp32, then (m, l)
// [B, Hq, nS, 2] fp32, then a 256-byte block whose first word is the split
// kernel's work counter.
inline size_t decode_num_splits(int S_max, int Bc, int split_tiles) {
  size_t nT = ((size_t)S_max + Bc - 1) / Bc;
  return (nT + split_tiles - 1) / split_tiles;
}

constexpr size_t kDecodeQueueBytes = 256;

inline size_t decode_workspace_bytes(int B, int Hq, int S_max, int d, int Bc, int split_tiles) {
  size_t nS = decode_num_splits(S_max, Bc, split_tiles);
  return (size_t)B * Hq * nS * ((size_t)d + 2) * sizeof(float) + kDecodeQueueBytes;
}

inline size_t mask_workspace_bytes(int B, int H, int L, int d, int pool) {
  size_t nB = ((size_t)L + pool - 1) / pool;
  return 2 * (size_t)B * H * nB * d * sizeof(float);
}

// Compressed-key mask: pooled Q [B, H, nB, d], then the key windows
// [B, H, ceil(L / 16), d], fp32.
inline size_t compressed_mask_workspace_bytes(int B, int H, int L, int d, int pool) {
  size_t nB = ((size_t)L + pool - 1) / pool;
  size_t nW = ((size_t)L + 15) / 16;
  return (size_t)B * H * (nB + nW) * d * sizeof(float);
}

inline size_t sparge_workspace_bytes(int B, int H, int L, int d, int pool) {
  size_t nB = ((size_t)L + pool - 1) / pool;
  return mask_workspace_bytes(B, H, L, d, pool) + 2 * (size_t)B * H * nB * sizeof(float);
}

}  // namespace ssa
