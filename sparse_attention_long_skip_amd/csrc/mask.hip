// Pooled-score block mask (block-sparse prefill predictor) for gfx950.
//
// Operation (MInference page, block-sparse pattern: mean-pool Q and K per
// block and score block pairs with the pooled vectors, since pooling
// commutes with the matrix product; its block_sparse_attention(topk=64);
// NOSA page, section 3: init_blocks=1 and window_size=1024 are kept besides
// the top-k):
//   q_bar[b], k_bar[c] = means over the rows of each block of `pool` tokens;
//   score(b, c) = q_bar[b] . k_bar[c] / sqrt(d), c <= b;
//   kept(b) = top-k by score (ties: lower c) + sink blocks + local window,
//   written in ascending order.
//
// Kernels: (1) pool -- one workgroup per (block, head, batch, Q-or-K), a
// single coalesced pass over Q and K (the HBM-bound part); (2) select -- one
// workgroup per (4 query blocks, head, batch): scores into LDS as 64-bit
// keys (order-preserving float bits, then the inverted index so that equal
// scores put the lower index first); then one wave per row finds the top-k
// threshold by radix selection with ballot counts and compacts the kept set
// in ascending order.
#include "common.h"
#include "launch.h"

namespace ssa {

namespace {

struct MaskArgs {
  const uint16_t* q;
  const uint16_t* k;
  float* qbar;  // [B, H, nB, D]
  float* kbar;  // [B, H, nB, D]
  int32_t* block_idx;
  int32_t* block_cnt;
  float* block_scores;
  int B, H, L, nB, nBp, pool, topk, sink, W, max_blocks;
  float inv_sqrt_d;
};

template <int D>
__global__ __launch_bounds__(256) void pool_kernel(MaskArgs a) {
  constexpr int CPR = D / 8;
  constexpr int RG = 256 / CPR;
  __shared__ float part[RG][D + 1];
  const int blk = blockIdx.x;
  const int hh = blockIdx.y;
  const int b = blockIdx.z >> 1;
  const bool is_k = blockIdx.z & 1;
  const uint16_t* src = (is_k ? a.k : a.q) + ((size_t)b * a.H + hh) * a.L * D;
  float* dst = (is_k ? a.kbar : a.qbar) + (((size_t)b * a.H + hh) * a.nB + blk) * D;
  const int r0 = blk * a.pool;
  const int r1 = min(a.L, r0 + a.pool);
  const int t = threadIdx.x;
  const int cc = t % CPR;
  const int rg = t / CPR;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = r0 + rg; r < r1; r += RG) {
    const u32x4 x = load16(src + (size_t)r * D + cc * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_lo(x[e]);
      acc[2 * e + 1] += bf16_hi(x[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][cc * 8 + e] = acc[e];
  __syncthreads();
  if (t < D) {
    float s = 0.f;
    for (int g = 0; g < RG; ++g) s += part[g][t];
    dst[t] = s / (float)(r1 - r0);
  }
}

__device__ __forceinline__ uint32_t order_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One workgroup per (QPB consecutive query blocks, head, batch). Scores of
// every causal candidate are turned into 64-bit keys (order-preserving float
// bits, then the inverted index, so a larger key is a higher score or, on a
// tie, a lower index). A candidate is in the top-k iff its key is at least
// the topk-th largest key. The kept set is compacted in ascending order with
// wave ballots.
template <int D, int QPB>
__global__ __launch_bounds__(256) void select_kernel(MaskArgs a) {
  constexpr int NT = 256;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ float qv[QPB][D];
  const int qb0 = blockIdx.x * QPB;
  const int hh = blockIdx.y;
  const int b = blockIdx.z;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = t >> 6;
  const int nq = min(QPB, a.nB - qb0);
  const int N_max = qb0 + nq;  // candidates 0 .. N_max - 1 cover every row here
  const int nBp = a.nBp;
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);  // [QPB][nBp]

  const size_t hb = (size_t)b * a.H + hh;
  for (int x = t; x < nq * D; x += NT) qv[x / D][x % D] = a.qbar[(hb * a.nB + qb0 + x / D) * D + x % D];
  __syncthreads();

  // Scores: each pooled key row is read once for all QPB query blocks.
  const float* kb = a.kbar + hb * a.nB * D;
  for (int c = t; c < N_max; c += NT) {
    float acc[QPB];
#pragma unroll
    for (int q = 0; q < QPB; ++q) acc[q] = 0.f;
    const float* kr = kb + (size_t)c * D;
#pragma unroll 4
    for (int e = 0; e < D; e += 4) {
      const f32x4 kx = *reinterpret_cast<const f32x4*>(kr + e);
#pragma unroll
      for (int q = 0; q < QPB; ++q) {
        acc[q] = fmaf(qv[q][e], kx[0], acc[q]);
        acc[q] = fmaf(qv[q][e + 1], kx[1], acc[q]);
        acc[q] = fmaf(qv[q][e + 2], kx[2], acc[q]);
        acc[q] = fmaf(qv[q][e + 3], kx[3], acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < QPB; ++q) {
      if (q >= nq) break;
      const int qb = qb0 + q;
      uint64_t key = 0;
      if (c <= qb) {
        const float sc = acc[q] * a.inv_sqrt_d;
        if (a.block_scores) a.block_scores[(hb * a.nB + qb) * a.nB + c] = sc;
        key = ((uint64_t)order_bits(sc) << 32) | (uint64_t)(0xffffffffu - (uint32_t)c);
      }
      keys[q * nBp + c] = key;
    }
  }
  if (a.block_scores)
    for (int q = 0; q < nq; ++q)
      for (int c = qb0 + q + 1 + t; c < a.nB; c += NT)
        a.block_scores[(hb * a.nB + qb0 + q) * a.nB + c] = -INFINITY;
  __syncthreads();

  // Selection: wave wv owns row qb0 + wv (QPB == 4 rows per workgroup, or
  // one row handled by wave 0). The top-k threshold is the topk-th largest
  // key T: the largest value with #{key >= T} >= topk (keys are distinct,
  // so exactly topk keys are >= T), found by a 64-round radix selection
  // whose counts are wave ballots; no barriers.
  constexpr int NREG = 8;  // rows with at most 512 candidates keep keys in registers
  const int q = (QPB == 1) ? 0 : wv;
  if ((QPB == 1 && wv != 0) || q >= nq) return;
  const int qb = qb0 + q;
  const int N = qb + 1;
  const uint64_t* kq = keys + q * nBp;
  const int nch = (N + 63) / 64;
  uint64_t kr[NREG];
  const bool in_reg = nch <= NREG;
  if (in_reg) {
#pragma unroll
    for (int r = 0; r < NREG; ++r) kr[r] = (r * 64 + lane < N) ? kq[r * 64 + lane] : 0ull;
  }
  auto key_at = [&](int r) -> uint64_t {
    if (in_reg) {
      uint64_t v = 0;
#pragma unroll
      for (int rr = 0; rr < NREG; ++rr) v = (rr == r) ? kr[rr] : v;
      return v;
    }
    const int c = r * 64 + lane;
    return c < N ? kq[c] : 0ull;
  };
  uint64_t thr = 0;
  const bool by_score = a.topk > 0 && a.topk < N;
  if (by_score) {
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t cand = thr | (1ull << bit);
      int cnt = 0;
      if (in_reg) {
#pragma unroll
        for (int r = 0; r < NREG; ++r) cnt += __popcll(__ballot(kr[r] >= cand));
      } else {
        for (int r = 0; r < nch; ++r) cnt += __popcll(__ballot(key_at(r) >= cand));
      }
      if (cnt >= a.topk) thr = cand;
    }
  }
  const bool all_top = a.topk >= N;
  int32_t* out = a.block_idx + (hb * a.nB + qb) * a.max_blocks;
  int base = 0;
  for (int r = 0; r < nch; ++r) {
    const int c = r * 64 + lane;
    bool kept = false;
    if (c < N) kept = (c < a.sink) || (c >= N - a.W) || all_top || (by_score && key_at(r) >= thr);
    const uint64_t bal = __ballot(kept);
    if (kept) out[base + __popcll(bal & ((1ull << lane) - 1ull))] = c;
    base += __popcll(bal);
  }
  for (int r = base + lane; r < a.max_blocks; r += 64) out[r] = -1;
  if (lane == 0) a.block_cnt[hb * a.nB + qb] = base;
}

template <int D>
hipError_t launch(const MaskArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((pool_kernel<D>), dim3(a.nB, a.H, a.B * 2), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.nB <= 1024) {
    constexpr int QPB = 4;
    const size_t shm = (size_t)QPB * a.nBp * sizeof(uint64_t);
    hipLaunchKernelGGL((select_kernel<D, QPB>), dim3((a.nB + QPB - 1) / QPB, a.H, a.B), dim3(256), shm,
                       stream, a);
  } else {
    const size_t shm = (size_t)a.nBp * sizeof(uint64_t);
    hipLaunchKernelGGL((select_kernel<D, 1>), dim3(a.nB, a.H, a.B), dim3(256), shm, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_mask(const MaskParams& p, hipStream_t stream) {
  MaskArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.B = p.B;
  a.H = p.H;
  a.L = p.L;
  a.pool = p.pool;
  a.nB = (p.L + p.pool - 1) / p.pool;
  a.nBp = a.nB;
  a.topk = p.topk;
  a.sink = p.sink_blocks;
  a.W = p.window_tokens > 0 ? (p.window_tokens + p.pool - 1) / p.pool : 0;
  a.max_blocks = p.max_blocks;
  a.block_idx = p.block_idx;
  a.block_cnt = p.block_cnt;
  a.block_scores = p.block_scores;
  a.qbar = static_cast<float*>(p.workspace);
  a.kbar = a.qbar + (size_t)p.B * p.H * a.nB * p.d;
  a.inv_sqrt_d = 1.f / sqrtf((float)p.d);
  if (p.d == 128) return launch<128>(a, stream);
  if (p.d == 64) return launch<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ssa
