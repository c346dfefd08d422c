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
// workgroup per (query block, head, batch): scores into LDS as 64-bit sort
// keys (order-preserving float bits, then the inverted index so that equal
// scores put the lower index first), a bitonic sort, flags for the kept
// set, and an ordered compaction.
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
  int B, H, L, nB, pool, topk, sink, W, max_blocks;
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

template <int D>
__global__ __launch_bounds__(256) void select_kernel(MaskArgs a) {
  constexpr int NT = 256;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ float qv[D];
  __shared__ int seg_count[NT];
  const int qb = blockIdx.x;
  const int hh = blockIdx.y;
  const int b = blockIdx.z;
  const int t = threadIdx.x;
  const int N = qb + 1;  // causal candidates 0..qb
  int Np = 1;
  while (Np < N) Np <<= 1;
  const int nBp = [&] { int x = 1; while (x < a.nB) x <<= 1; return x; }();
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);
  unsigned char* flags = smem + (size_t)nBp * sizeof(uint64_t);

  const size_t hb = (size_t)b * a.H + hh;
  if (t < D) qv[t] = a.qbar[(hb * a.nB + qb) * D + t];
  __syncthreads();

  const float* kb = a.kbar + hb * a.nB * D;
  for (int c = t; c < Np; c += NT) {
    uint64_t key = 0;
    if (c < N) {
      const float* kr = kb + (size_t)c * D;
      float s = 0.f;
#pragma unroll 8
      for (int e = 0; e < D; e += 4) {
        const f32x4 kx = *reinterpret_cast<const f32x4*>(kr + e);
        s = fmaf(qv[e], kx[0], s);
        s = fmaf(qv[e + 1], kx[1], s);
        s = fmaf(qv[e + 2], kx[2], s);
        s = fmaf(qv[e + 3], kx[3], s);
      }
      s *= a.inv_sqrt_d;
      if (a.block_scores) a.block_scores[(hb * a.nB + qb) * a.nB + c] = s;
      key = ((uint64_t)order_bits(s) << 32) | (uint64_t)(0xffffffffu - (uint32_t)c);
    }
    keys[c] = key;
    if (c < N) flags[c] = 0;
  }
  if (a.block_scores)
    for (int c = N + t; c < a.nB; c += NT) a.block_scores[(hb * a.nB + qb) * a.nB + c] = -INFINITY;
  __syncthreads();

  // Bitonic sort, descending.
  for (int kk = 2; kk <= Np; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int i = t; i < Np; i += NT) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const uint64_t x = keys[i], y = keys[ixj];
          const bool desc = (i & kk) == 0;
          if (desc ? (x < y) : (x > y)) {
            keys[i] = y;
            keys[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  const int ntop = min(a.topk, N);
  for (int r = t; r < ntop; r += NT) flags[0xffffffffu - (uint32_t)(keys[r] & 0xffffffffu)] = 1;
  for (int c = t; c < min(a.sink, N); c += NT) flags[c] = 1;
  for (int c = max(0, N - a.W) + t; c < N; c += NT) flags[c] = 1;
  __syncthreads();

  // Ordered compaction: each thread owns a contiguous segment.
  const int seg = (N + NT - 1) / NT;
  const int c0 = min(N, t * seg), c1 = min(N, c0 + seg);
  int cnt = 0;
  for (int c = c0; c < c1; ++c) cnt += flags[c];
  seg_count[t] = cnt;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const int v = (t >= off) ? seg_count[t - off] : 0;
    __syncthreads();
    seg_count[t] += v;
    __syncthreads();
  }
  const int total = seg_count[NT - 1];
  int pos = seg_count[t] - cnt;
  int32_t* out = a.block_idx + (hb * a.nB + qb) * a.max_blocks;
  for (int c = c0; c < c1; ++c)
    if (flags[c]) out[pos++] = c;
  for (int r = total + t; r < a.max_blocks; r += NT) out[r] = -1;
  if (t == 0) a.block_cnt[hb * a.nB + qb] = total;
}

template <int D>
hipError_t launch(const MaskArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((pool_kernel<D>), dim3(a.nB, a.H, a.B * 2), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int nBp = 1;
  while (nBp < a.nB) nBp <<= 1;
  const size_t shm = (size_t)nBp * (sizeof(uint64_t) + 1);
  hipLaunchKernelGGL((select_kernel<D>), dim3(a.nB, a.H, a.B), dim3(256), shm, stream, a);
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
