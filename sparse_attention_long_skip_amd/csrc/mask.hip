// Block-sparse prefill predictors for gfx950: the pooled-score top-k mask
// and the SpargeAttn stage-one mask.
//
// Top-k mask (MInference page, block-sparse pattern: mean-pool Q and K per
// block and score block pairs with the pooled vectors, since pooling
// commutes with the matrix product; its block_sparse_attention(topk=64);
// NOSA page, section 3: init_blocks=1 and window_size=1024 are kept besides
// the top-k):
//   q_bar[b], k_bar[c] = means over the rows of each block of `pool` tokens;
//   score(b, c) = q_bar[b] . k_bar[c] / sqrt(d), c <= b;
//   kept(b) = top-k by score (ties: lower c) + sink blocks + local window,
//   written in ascending order.
//
// SpargeAttn stage one (SpargeAttn page, two-stage online filter, "sparse
// block online prediction"): a block whose tokens have a mean pairwise
// cosine similarity above theta is compressed to its mean token; the
// compressed map P_hat[b, :] is a softmax of the pooled scores over the
// compressed key blocks c <= b; the Top-tau of them (by P_hat mass, or by
// count) are kept; uncompressed key blocks are always kept and an
// uncompressed query block keeps every causal block.
//
// Kernels: (1) pool -- one workgroup per (block, head, batch, Q-or-K), a
// single coalesced pass over Q and K (the HBM-bound part), optionally also
// the block self-similarity ||mean of the unit rows||^2; (2) select -- one
// workgroup per (4 query blocks, head, batch): scores into LDS as 44-bit
// keys (order-preserving float bits, then the inverted index so that equal
// scores put the lower index first); then one wave per row finds the cut by
// radix selection over the keys below their common prefix, with ballot counts (top-k, Top-tau count)
// or wave sums of P_hat (Top-tau mass), and compacts the kept set in
// ascending order.
#include "common.h"
#include "launch.h"

namespace ssa {

namespace {

struct MaskArgs {
  const uint16_t* q;
  const uint16_t* k;
  float* qbar;  // [B, H, nB, D]
  float* kbar;  // mean keys [B, H, D / 4, nB, 4] (4-channel groups, so that
                //   consecutive blocks are adjacent); compressed windows
                //   [B, H, nW, D]
  int32_t* block_idx;
  int32_t* block_cnt;
  float* block_scores;
  float* simq;       // [B, H, nB] block self-similarity of Q (SpargeAttn mode)
  float* simk;       // [B, H, nB] same for K
  float* block_sim;  // nullable [B, H, 2, nB]: copies of simq, simk
  int B, H, L, nB, nBp, pool, topk, sink, W, max_blocks;
  float inv_sqrt_d;
  float theta;  // compression threshold on the self-similarity
  float tau;    // Top-tau share (mass mode compares in fp32)
  double tau_d; // the same share, for ceil(tau * n) in fp64 (count mode)
  int tau_mode; // 0: P_hat mass, 1: count
  int nW;       // compressed key windows (overlap mode): ceil(L / kStride)
  int q_only;   // pool kernel: grid z = batch, queries only
};

// Overlapping key compression (NOSA page, section 1: CompressK with
// kernel_size=32, stride=16): window m averages keys [16m, 16m + 32); a key
// block of 64 tokens owns the 4 windows that start inside it.
constexpr int kStride = 16;
constexpr int kKernel = 32;
constexpr int kWinPerBlock = 64 / kStride;

template <int D, bool SIM>
__global__ __launch_bounds__(256) void pool_kernel(MaskArgs a) {
  constexpr int CPR = D / 8;  // lanes per row (8 channels each), a power of two within a wave
  constexpr int RG = 256 / CPR;
  __shared__ float part[SIM ? 2 : 1][RG][D + 1];
  __shared__ float red[4];
  const int blk = blockIdx.x;
  const int hh = blockIdx.y;
  const int b = a.q_only ? blockIdx.z : (blockIdx.z >> 1);
  const bool is_k = a.q_only ? false : (blockIdx.z & 1);
  const size_t hb = (size_t)b * a.H + hh;
  const uint16_t* src = (is_k ? a.k : a.q) + hb * a.L * D;
  float* dst = (is_k ? a.kbar : a.qbar) + (hb * a.nB + blk) * D;
  const int r0 = blk * a.pool;
  const int r1 = min(a.L, r0 + a.pool);
  const int t = threadIdx.x;
  const int cc = t % CPR;
  const int rg = t / CPR;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float accn[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // The trip count depends on rg only, so the CPR lanes of one row are
  // active together and the row-norm shuffles stay within active lanes.
  for (int r = r0 + rg; r < r1; r += RG) {
    const u32x4 x = load16(src + (size_t)r * D + cc * 8);
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16_lo(x[e]);
      f[2 * e + 1] = bf16_hi(x[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += f[e];
    if constexpr (SIM) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
#pragma unroll
      for (int o = CPR / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
      const float inv = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;  // a zero row adds nothing
#pragma unroll
      for (int e = 0; e < 8; ++e) accn[e] = fmaf(f[e], inv, accn[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    part[0][rg][cc * 8 + e] = acc[e];
    if constexpr (SIM) part[SIM ? 1 : 0][rg][cc * 8 + e] = accn[e];
  }
  sync_lds();
  const float n = (float)(r1 - r0);
  float un = 0.f;
  if (t < D) {
    float sm = 0.f, sn = 0.f;
    for (int g = 0; g < RG; ++g) {
      sm += part[0][g][t];
      if constexpr (SIM) sn += part[SIM ? 1 : 0][g][t];
    }
    if (is_k)  // 4-channel groups: the selection reads one group of 64 blocks per load
      a.kbar[((hb * (D / 4) + t / 4) * a.nB + blk) * 4 + (t & 3)] = sm / n;
    else
      dst[t] = sm / n;
    un = sn / n;  // channel t of the mean unit row
  }
  if constexpr (SIM) {
    // self-similarity = squared norm of the mean unit row (threads >= D add 0)
    const float w = wave_sum(un * un);
    if ((t & (kWave - 1)) == 0) red[t / kWave] = w;
    sync_lds();
    if (t == 0) {
      const float sim = red[0] + red[1] + red[2] + red[3];
      (is_k ? a.simk : a.simq)[hb * a.nB + blk] = sim;
      if (a.block_sim) a.block_sim[(hb * 2 + (is_k ? 1 : 0)) * a.nB + blk] = sim;
    }
  }
}

// Compressed keys of one 64-token block: the rows [64 blk, 64 blk + 80) (cut
// at L) are staged in LDS as bf16, then each thread sums one channel of one
// window. One workgroup per (block, head, batch).
template <int D>
__global__ __launch_bounds__(256) void compress_k_kernel(MaskArgs a) {
  constexpr int CPR = D / 8;
  constexpr int ROWS = (kWinPerBlock - 1) * kStride + kKernel;  // 80
  __shared__ __attribute__((aligned(16))) uint16_t rows[ROWS][D];
  const int blk = blockIdx.x;
  const size_t hb = (size_t)blockIdx.z * a.H + blockIdx.y;
  const uint16_t* src = a.k + hb * a.L * D;
  const int r0 = blk * 64;
  const int nr = min(ROWS, a.L - r0);
  const int t = threadIdx.x;
  for (int x = t; x < nr * CPR; x += 256) {
    const int r = x / CPR, cc = x % CPR;
    store16(&rows[r][cc * 8], load16(src + (size_t)(r0 + r) * D + cc * 8));
  }
  sync_lds();
  const int ch = t % D;
  for (int w = t / D; w < kWinPerBlock; w += 256 / D) {
    const int m = blk * kWinPerBlock + w;
    if (m >= a.nW) break;
    const int lo = w * kStride;
    const int hi = min(lo + kKernel, nr);
    float acc = 0.f;
    for (int r = lo; r < hi; ++r) acc += __uint_as_float((uint32_t)rows[r][ch] << 16);
    a.kbar[(hb * a.nW + m) * D + ch] = acc / (float)(hi - lo);
  }
}

__device__ __forceinline__ uint32_t order_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_order_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o, kWave));
  return x;
}

// Selection keys: order-preserving score bits above a 12-bit inverted block
// index (nB <= 4096), so a larger key is a higher score or, on a tie, a
// lower index. Key 0 is "no candidate".
constexpr int kIdxBits = 12;
constexpr uint32_t kIdxMask = (1u << kIdxBits) - 1;

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t x, int o) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, o, kWave);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), o, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// One workgroup per (QPB consecutive query blocks, head, batch). Scores of
// every causal candidate are turned into 44-bit keys (order-preserving float
// bits, then the 12-bit inverted index, so a larger key is a higher score
// or, on a tie, a lower index). A candidate is in the top-k iff its key is at least
// the topk-th largest key. The kept set is compacted in ascending order with
// wave ballots.
template <int D, int QPB, bool SPARGE, bool COMP>
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
  sync_lds();

  // Scores: each pooled key row is read once for all QPB query blocks. With
  // compressed keys a block's score is the best of its windows.
  const float* kb = a.kbar + hb * (COMP ? (size_t)a.nW : (size_t)a.nB) * D;
  for (int c = t; c < N_max; c += NT) {
    float acc[QPB];
#pragma unroll
    for (int q = 0; q < QPB; ++q) acc[q] = -INFINITY;
    const int nwin = COMP ? min(kWinPerBlock, a.nW - c * kWinPerBlock) : 1;
    for (int w = 0; w < nwin; ++w) {
      // compressed windows are rows of D; mean keys come in 4-channel groups
      const float* kr = COMP ? kb + (size_t)(c * kWinPerBlock + w) * D : kb + (size_t)c * 4;
      const size_t kstep = COMP ? 4 : (size_t)a.nB * 4;
      float part[QPB];
#pragma unroll
      for (int q = 0; q < QPB; ++q) part[q] = 0.f;
#pragma unroll 4
      for (int e = 0; e < D; e += 4) {
        const f32x4 kx = *reinterpret_cast<const f32x4*>(kr + (size_t)(e / 4) * kstep);
#pragma unroll
        for (int q = 0; q < QPB; ++q) {
          part[q] = fmaf(qv[q][e], kx[0], part[q]);
          part[q] = fmaf(qv[q][e + 1], kx[1], part[q]);
          part[q] = fmaf(qv[q][e + 2], kx[2], part[q]);
          part[q] = fmaf(qv[q][e + 3], kx[3], part[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < QPB; ++q) acc[q] = fmaxf(acc[q], part[q]);
    }
#pragma unroll
    for (int q = 0; q < QPB; ++q) {
      if (q >= nq) break;
      const int qb = qb0 + q;
      uint64_t key = 0;
      if (c <= qb) {
        const float sc = acc[q] * a.inv_sqrt_d;
        if (a.block_scores) a.block_scores[(hb * a.nB + qb) * a.nB + c] = sc;
        key = ((uint64_t)order_bits(sc) << kIdxBits) | (uint64_t)(kIdxMask - (uint32_t)c);
      }
      keys[q * nBp + c] = key;
    }
  }
  if (a.block_scores)
    for (int q = 0; q < nq; ++q)
      for (int c = qb0 + q + 1 + t; c < a.nB; c += NT)
        a.block_scores[(hb * a.nB + qb0 + q) * a.nB + c] = -INFINITY;
  sync_lds();

  // Selection: wave wv owns row qb0 + wv (QPB == 4 rows per workgroup, or
  // one row handled by wave 0). The top-k threshold is the topk-th largest
  // key T: the largest value with #{key >= T} >= topk (keys are distinct,
  // so exactly topk keys are >= T), found by a radix descent over the bits
  // below the row's common key prefix, with wave-ballot counts; no barriers.
  constexpr int NREG = 8;  // rows with at most 512 candidates keep keys in registers
  const int q = (QPB == 1) ? 0 : wv;
  if ((QPB == 1 && wv != 0) || q >= nq) return;
  const int qb = qb0 + q;
  const int N = qb + 1;
  uint64_t* kq = keys + q * nBp;
  const int nch = (N + 63) / 64;
  uint64_t kr[NREG];
  float pr[NREG] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
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
  // The live (nonzero) keys share their bits above `top`: the descent starts
  // from that common prefix. Returns top (-1 when at most one distinct live
  // key exists, then *thr0 is that key or 0).
  auto common_prefix = [&](uint64_t* thr0) -> int {
    uint64_t ka = ~0ull, ko = 0ull;
    for (int r = 0; r < nch; ++r) {
      const uint64_t kv = key_at(r);
      if (kv) {
        ka &= kv;
        ko |= kv;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      ka &= shfl_xor64(ka, o);
      ko |= shfl_xor64(ko, o);
    }
    if (ko == 0ull || ka == ko) {
      *thr0 = ko;
      return -1;
    }
    const int top = 63 - __clzll((long long)(ka ^ ko));
    *thr0 = top == 63 ? 0ull : (ka & ~((2ull << top) - 1ull));
    return top;
  };
  // Largest key T with #{keys >= T} >= need (zero keys never count).
  auto select_by_count = [&](int need) -> uint64_t {
    uint64_t thr;
    const int top = common_prefix(&thr);
    for (int bit = top; bit >= 0; --bit) {
      const uint64_t cand = thr | (1ull << bit);
      int cnt = 0;
      if (in_reg) {
#pragma unroll
        for (int r = 0; r < NREG; ++r) cnt += __popcll(__ballot(kr[r] >= cand));
      } else {
        for (int r = 0; r < nch; ++r) cnt += __popcll(__ballot(key_at(r) >= cand));
      }
      if (cnt >= need) thr = cand;
    }
    return thr;
  };
  int32_t* out = a.block_idx + (hb * a.nB + qb) * a.max_blocks;
  int base = 0;
  if constexpr (!SPARGE) {
    const uint64_t thr = (a.topk > 0 && a.topk < N) ? select_by_count(a.topk) : 0ull;
    const bool by_score = a.topk > 0 && a.topk < N;
    const bool all_top = a.topk >= N;
    for (int r = 0; r < nch; ++r) {
      const int c = r * 64 + lane;
      bool kept = false;
      if (c < N) kept = (c < a.sink) || (c >= N - a.W) || all_top || (by_score && key_at(r) >= thr);
      const uint64_t bal = __ballot(kept);
      if (kept) out[base + __popcll(bal & ((1ull << lane) - 1ull))] = c;
      base += __popcll(bal);
    }
  } else {
    // Compressed candidates keep their keys; the others get key 0 (never
    // selected, always kept). P_hat mass per candidate is exp(s - s_max);
    // the normalisation is folded into the target tau * Z.
    float* pq = reinterpret_cast<float*>(keys + QPB * nBp) + q * nBp;
    const float* sk = a.simk + hb * a.nB;
    const bool dense_row = !(a.simq[hb * a.nB + qb] > a.theta);
    uint64_t thr = 0;
    if (!dense_row) {
      int ncomp = 0;
      uint32_t hi = 0;
      for (int r = 0; r < nch; ++r) {
        const int c = r * 64 + lane;
        const bool comp = c < N && sk[c] > a.theta;
        const uint64_t kv = comp ? key_at(r) : 0ull;
        if (in_reg) {
#pragma unroll
          for (int rr = 0; rr < NREG; ++rr) kr[rr] = (rr == r) ? kv : kr[rr];
        } else if (c < N) {
          kq[c] = kv;
        }
        ncomp += __popcll(__ballot(comp));
        hi = max(hi, (uint32_t)(kv >> kIdxBits));
      }
      if (ncomp > 0) {
        if (a.tau_mode == 1) {
          const int need = (int)ceil(a.tau_d * (double)ncomp);
          thr = need >= ncomp ? 1ull : select_by_count(need);
        } else {
          const float smax = from_order_bits(wave_max_u32(hi));
          constexpr float kLog2e = 1.4426950408889634f;
          float zl = 0.f;
          for (int r = 0; r < nch; ++r) {
            const uint64_t kv = key_at(r);
            const float p = kv ? fast_exp2((from_order_bits((uint32_t)(kv >> kIdxBits)) - smax) * kLog2e) : 0.f;
            if (in_reg) {
#pragma unroll
              for (int rr = 0; rr < NREG; ++rr) pr[rr] = (rr == r) ? p : pr[rr];
            } else if (r * 64 + lane < N) {
              pq[r * 64 + lane] = p;
            }
            zl += p;
          }
          // Mass of {key >= T}: fp32 sums of non-negative terms in a fixed
          // order, so it never grows with T and the radix descent is exact
          // for this predicate. The full set (T = 1) has mass Z >= tau * Z.
          const float target = a.tau * wave_sum(zl);
          const int top = common_prefix(&thr);
          for (int bit = top; bit >= 0; --bit) {
            const uint64_t cand = thr | (1ull << bit);
            float m = 0.f;
            if (in_reg) {
#pragma unroll
              for (int r = 0; r < NREG; ++r) m += kr[r] >= cand ? pr[r] : 0.f;
            } else {
              for (int r = 0; r < nch; ++r) {
                const int c = r * 64 + lane;
                m += (c < N && kq[c] >= cand) ? pq[c] : 0.f;
              }
            }
            if (wave_sum(m) >= target) thr = cand;
          }
        }
      }
    }
    for (int r = 0; r < nch; ++r) {
      const int c = r * 64 + lane;
      bool kept = false;
      if (c < N) {
        const uint64_t kv = dense_row ? 0ull : key_at(r);
        kept = dense_row || kv == 0ull || kv >= thr;
      }
      const uint64_t bal = __ballot(kept);
      if (kept) out[base + __popcll(bal & ((1ull << lane) - 1ull))] = c;
      base += __popcll(bal);
    }
  }
  for (int r = base + lane; r < a.max_blocks; r += 64) out[r] = -1;
  if (lane == 0) a.block_cnt[hb * a.nB + qb] = base;
}

template <int D, bool SPARGE, bool COMP>
hipError_t launch(const MaskArgs& a, hipStream_t stream) {
  if (COMP) {
    // query blocks: plain means; keys: overlapping windows
    MaskArgs aq = a;
    aq.q_only = 1;
    hipLaunchKernelGGL((pool_kernel<D, false>), dim3(a.nB, a.H, a.B), dim3(256), 0, stream, aq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((compress_k_kernel<D>), dim3(a.nB, a.H, a.B), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((pool_kernel<D, SPARGE>), dim3(a.nB, a.H, a.B * 2), dim3(256), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t per_row = sizeof(uint64_t) + (SPARGE ? sizeof(float) : 0);
  if (a.nB <= 1024) {
    constexpr int QPB = 4;
    hipLaunchKernelGGL((select_kernel<D, QPB, SPARGE, COMP>), dim3((a.nB + QPB - 1) / QPB, a.H, a.B),
                       dim3(256), QPB * a.nBp * per_row, stream, a);
  } else {
    hipLaunchKernelGGL((select_kernel<D, 1, SPARGE, COMP>), dim3(a.nB, a.H, a.B), dim3(256),
                       a.nBp * per_row, stream, a);
  }
  return hipGetLastError();
}

MaskArgs common_args(const MaskParams& p) {
  MaskArgs a = {};
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.B = p.B;
  a.H = p.H;
  a.L = p.L;
  a.pool = p.pool;
  a.nB = (p.L + p.pool - 1) / p.pool;
  a.nBp = a.nB;
  a.max_blocks = p.max_blocks;
  a.block_idx = p.block_idx;
  a.block_cnt = p.block_cnt;
  a.block_scores = p.block_scores;
  a.qbar = static_cast<float*>(p.workspace);
  a.kbar = a.qbar + (size_t)p.B * p.H * a.nB * p.d;
  a.inv_sqrt_d = 1.f / sqrtf((float)p.d);
  return a;
}

}  // namespace

hipError_t launch_block_mask(const MaskParams& p, hipStream_t stream) {
  MaskArgs a = common_args(p);
  a.topk = p.topk;
  a.sink = p.sink_blocks;
  a.W = p.window_tokens > 0 ? (p.window_tokens + p.pool - 1) / p.pool : 0;
  a.nW = (p.L + kStride - 1) / kStride;
  if (p.compressed) {
    if (p.d == 128) return launch<128, false, true>(a, stream);
    if (p.d == 64) return launch<64, false, true>(a, stream);
  } else {
    if (p.d == 128) return launch<128, false, false>(a, stream);
    if (p.d == 64) return launch<64, false, false>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_sparge_mask(const SpargeParams& p, hipStream_t stream) {
  MaskArgs a = common_args(p.m);
  const size_t per_head = (size_t)p.m.B * p.m.H * a.nB;
  a.simq = a.kbar + per_head * p.m.d;
  a.simk = a.simq + per_head;
  a.block_sim = p.block_sim;
  a.theta = p.theta;
  a.tau = (float)p.tau;
  a.tau_d = p.tau;
  a.tau_mode = p.tau_mode;
  if (p.m.d == 128) return launch<128, true, false>(a, stream);
  if (p.m.d == 64) return launch<64, true, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ssa
