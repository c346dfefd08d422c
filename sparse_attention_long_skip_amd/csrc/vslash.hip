// Vertical-slash block estimator for gfx950.
//
// Operation (MInference page: the vertical-slash pattern is estimated by
// attending from the last query vector(s) to every key, which gives the best
// vertical lines -- key columns -- and slash lines -- diagonals; its
// vertical_slash_sparse_attention(q, k, v, vertical_topk, slash) call):
//   rows i < R of the last R queries (positions p_i = L - R + i) attend
//   causally, A[i, j] = softmax_{j <= p_i}(q_i . k_j / sqrt(d));
//   v[j] = sum_i A[i, j]; s[o] = sum_i A[i, p_i - o];
//   the n_vertical best keys and n_slash best offsets are chosen (ties: lower
//   index first), and every 64 x 64 tile (b, c <= b) that holds an allowed
//   entry on a chosen line is listed for the block-sparse prefill.
//
// Kernels, one launch each:
//   (1) vs_pass<D, 0>: per chunk of 256 keys, S^T = K Q^T on 32x32x16 bf16
//       MFMA (keys from HBM as the A operand, the R <= 64 query rows held as
//       the B operand), online per-row (max, sum) partials in log2 units;
//   (2) vs_rowstats: per-row max and 1/sum over the chunks;
//   (3) vs_pass<D, 1>: recompute the chunk's scores, A into an LDS tile, then
//       column sums (v, complete) and diagonal sums (partial at the chunk's
//       edges) per chunk;
//   (4) vs_slash_combine: s[o] from the at most two chunks holding offset o,
//       in chunk order (deterministic);
//   (5) vs_select: one workgroup per (line kind, head): the n-th largest score
//       by a 4-pass radix select on 8-bit digits (LDS histogram, block scan),
//       ties resolved by index with a block scan; emits per-tile vertical flags, the prefix
//       count of chosen offsets and, optionally, the sorted index lists;
//   (6) vs_cover: one wave per query tile tests every causal key tile with
//       the flags and prefix counts and compacts the list with ballots.
#include "common.h"
#include "launch.h"

namespace ssa {

namespace {

constexpr int CH = kVsChunk;    // keys per chunk (pass kernels)
constexpr int SPW = kVsSpw;     // stride of the per-chunk diagonal partials
constexpr int TILE = 64;        // block-sparse tile (Br = Bc)
constexpr int SEL_T = 1024;     // threads of the selection kernel

struct VsArgs {
  const uint16_t* q;
  const uint16_t* k;
  int B, H, L, R, nchunk, nB, n_vert, n_slash, max_blocks;
  float c_log2;  // log2(e) / sqrt(d)
  float* part;   // [B, H, nchunk, 64, 2] (max, sum) in log2 units
  float* stats;  // [B, H, 64, 2] (max, 1 / sum)
  float* v;      // [B, H, L]
  float* s;      // [B, H, L]
  float* spart;  // [B, H, nchunk, SPW]
  int32_t* vt;   // [B, H, nB] tile holds a chosen vertical
  int32_t* P;    // [B, H, L + 1] chosen offsets below o
  int32_t* block_idx;
  int32_t* block_cnt;
  int32_t* vert_idx;   // nullable [B, H, n_vert]
  int32_t* slash_idx;  // nullable [B, H, n_slash]
  float* v_out;        // nullable [B, H, L]
  float* s_out;        // nullable [B, H, L]
};

__device__ __forceinline__ uint32_t order_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int D, int PASS>
__global__ __launch_bounds__(256) void vs_pass(VsArgs a) {
  constexpr int KS = D / 16;  // MFMA k-steps
  __shared__ float A_lds[PASS ? 32 : 1][CH + 1];  // one half (32 query rows) of the A tile
  __shared__ float red[4][64][2];
  const int chunk = blockIdx.x;
  const size_t hb = (size_t)blockIdx.z * a.H + blockIdx.y;
  const uint16_t* kp = a.k + hb * a.L * D;
  const uint16_t* qp = a.q + hb * a.L * D;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = t >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;
  const int j0 = chunk * CH;

  // B operand: query rows rb * 32 + col (zero beyond R), 16 d-elements per step.
  bf16x8 qop[2][KS];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int i = rb * 32 + col;
    const bool ok = i < a.R;
    const uint16_t* row = qp + (size_t)(a.L - a.R + (ok ? i : 0)) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < KS; ++s) qop[rb][s] = ok ? as_bf16x8(load16(row + 16 * s)) : bf16x8{};
  }
  float mrow[2] = {0.f, 0.f}, invl[2] = {0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  if constexpr (PASS == 1) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int i = rb * 32 + col;
      mrow[rb] = i < a.R ? a.stats[(hb * 64 + i) * 2] : 0.f;
      invl[rb] = i < a.R ? a.stats[(hb * 64 + i) * 2 + 1] : 0.f;
    }
  }

  // S^T tile of keys g * 32 .. g * 32 + 31 of the chunk against both row blocks
  auto scores = [&](int g, f32x16* acc) __attribute__((always_inline)) {
    const int jk = j0 + g * 32 + col;  // this lane's key for the A operand
    bf16x8 kop[KS];
    const uint16_t* krow = kp + (size_t)(jk < a.L ? jk : 0) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < KS; ++s) kop[s] = jk < a.L ? as_bf16x8(load16(krow + 16 * s)) : bf16x8{};
    acc[0] = f32x16{};
    acc[1] = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      acc[0] = mfma32(kop[s], qop[0][s], acc[0]);
      acc[1] = mfma32(kop[s], qop[1][s], acc[1]);
    }
  };
  if constexpr (PASS == 1) {
    // The A tile goes through LDS one 32-row half at a time (half the LDS,
    // so twice the workgroups per CU); the column and diagonal sums carry
    // their running totals across the halves, adding rows in the same
    // increasing order as over the whole tile.
    constexpr int NG = CH / 32 / 4;  // key groups per wave
    f32x16 acc[NG][2];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) scores(wv + 4 * gi, acc[gi]);
    float csum = 0.f;
    float dsum[2] = {0.f, 0.f};  // diagonals e = t and e = t + 256
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      sync_lds();  // the previous half has been read
      const int i = rb * 32 + col;
      const int p = a.L - a.R + i;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const int g = wv + 4 * gi;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jl = g * 32 + 8 * (r / 4) + 4 * h + (r % 4);
          const int j = j0 + jl;
          const bool ok = i < a.R && j < a.L && j <= p;
          A_lds[col][jl] = ok ? fast_exp2(acc[gi][rb][r] * a.c_log2 - mrow[rb]) * invl[rb] : 0.f;
        }
      }
      sync_lds();
      const int r_lo = rb * 32, r_hi = min(a.R, rb * 32 + 32);  // rows of this half
      if (j0 + t < a.L)
        for (int r = r_lo; r < r_hi; ++r) csum += A_lds[r - r_lo][t];
      // diagonal e meets row r at chunk column r + CH - 1 - e
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int e = t + 256 * k;
        if (e < CH + a.R - 1) {
          const int i0 = max(max(0, e - CH + 1), r_lo);
          const int i1 = min(min(a.R - 1, e), r_hi - 1);
          for (int r = i0; r <= i1; ++r) dsum[k] += A_lds[r - r_lo][r + CH - 1 - e];
        }
      }
    }
    if (j0 + t < a.L) a.v[hb * a.L + j0 + t] = csum;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = t + 256 * k;
      if (e < CH + a.R - 1) a.spart[(hb * a.nchunk + chunk) * SPW + e] = dsum[k];
    }
    return;
  }

  // pass 0: online (max, sum) of every row over this chunk's keys
  for (int g = wv; g < CH / 32; g += 4) {
    f32x16 acc[2];
    scores(g, acc);
    // lane holds query row rb * 32 + col; register r holds key
    // g * 32 + 8 (r / 4) + 4 h + r % 4 of the chunk
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int i = rb * 32 + col;
      const int p = a.L - a.R + i;
      float mx = m_run[rb];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + g * 32 + 8 * (r / 4) + 4 * h + (r % 4);
        if (i < a.R && j < a.L && j <= p) mx = fmaxf(mx, acc[rb][r] * a.c_log2);
      }
      if (mx != -INFINITY) {
        float l = m_run[rb] == -INFINITY ? 0.f : l_run[rb] * fast_exp2(m_run[rb] - mx);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + g * 32 + 8 * (r / 4) + 4 * h + (r % 4);
          if (i < a.R && j < a.L && j <= p) l += fast_exp2(acc[rb][r] * a.c_log2 - mx);
        }
        m_run[rb] = mx;
        l_run[rb] = l;
      }
    }
  }

  if constexpr (PASS == 0) {
    // the two lanes of a row (h = 0, 1), then the four waves
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float mo = __shfl_xor(m_run[rb], 32, kWave);
      const float lo = __shfl_xor(l_run[rb], 32, kWave);
      const float mx = fmaxf(m_run[rb], mo);
      float l = 0.f;
      if (mx != -INFINITY) {
        if (m_run[rb] != -INFINITY) l += l_run[rb] * fast_exp2(m_run[rb] - mx);
        if (mo != -INFINITY) l += lo * fast_exp2(mo - mx);
      }
      if (h == 0) {
        red[wv][rb * 32 + col][0] = mx;
        red[wv][rb * 32 + col][1] = l;
      }
    }
    sync_lds();
    if (t < 64) {
      float mx = -INFINITY;
      for (int w = 0; w < 4; ++w) mx = fmaxf(mx, red[w][t][0]);
      float l = 0.f;
      if (mx != -INFINITY)
        for (int w = 0; w < 4; ++w)
          if (red[w][t][0] != -INFINITY) l += red[w][t][1] * fast_exp2(red[w][t][0] - mx);
      float* o = a.part + ((hb * a.nchunk + chunk) * 64 + t) * 2;
      o[0] = mx;
      o[1] = l;
    }
  }
}

// Row statistics over the chunks: 16 slices of chunks per row, combined in LDS.
__global__ __launch_bounds__(1024) void vs_rowstats(VsArgs a) {
  constexpr int NSL = 16;
  __shared__ float red[NSL][64][2];
  const size_t hb = (size_t)blockIdx.y * a.H + blockIdx.x;
  const int i = threadIdx.x & 63;
  const int sl = threadIdx.x >> 6;
  float mx = -INFINITY, l = 0.f;
  if (i < a.R) {
    for (int c = sl; c < a.nchunk; c += NSL) {
      const float* p = a.part + ((hb * a.nchunk + c) * 64 + i) * 2;
      const float pm = p[0], pl = p[1];
      if (pm == -INFINITY) continue;
      const float m2 = fmaxf(mx, pm);
      l = (mx == -INFINITY ? 0.f : l * fast_exp2(mx - m2)) + pl * fast_exp2(pm - m2);
      mx = m2;
    }
  }
  red[sl][i][0] = mx;
  red[sl][i][1] = l;
  sync_lds();
  if (sl != 0 || i >= a.R) return;
  float m = -INFINITY;
  for (int k = 0; k < NSL; ++k) m = fmaxf(m, red[k][i][0]);
  float tot = 0.f;
  for (int k = 0; k < NSL; ++k)
    if (red[k][i][0] != -INFINITY) tot += red[k][i][1] * fast_exp2(red[k][i][0] - m);
  a.stats[(hb * 64 + i) * 2] = m;
  a.stats[(hb * 64 + i) * 2 + 1] = 1.f / tot;  // tot >= 1: the row's own max term
}

__global__ __launch_bounds__(256) void vs_slash_combine(VsArgs a) {
  const size_t hb = (size_t)blockIdx.z * a.H + blockIdx.y;
  const int o = blockIdx.x * 256 + threadIdx.x;
  if (o >= a.L) return;
  // chunk c holds offset o at e = y + c * CH, for 0 <= e < CH + R - 1
  const int y = o - a.L + a.R + CH - 1;
  int c = y >= 0 ? 0 : (-y + CH - 1) / CH;
  float sum = 0.f;
  for (; c < a.nchunk && y + c * CH < CH + a.R - 1; ++c)
    sum += a.spart[(hb * a.nchunk + c) * SPW + (y + c * CH)];
  a.s[hb * a.L + o] = sum;
  if (a.s_out) a.s_out[hb * a.L + o] = sum;
  if (a.v_out) a.v_out[hb * a.L + o] = a.v[hb * a.L + o];
}

// Block-wide exclusive prefix sum over thread order.
__device__ int block_exclusive_scan(int x, int* scratch) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += y;
  }
  sync_lds();
  if (lane == 63) scratch[w] = inc;
  sync_lds();
  int before = 0;
  for (int i = 0; i < w; ++i) before += scratch[i];
  return before + inc - x;
}

// Block-wide exclusive prefix sum of 64-bit values; *total gets the sum of all.
__device__ uint64_t block_exclusive_scan64(uint64_t x, uint64_t* scratch, uint64_t* total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  uint64_t inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t lo = __shfl_up((uint32_t)inc, o, kWave);
    const uint32_t hi = __shfl_up((uint32_t)(inc >> 32), o, kWave);
    if (lane >= o) inc += ((uint64_t)hi << 32) | lo;
  }
  sync_lds();
  if (lane == 63) scratch[w] = inc;
  sync_lds();
  uint64_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < SEL_T / 64; ++i) {
    const uint64_t v = scratch[i];
    before += i < w ? v : 0ull;
    all += v;
  }
  *total = all;
  return before + inc - x;
}

__global__ __launch_bounds__(SEL_T) void vs_select(VsArgs a) {
  __shared__ int scratch[SEL_T / 64];
  __shared__ uint64_t scratch64[SEL_T / 64];
  const bool slash = blockIdx.x == 1;
  const size_t hb = (size_t)blockIdx.z * a.H + blockIdx.y;
  const float* x = (slash ? a.s : a.v) + hb * a.L;
  const int n = slash ? a.n_slash : a.n_vert;
  const int L = a.L;
  const int t = threadIdx.x;

  // The n-th largest key T, 8 bits at a time: per pass, a histogram of the
  // next digit over the keys that match the digits found so far, then the
  // largest digit whose suffix count reaches the rank still needed. After
  // the last pass `need` is how many keys equal to T are taken.
  // 16 copies of the histogram (by lane % 16, rows padded to spread banks)
  // so that keys sharing a digit do not all hit one LDS address.
  constexpr int NCOPY = 16, HS = 257;
  __shared__ int hist[NCOPY * HS];
  __shared__ int pick[2];
  uint32_t thr = 0, mask = 0;
  int need = n;
  const bool take_all = n >= L;
  const bool by_rank = n > 0 && !take_all;
  // Up to SEL_T * NR keys are read once into registers (all four passes
  // then run on them); longer rows are re-read every pass.
  constexpr int NR = 32;
  const bool in_reg = L <= SEL_T * NR;
  uint32_t ur[NR];
  if (by_rank && in_reg) {
#pragma unroll
    for (int e = 0; e < NR; ++e) {
      const int j = e * SEL_T + t;
      ur[e] = j < L ? order_bits(x[j]) : 0u;
    }
  }
  if (by_rank) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int e = t; e < NCOPY * HS; e += SEL_T) hist[e] = 0;
      sync_lds();
      int* mine = hist + (t & (NCOPY - 1)) * HS;
      if (in_reg) {
#pragma unroll
        for (int e = 0; e < NR; ++e) {
          const int j = e * SEL_T + t;
          if (j < L && (ur[e] & mask) == thr) atomicAdd(&mine[(ur[e] >> shift) & 255], 1);
        }
      } else {
        for (int b0 = 0; b0 < L; b0 += SEL_T * 8) {  // 8 loads in flight per thread
          uint32_t u[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = b0 + e * SEL_T + t;
            u[e] = j < L ? order_bits(x[j]) : 0u;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = b0 + e * SEL_T + t;
            if (j < L && (u[e] & mask) == thr) atomicAdd(&mine[(u[e] >> shift) & 255], 1);
          }
        }
      }
      sync_lds();
      // thread t looks at digit 255 - t: suffix count S = excl + own
      int own = 0;
      if (t < 256)
        for (int cpy = 0; cpy < NCOPY; ++cpy) own += hist[cpy * HS + 255 - t];
      const int excl = block_exclusive_scan(own, scratch);
      if (t < 256 && excl < need && excl + own >= need) {
        pick[0] = 255 - t;
        pick[1] = need - excl;
      }
      sync_lds();
      thr |= (uint32_t)pick[0] << shift;
      mask |= 255u << shift;
      need = pick[1];
      sync_lds();  // pick is rewritten next pass
    }
  }
  const int need_eq = by_rank ? need : 0;

  // Ordered sweep over steps of SEL_T * PER keys, PER consecutive keys per
  // thread (the next step's keys are loaded before this step's scan): a key
  // above T is taken, a key equal to T is taken while fewer than need_eq
  // equal keys precede it. One block scan of the packed (above, equal)
  // counts per step gives each key's rank. A wave covers 4 tiles of 64 keys
  // (16 lanes each).
  constexpr int PER = 4;
  constexpr int STEP = SEL_T * PER;
  int32_t* list = slash ? a.slash_idx : a.vert_idx;
  const int nlist = slash ? a.n_slash : a.n_vert;
  int32_t* P = a.P + hb * (L + 1);
  auto load_step = [&](int base, float* o) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int j = base + PER * t + e;
      o[e] = (by_rank && j < L) ? x[j] : 0.f;
    }
  };
  float xv[PER], xn[PER] = {};
  load_step(0, xv);
  uint64_t run = 0;  // (above << 32) | equal, over the keys before this step
  for (int base = 0; base < L; base += STEP) {
    if (base + STEP < L) load_step(base + STEP, xn);
    int cc[PER];  // 2: above T, 1: equal to T, 0: not taken
    uint64_t mine = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int j = base + PER * t + e;
      int c = 0;
      if (j < L) {
        if (take_all) {
          c = 2;
        } else if (by_rank) {
          const uint32_t u = order_bits(xv[e]);
          c = u > thr ? 2 : (u == thr ? 1 : 0);
        }
      }
      cc[e] = c;
      mine += c == 2 ? (1ull << 32) : (uint64_t)(c == 1);
    }
    uint64_t total;
    uint64_t acc = run + block_exclusive_scan64(mine, scratch64, &total);
    run += total;
    bool any = false;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int j = base + PER * t + e;
      const int gt_before = (int)(acc >> 32);
      const int eq_before = (int)(acc & 0xffffffffu);
      const bool sel = cc[e] == 2 || (cc[e] == 1 && eq_before < need_eq);
      const int pos = gt_before + min(eq_before, need_eq);
      if (j < L) {
        if (slash) P[j] = pos;
        if (sel && list && pos < nlist) list[hb * nlist + pos] = j;
      }
      any |= sel;
      acc += cc[e] == 2 ? (1ull << 32) : (uint64_t)(cc[e] == 1);
    }
    if (!slash) {
      const uint64_t bal = __ballot(any);
      if ((t & 63) == 0) {
        const int tile0 = (base + (t >> 6) * 64 * PER) / TILE;
#pragma unroll
        for (int q = 0; q < PER; ++q)
          if ((tile0 + q) * TILE < L) a.vt[hb * a.nB + tile0 + q] = ((bal >> (16 * q)) & 0xffffull) ? 1 : 0;
      }
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) xv[e] = xn[e];
  }
  if (t == 0) {
    const int taken = take_all ? L : (by_rank ? n : 0);
    if (slash) P[L] = taken;
    if (list)
      for (int r = min(n, L); r < nlist; ++r) list[hb * nlist + r] = -1;  // n above L
  }
}

__global__ __launch_bounds__(256) void vs_cover(VsArgs a) {
  const size_t hb = (size_t)blockIdx.z * a.H + blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int qb = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (qb >= a.nB) return;
  const int L = a.L;
  const int r_lo = qb * TILE;
  const int r_hi = min(L - 1, r_lo + TILE - 1);
  const int32_t* P = a.P + hb * (L + 1);
  const int32_t* vt = a.vt + hb * a.nB;
  int32_t* out = a.block_idx + (hb * a.nB + qb) * a.max_blocks;
  int base = 0;
  for (int c0 = 0; c0 <= qb; c0 += 64) {
    const int c = c0 + lane;
    bool kept = false;
    if (c <= qb) {
      const int j_lo = c * TILE;
      const int j_hi = min(L - 1, j_lo + TILE - 1);
      const int lo = max(0, r_lo - j_hi);
      const int hi = r_hi - j_lo;  // <= L - 1
      kept = vt[c] != 0 || P[hi + 1] - P[lo] > 0;
    }
    const uint64_t bal = __ballot(kept);
    if (kept) out[base + __popcll(bal & ((1ull << lane) - 1ull))] = c;
    base += __popcll(bal);
  }
  for (int r = base + lane; r < a.max_blocks; r += 64) out[r] = -1;
  if (lane == 0) a.block_cnt[hb * a.nB + qb] = base;
}

template <int D>
hipError_t launch(const VsArgs& a, hipStream_t stream) {
  const dim3 g_pass(a.nchunk, a.H, a.B);
  hipLaunchKernelGGL((vs_pass<D, 0>), g_pass, dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vs_rowstats, dim3(a.H, a.B), dim3(1024), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((vs_pass<D, 1>), g_pass, dim3(256), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vs_slash_combine, dim3((a.L + 255) / 256, a.H, a.B), dim3(256), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vs_select, dim3(2, a.H, a.B), dim3(SEL_T), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vs_cover, dim3((a.nB + 3) / 4, a.H, a.B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_vertical_slash(const VsParams& p, hipStream_t stream) {
  VsArgs a = {};
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.B = p.B;
  a.H = p.H;
  a.L = p.L;
  a.R = p.last_q;
  a.nchunk = (p.L + CH - 1) / CH;
  a.nB = (p.L + TILE - 1) / TILE;
  a.n_vert = p.n_vertical;
  a.n_slash = p.n_slash;
  a.max_blocks = p.max_blocks;
  a.c_log2 = 1.4426950408889634f / sqrtf((float)p.d);
  VsWorkspace w(p.B, p.H, p.L);
  char* base = static_cast<char*>(p.workspace);
  a.part = reinterpret_cast<float*>(base + w.part);
  a.stats = reinterpret_cast<float*>(base + w.stats);
  a.v = reinterpret_cast<float*>(base + w.v);
  a.s = reinterpret_cast<float*>(base + w.s);
  a.spart = reinterpret_cast<float*>(base + w.spart);
  a.vt = reinterpret_cast<int32_t*>(base + w.vt);
  a.P = reinterpret_cast<int32_t*>(base + w.P);
  a.block_idx = p.block_idx;
  a.block_cnt = p.block_cnt;
  a.vert_idx = p.vertical_idx;
  a.slash_idx = p.slash_idx;
  a.v_out = p.vertical_scores;
  a.s_out = p.slash_scores;
  if (p.d == 128) return launch<128>(a, stream);
  if (p.d == 64) return launch<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ssa
