// Threshold calibration on the device: the lambda that skips a target share
// of the visited tiles, from the per-tile margins of a statistics launch.
//
// Operation (TRT-LLM "Skip Softmax" page, efficiency and accuracy section:
// an automatic calibration finds the sparsity threshold; Model Optimizer
// tutorial, step 4: search for the threshold that meets a target sparsity).
// A tile's margin does not depend on lambda (a skipped tile never raises
// the running max), so the skip set at lambda is {margin < lambda} and the
// skip ratio is the empirical distribution of the margins. The rule: among
// the sorted non-NaN margins g[0..n), take the consecutive pairs (g[r-1],
// g[r]) with r in [lo, hi] -- the ranks within +-window of the target rank
// -- and put lambda at the midpoint of the widest gap between two finite
// margins (the first such pair on ties), so that as few tiles as possible
// sit near the threshold; without a finite pair, lambda = g[want] if finite,
// else 0; lambda is clamped to <= 0.
//
// Design (no sort):
//  * margins map to order-preserving 32-bit keys (-0 taken as +0); an exact
//    radix select in three histogram passes (11, 11 and 10 key bits,
//    LDS-privatised histograms, one pass over the margins each) finds the
//    values at the window's end ranks, together with the count of margins
//    below each;
//  * the window's finite values [v_a, v_b] are dealt to nb = 2m + 2 buckets
//    of equal width (m pairs in the window). The widest gap is at least
//    (v_b - v_a) / m, more than twice a bucket's width, so it always runs
//    from the largest value of one non-empty bucket to the smallest of the
//    next one (bucket assignment is monotone in the value): one pass records
//    each bucket's min and max key with atomics, and an ordered scan of the
//    buckets finds the first widest gap. Gaps and the midpoint are taken in
//    fp64 from the fp32 margins;
//  * a last pass counts the margins below lambda (the achieved ratio).
// Every pass is a grid-stride sweep of coalesced loads; the scans run in one
// workgroup. The launches carry their state in the workspace, so the whole
// calibration is stream-ordered with no host round trip.
#include "common.h"
#include "launch.h"

namespace ssa {

namespace {

constexpr int kThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kChunk = 16;  // buckets per thread in the gap scan

struct CalState {
  unsigned long long n_valid, n_neginf, n_posinf, n_below;
  long long rank[3];         // target ranks: window start, window end, fallback
  long long less[3];         // margins with a smaller key than the target's value
  unsigned int prefix[3];    // key prefix found so far per target
  unsigned int key[3];       // exact keys after the third pass
  int done;                  // 1: lambda is final (no bucket pass needed)
  int error;                 // 1: the bucket count exceeded the workspace
  long long nb;              // buckets in use
  double v_a, inv_w;
  unsigned int key_a, key_b;
  double lambda;
};

struct GapSummary {
  int has;
  float first_min, last_max;
  float best_a, best_b;
  double best;
};

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

__device__ __forceinline__ unsigned int fkey(float x) {
  unsigned int u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float fkey_inv(unsigned int k) {
  const unsigned int u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__global__ __launch_bounds__(kScanThreads) void cal_init(CalState* st, unsigned int* hist, int nhist) {
  const int t = threadIdx.x;
  for (int i = t; i < nhist; i += kScanThreads) hist[i] = 0u;
  if (t == 0) {
    st->n_valid = st->n_neginf = st->n_posinf = st->n_below = 0ull;
    st->done = 0;
    st->error = 0;
    st->lambda = 0.0;
    for (int j = 0; j < 3; ++j) {
      st->rank[j] = 0;
      st->less[j] = 0;
      st->prefix[j] = 0u;
      st->key[j] = 0u;
    }
  }
}

// PASS 1: histogram of key bits 31..21 (and the valid / infinite counts);
// PASS 2: bits 20..10 of the margins whose top 11 bits match each target's;
// PASS 3: bits 9..0 of those matching the 22-bit prefix.
template <int PASS>
__global__ __launch_bounds__(kThreads) void cal_hist(const float* __restrict__ g, long long n,
                                                     CalState* st, unsigned int* hist) {
  constexpr int NB = PASS == 3 ? 1024 : 2048;
  constexpr int NT = PASS == 1 ? 1 : 3;
  __shared__ unsigned int h[NT * NB];
  __shared__ unsigned long long cnt[3];
  const int t = threadIdx.x;
  for (int i = t; i < NT * NB; i += kThreads) h[i] = 0u;
  if (t < 3) cnt[t] = 0ull;
  if (PASS > 1 && st->done) return;
  unsigned int pre[3] = {0u, 0u, 0u};
  if (PASS > 1)
    for (int j = 0; j < 3; ++j) pre[j] = st->prefix[j];
  sync_lds();
  unsigned long long nv = 0, nni = 0, npi = 0;
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long i = (long long)blockIdx.x * kThreads + t; i < n; i += stride) {
    const float x = g[i];
    if (x != x) continue;
    const unsigned int k = fkey(x);
    if (PASS == 1) {
      atomicAdd(&h[k >> 21], 1u);
      ++nv;
      nni += (x == -INFINITY);
      npi += (x == INFINITY);
    } else if (PASS == 2) {
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if ((k >> 21) == pre[j]) atomicAdd(&h[j * NB + ((k >> 10) & 2047u)], 1u);
    } else {
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if ((k >> 10) == pre[j]) atomicAdd(&h[j * NB + (k & 1023u)], 1u);
    }
  }
  if (PASS == 1) {
    nv = wave_sum_u64(nv);
    nni = wave_sum_u64(nni);
    npi = wave_sum_u64(npi);
    if ((t & 63) == 0) {
      atomicAdd(&cnt[0], nv);
      atomicAdd(&cnt[1], nni);
      atomicAdd(&cnt[2], npi);
    }
  }
  sync_lds();
  for (int i = t; i < NT * NB; i += kThreads)
    if (h[i]) atomicAdd(&hist[i], h[i]);
  if (PASS == 1 && t == 0) {
    if (cnt[0]) atomicAdd(&st->n_valid, cnt[0]);
    if (cnt[1]) atomicAdd(&st->n_neginf, cnt[1]);
    if (cnt[2]) atomicAdd(&st->n_posinf, cnt[2]);
  }
}

// The rule's ranks (thread 0), in the same fp64 arithmetic as the
// definition: want = round-half-even(target * n), lo = max(1, floor((target
// - window) * n)), hi = min(n - 1, ceil((target + window) * n)), widened to
// include want; finite pairs need both ranks inside the finite run.
__device__ void cal_targets(CalState* st, double target, double window) {
  const long long n = (long long)st->n_valid;
  if (n < 2) {
    st->lambda = 0.0;
    st->done = 1;
    return;
  }
  const long long want = (long long)rint(target * (double)n);
  long long lo = (long long)floor((target - window) * (double)n);
  long long hi = (long long)ceil((target + window) * (double)n);
  lo = lo < 1 ? 1 : lo;
  hi = hi > n - 1 ? n - 1 : hi;
  const long long wlo = want < 1 ? 1 : want;
  const long long whi = want > n - 1 ? n - 1 : want;
  lo = lo < wlo ? lo : wlo;
  hi = hi > whi ? hi : whi;
  const long long first_fin = (long long)st->n_neginf;
  const long long last_fin = n - 1 - (long long)st->n_posinf;
  const long long plo = lo > first_fin + 1 ? lo : first_fin + 1;
  const long long phi = hi < last_fin ? hi : last_fin;
  long long wc = want < 0 ? 0 : want;
  wc = wc > n - 1 ? n - 1 : wc;
  if (plo <= phi) {
    st->rank[0] = plo - 1;
    st->rank[1] = phi;
    st->rank[2] = plo - 1;
    st->nb = 2 * (phi - plo + 1) + 2;
  } else if (wc < first_fin || wc > last_fin) {
    st->lambda = 0.0;  // the fallback margin is infinite
    st->done = 1;
  } else {
    st->rank[0] = st->rank[1] = st->rank[2] = wc;
    st->nb = -1;  // fallback: lambda = g[want]
  }
}

// One workgroup: for each target rank find the histogram bin that holds it
// (exclusive prefix sums over the bins, two bins per thread).
template <int PASS>
__global__ __launch_bounds__(kScanThreads) void cal_scan(CalState* st, const unsigned int* hist, double target,
                                                         double window, long long nb_max) {
  constexpr int NB = PASS == 3 ? 1024 : 2048;
  constexpr int SH = PASS == 1 ? 21 : (PASS == 2 ? 11 : 10);
  __shared__ unsigned long long wsum[kScanThreads / 64];
  __shared__ int done;
  const int t = threadIdx.x;
  if (t == 0) {
    if (PASS == 1) cal_targets(st, target, window);
    done = st->done;
  }
  sync_lds();
  if (done) return;
  for (int j = 0; j < 3; ++j) {
    const unsigned int* hj = hist + (PASS == 1 ? 0 : j * NB);
    const long long want = st->rank[j] - st->less[j];
    const int b0 = t * (NB / kScanThreads);
    unsigned long long c[NB / kScanThreads];
    unsigned long long mine = 0;
#pragma unroll
    for (int e = 0; e < NB / kScanThreads; ++e) {
      c[e] = hj[b0 + e];
      mine += c[e];
    }
    // exclusive scan over the workgroup
    unsigned long long incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long y = __shfl_up(incl, o, 64);
      if ((t & 63) >= o) incl += y;
    }
    if ((t & 63) == 63) wsum[t >> 6] = incl;
    sync_lds();
    unsigned long long base = 0;
    for (int w = 0; w < (t >> 6); ++w) base += wsum[w];
    unsigned long long ex = base + incl - mine;
#pragma unroll
    for (int e = 0; e < NB / kScanThreads; ++e) {
      if ((long long)ex <= want && want < (long long)(ex + c[e])) {
        st->prefix[j] = (PASS == 1 ? 0u : (st->prefix[j] << SH)) | (unsigned int)(b0 + e);
        st->less[j] += (long long)ex;
      }
      ex += c[e];
    }
    sync_lds();
  }
  if (PASS == 3 && t == 0) {
    for (int j = 0; j < 3; ++j) st->key[j] = st->prefix[j];
    if (st->nb < 0) {
      const double lam = (double)fkey_inv(st->key[2]);
      st->lambda = lam < 0.0 ? lam : 0.0;
      st->done = 1;
      return;
    }
    const float a = fkey_inv(st->key[0]);
    const float b = fkey_inv(st->key[1]);
    if (a == b) {
      const double lam = 0.5 * ((double)a + (double)b);
      st->lambda = lam < 0.0 ? lam : 0.0;
      st->done = 1;
      return;
    }
    if (st->nb > nb_max) {
      st->error = 1;
      st->done = 1;
      return;
    }
    st->v_a = (double)a;
    st->inv_w = (double)st->nb / ((double)b - (double)a);
    st->key_a = st->key[0];
    st->key_b = st->key[1];
  }
}

__global__ __launch_bounds__(kThreads) void cal_bucket_init(const CalState* st, unsigned int* bmin, unsigned int* bmax,
                                                            long long nb_max) {
  if (st->done) return;
  const long long nb = st->nb < nb_max ? st->nb : nb_max;
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < nb; i += stride) {
    bmin[i] = 0xFFFFFFFFu;
    bmax[i] = 0u;
  }
}

__global__ __launch_bounds__(kThreads) void cal_bucket(const float* __restrict__ g, long long n, const CalState* st,
                                                       unsigned int* bmin, unsigned int* bmax) {
  if (st->done) return;
  const unsigned int ka = st->key_a, kb = st->key_b;
  const double va = st->v_a, iw = st->inv_w;
  const long long nb = st->nb;
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    const float x = g[i];
    if (x != x) continue;
    const unsigned int k = fkey(x);
    if (k < ka || k > kb) continue;
    long long bk = (long long)floor(((double)x - va) * iw);
    bk = bk < 0 ? 0 : (bk > nb - 1 ? nb - 1 : bk);
    atomicMin(&bmin[bk], k);
    atomicMax(&bmax[bk], k);
  }
}

__device__ __forceinline__ void gap_merge(GapSummary& L, const GapSummary& R) {
  if (!R.has) return;
  if (!L.has) {
    L = R;
    return;
  }
  const double mid = (double)R.first_min - (double)L.last_max;
  if (mid > L.best) {
    L.best = mid;
    L.best_a = L.last_max;
    L.best_b = R.first_min;
  }
  if (R.best > L.best) {
    L.best = R.best;
    L.best_a = R.best_a;
    L.best_b = R.best_b;
  }
  L.last_max = R.last_max;
}

// Per chunk of kChunk buckets: first min, last max and the first widest gap
// between consecutive non-empty buckets inside the chunk.
__global__ __launch_bounds__(kThreads) void cal_gap_chunks(const CalState* st, const unsigned int* bmin,
                                                           const unsigned int* bmax, GapSummary* sum) {
  if (st->done) return;
  const long long nb = st->nb;
  const long long nchunk = (nb + kChunk - 1) / kChunk;
  const long long c = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (c >= nchunk) return;
  GapSummary s;
  s.has = 0;
  s.best = -1.0;
  s.first_min = s.last_max = s.best_a = s.best_b = 0.f;
  const long long b1 = (c + 1) * kChunk < nb ? (c + 1) * kChunk : nb;
  for (long long b = c * kChunk; b < b1; ++b) {
    const unsigned int hi = bmax[b];
    if (hi == 0u) continue;
    GapSummary r;
    r.has = 1;
    r.first_min = fkey_inv(bmin[b]);
    r.last_max = fkey_inv(hi);
    r.best = -1.0;
    r.best_a = r.best_b = 0.f;
    gap_merge(s, r);
  }
  sum[c] = s;
}

// One workgroup: merge the chunk summaries in order; lambda = midpoint of
// the first widest gap, clamped to <= 0.
__global__ __launch_bounds__(kScanThreads) void cal_gap_final(CalState* st, const GapSummary* sum) {
  __shared__ GapSummary part[kScanThreads];
  if (st->done) return;
  const long long nchunk = (st->nb + kChunk - 1) / kChunk;
  const int t = threadIdx.x;
  const long long per = (nchunk + kScanThreads - 1) / kScanThreads;
  GapSummary s;
  s.has = 0;
  s.best = -1.0;
  s.first_min = s.last_max = s.best_a = s.best_b = 0.f;
  for (long long c = t * per; c < (t + 1) * per && c < nchunk; ++c) gap_merge(s, sum[c]);
  part[t] = s;
  // ordered tree merge: part[t] absorbs part[t + h] (the merge is
  // associative and keeps the first of equal gaps)
  for (int h = 1; h < kScanThreads; h <<= 1) {
    sync_lds();
    if ((t & (2 * h - 1)) == 0) {
      GapSummary a = part[t];
      gap_merge(a, part[t + h]);
      part[t] = a;
    }
  }
  if (t == 0) {
    const GapSummary a = part[0];
    const double lam = 0.5 * ((double)a.best_a + (double)a.best_b);
    st->lambda = lam < 0.0 ? lam : 0.0;
    st->done = 1;
  }
}

__global__ __launch_bounds__(kThreads) void cal_count(const float* __restrict__ g, long long n, CalState* st) {
  const double lam = st->lambda;
  unsigned long long below = 0;
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
    below += ((double)g[i] < lam);
  below = wave_sum_u64(below);
  if ((threadIdx.x & 63) == 0 && below) atomicAdd(&st->n_below, below);
}

__global__ void cal_finish(const CalState* st, double* result) {
  if (threadIdx.x != 0) return;
  const double nv = (double)st->n_valid;
  result[0] = st->error ? __longlong_as_double(0x7FF8000000000000ll) : st->lambda;
  result[1] = st->n_valid ? (double)st->n_below / nv : 0.0;
  result[2] = nv;
  result[3] = (double)st->n_below;
}

}  // namespace

CalWorkspace::CalWorkspace(long long n, double window) {
  // pairs in the rank window: at most ceil(2 window n) + 3; a margin of a
  // few pairs covers fp64 rounding of the rank bounds
  const long long m = (long long)ceil(2.0 * window * (double)n) + 8;
  nb_max = 2 * m + 2;
  const long long nchunk = (nb_max + kChunk - 1) / kChunk;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  state = take(sizeof(CalState));
  hist = take((size_t)(2048 + 3 * 2048 + 3 * 1024) * sizeof(unsigned int));
  bmin = take((size_t)nb_max * sizeof(unsigned int));
  bmax = take((size_t)nb_max * sizeof(unsigned int));
  sums = take((size_t)nchunk * sizeof(GapSummary));
  total = off;
}

hipError_t launch_lambda_for_ratio(const float* margins, long long n, double target, double window,
                                   double* result, void* workspace, hipStream_t stream) {
  const CalWorkspace ws(n, window);
  char* base = static_cast<char*>(workspace);
  CalState* st = reinterpret_cast<CalState*>(base + ws.state);
  unsigned int* h1 = reinterpret_cast<unsigned int*>(base + ws.hist);
  unsigned int* h2 = h1 + 2048;
  unsigned int* h3 = h2 + 3 * 2048;
  unsigned int* bmin = reinterpret_cast<unsigned int*>(base + ws.bmin);
  unsigned int* bmax = reinterpret_cast<unsigned int*>(base + ws.bmax);
  GapSummary* sums = reinterpret_cast<GapSummary*>(base + ws.sums);
  long long gb = (n + kThreads * 8 - 1) / (kThreads * 8);
  const unsigned int grid = (unsigned int)(gb < 1 ? 1 : (gb > 4096 ? 4096 : gb));
  hipLaunchKernelGGL(cal_init, dim3(1), dim3(kScanThreads), 0, stream, st, h1, 2048 + 3 * 2048 + 3 * 1024);
  hipLaunchKernelGGL(cal_hist<1>, dim3(grid), dim3(kThreads), 0, stream, margins, n, st, h1);
  hipLaunchKernelGGL(cal_scan<1>, dim3(1), dim3(kScanThreads), 0, stream, st, h1, target, window, ws.nb_max);
  hipLaunchKernelGGL(cal_hist<2>, dim3(grid), dim3(kThreads), 0, stream, margins, n, st, h2);
  hipLaunchKernelGGL(cal_scan<2>, dim3(1), dim3(kScanThreads), 0, stream, st, h2, target, window, ws.nb_max);
  hipLaunchKernelGGL(cal_hist<3>, dim3(grid), dim3(kThreads), 0, stream, margins, n, st, h3);
  hipLaunchKernelGGL(cal_scan<3>, dim3(1), dim3(kScanThreads), 0, stream, st, h3, target, window, ws.nb_max);
  long long bb = (ws.nb_max + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(cal_bucket_init, dim3((unsigned int)(bb > 4096 ? 4096 : bb)), dim3(kThreads), 0, stream, st,
                     bmin, bmax, ws.nb_max);
  hipLaunchKernelGGL(cal_bucket, dim3(grid), dim3(kThreads), 0, stream, margins, n, st, bmin, bmax);
  const long long nchunk = (ws.nb_max + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(cal_gap_chunks, dim3((unsigned int)((nchunk + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     stream, st, bmin, bmax, sums);
  hipLaunchKernelGGL(cal_gap_final, dim3(1), dim3(kScanThreads), 0, stream, st, sums);
  hipLaunchKernelGGL(cal_count, dim3(grid), dim3(kThreads), 0, stream, margins, n, st);
  hipLaunchKernelGGL(cal_finish, dim3(1), dim3(64), 0, stream, st, result);
  return hipGetLastError();
}

}  // namespace ssa
