// Skip-Softmax split-K decode and log-sum-exp combine for gfx950.
//
// Operation (TRT-LLM "Skip Softmax" page: decode is bound by reading the KV
// cache, and a skipped tile's V block is never loaded): one new query token
// per sequence; the G query heads sharing a KV head are the rows of every
// tile decision; the cache is cut into splits of T key tiles, each with its
// own running max; partial (m, l, o) per split are merged with the
// log-sum-exp identity.
//
// Design: one wave per (sequence, KV head, split), so the vote and the
// softmax never need a workgroup barrier. Scores use 16x16x32 bf16 MFMA
// (S^T = K Q^T, K rows read straight from HBM as the A operand, the G query
// rows as B-operand columns). The K tile for step j+1 is prefetched into
// registers while step j runs; the V tile is issued only after the vote,
// and its P.V waits until the scores and vote of the next tile are done.
// P.V runs on the vector units: V rows are read with coalesced 16-byte loads
// (each row is 16 lanes x 16 B at d = 128) and the probabilities come from a
// small per-wave LDS table. Splits are dispatched split-major (every first
// split, then every second one, ...), so the short last splits run last.
#include <mutex>

#include "common.h"
#include "launch.h"

namespace ssa {

namespace {

constexpr int BC = 64;

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* seqlens;
  uint16_t* out;
  float* lse;
  int32_t* skip_counts;
  uint8_t* tile_state;
  float* tile_margin;
  float* ws_o;   // [B, Hq, nS, D]
  float* ws_ml;  // [B, Hq, nS, 2]
  int B, Hq, Hkv, S_max, T, nS, nT;
  float lam_raw;
  float c_log2;
  float inv_sqrt_d;
};

// Two waves per SIMD where the registers allow it without spilling (the
// K prefetch and V rows of one wave are already many bytes in flight; a
// second wave hides one wave's vector P.V behind the other's loads).
template <int D, int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu((D == 128 ? G <= 4 : G <= 8) ? 2 : 1)))
void decode_split_kernel(DecodeArgs a) {
  constexpr int NDS = D / 32;    // 32-wide reduction steps of the 16x16x32 products
  constexpr int CPR = D / 8;     // 16-byte chunks per V row
  constexpr int RG = 64 / CPR;   // row groups across the wave
  constexpr int KPG = BC / RG;   // keys per row group and tile

  // P and the rescale factor of a kept tile, double-buffered: the next kept
  // tile's are written while the pending tile's P.V still reads them.
  __shared__ __attribute__((aligned(16))) float p_lds[2][G][BC];
  __shared__ float alpha_lds[2][G];

  const int lane = threadIdx.x;
  const int c16 = lane & 15;  // score column = query row g
  const int q4 = lane >> 4;   // lane group: keys 4 q4 .. 4 q4 + 3 of each 16-key block
  // Split-major order: all first splits are dispatched before any second
  // split, so the short last splits of the sequences come at the end.
  const int kvh = blockIdx.x;
  const int b = blockIdx.y;
  const int sp = blockIdx.z;

  const int n = min(max(a.seqlens[b], 0), a.S_max);
  const int ntiles = (n + BC - 1) / BC;
  const int nsp = (ntiles + a.T - 1) / a.T;
  const size_t unit_s = ((size_t)b * a.Hkv + kvh) * a.nS + sp;
  if (sp >= nsp) {
    if (a.skip_counts && lane == 0) a.skip_counts[unit_s] = 0;
    return;
  }
  const int j0 = sp * a.T;
  const int j1 = min(ntiles, j0 + a.T);

  const uint16_t* kp = a.kc + ((size_t)b * a.Hkv + kvh) * a.S_max * D;
  const uint16_t* vp = a.vc + ((size_t)b * a.Hkv + kvh) * a.S_max * D;
  const int hq0 = kvh * G;

  // S^T = K Q^T with 16x16x32 products: K rows (16 keys per block) are the
  // A operand, the G query rows the B-operand columns (columns >= G zero).
  // A lane then holds 4 consecutive keys of each 16-key block for one query
  // row, and each K load covers 16 rows x 64 contiguous bytes.
  bf16x8 qf[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (c16 < G) x = load16(a.q + ((size_t)b * a.Hq + hq0 + c16) * D + ds * 32 + q4 * 8);
    qf[ds] = as_bf16x8(x);
  }

  u32x4 kreg[4][NDS];
  auto load_k = [&](int j) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = j * BC + kb * 16 + c16;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key < n) x = load16(kp + (size_t)key * D + ds * 32 + q4 * 8);
        kreg[kb][ds] = x;
      }
    }
  };

  const int rg = lane / CPR;
  const int cc = lane % CPR;
  float o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
  float m_prev = -INFINITY;
  float l_acc = 0.f;
  int skipped = 0;

  // The V rows of a kept tile are loaded right after its vote, and its P.V
  // runs one step later, after the scores and the vote of the next tile:
  // the V load has the next tile's matrix work to land behind.
  u32x4 vreg[KPG];
  bool pend = false;  // a kept tile awaits its P.V (V in vreg, P and alpha in LDS buffer pb)
  int pb = 0;
  auto pv_pending = [&]() __attribute__((always_inline)) {
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float al = alpha_lds[pb][g];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] *= al;
    }
#pragma unroll
    for (int m4 = 0; m4 < KPG; m4 += 4) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const f32x4 pg = *reinterpret_cast<const f32x4*>(&p_lds[pb][g][rg * KPG + m4]);
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          const u32x4 vv = vreg[m4 + mm];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            o[g][2 * e2] = fmaf(pg[mm], bf16_lo(vv[e2]), o[g][2 * e2]);
            o[g][2 * e2 + 1] = fmaf(pg[mm], bf16_hi(vv[e2]), o[g][2 * e2 + 1]);
          }
        }
      }
    }
    __syncthreads();
  };

  load_k(j0);
  for (int j = j0; j < j1; ++j) {
    f32x4 s[4];  // keys kb * 16 + 4 q4 + i of query row c16
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) s[kb] = mfma16(as_bf16x8(kreg[kb][ds]), qf[ds], s[kb]);
    }
    if (j + 1 < j1) load_k(j + 1);
    const int kbase = j * BC;
    if (kbase + BC > n) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (kbase + kb * 16 + q4 * 4 + e >= n) s[kb][e] = -INFINITY;
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) mloc = fmaxf(mloc, s[kb][e]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    float gap;
    if (c16 >= G || mloc == -INFINITY) gap = -INFINITY;
    else if (m_prev == -INFINITY) gap = INFINITY;
    else gap = mloc - m_prev;
    const float gw = wave_max(gap);
    const bool skip = gw < a.lam_raw;
    if (lane == 0) {
      const size_t ti = ((size_t)b * a.Hkv + kvh) * a.nT + j;
      if (a.tile_state) a.tile_state[ti] = skip ? 2 : 1;
      if (a.tile_margin) a.tile_margin[ti] = gw * a.inv_sqrt_d;
    }
    if (skip) {
      ++skipped;
      m_prev = fmaxf(m_prev, mloc);
      continue;
    }
    // Exponentials of this tile into the other P buffer (the scores are then
    // dead), the P.V of the pending tile, then this tile's V rows -- keys
    // kbase + rg*KPG + m, d chunk cc -- into the registers it freed.
    const int nb = pb ^ (pend ? 1 : 0);
    const float m_new = fmaxf(m_prev, mloc);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2((m_prev - m_use) * a.c_log2);
    const float mc = m_use * a.c_log2;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 pv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pv[e] = fast_exp2(fmaf(s[kb][e], a.c_log2, -mc));
        psum += pv[e];
      }
      if (c16 < G) *reinterpret_cast<f32x4*>(&p_lds[nb][c16][kb * 16 + q4 * 4]) = pv;
    }
    l_acc = l_acc * alpha + psum;
    m_prev = m_new;
    if (lane < G) alpha_lds[nb][lane] = alpha;
    if (pend) pv_pending();
    pb = nb;
#pragma unroll
    for (int m = 0; m < KPG; ++m) {
      const int key = kbase + rg * KPG + m;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < n) x = load16(vp + (size_t)key * D + cc * 8);
      vreg[m] = x;
    }
    pend = true;
  }
  if (pend) pv_pending();

  // Reduce o over the row groups (lanes with equal chunk index).
#pragma unroll
  for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] += __shfl_xor(o[g][e], off, kWave);
  float l_tot = l_acc + __shfl_xor(l_acc, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);
  const size_t base = ((size_t)b * a.Hq + hq0) * a.nS + sp;
  if (rg == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float* dst = a.ws_o + (base + (size_t)g * a.nS) * D + cc * 8;
      f32x4 x0 = {o[g][0], o[g][1], o[g][2], o[g][3]};
      f32x4 x1 = {o[g][4], o[g][5], o[g][6], o[g][7]};
      *reinterpret_cast<f32x4*>(dst) = x0;
      *reinterpret_cast<f32x4*>(dst + 4) = x1;
    }
  }
  if (lane < G) {
    float* ml = a.ws_ml + (base + (size_t)lane * a.nS) * 2;
    ml[0] = m_prev;
    ml[1] = l_tot;
  }
  if (a.skip_counts && lane == 0) a.skip_counts[unit_s] = skipped;
}

// One workgroup per (query head, sequence) merges the split partials in one
// pass: thread t (< D) keeps the log-sum-exp of the splits seen so far and
// the output element t weighted against it, rescaling both when a split
// raises the maximum; the partials are read 16 splits per batch of loads
// (every load issued before the first use).
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  constexpr int U = 16;
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int n = min(max(a.seqlens[b], 0), a.S_max);
  const int ntiles = (n + BC - 1) / BC;
  const int nsp = (ntiles + a.T - 1) / a.T;
  const size_t base = ((size_t)b * a.Hq + hq) * a.nS;
  // lse_s = m_s / sqrt(d) + ln l_s over the splits with l_s > 0;
  // top = max lse_s, tot = sum exp(lse_s - top),
  // acc = sum exp(m_s / sqrt(d) - top) o_s[t].
  float top = -INFINITY, tot = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < nsp; s0 += U) {
    float mm[U], ll[U], oo[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = s0 + u < nsp;
      mm[u] = ok ? a.ws_ml[(base + s0 + u) * 2] : 0.f;
      ll[u] = ok ? a.ws_ml[(base + s0 + u) * 2 + 1] : 0.f;
      oo[u] = ok ? a.ws_o[(base + s0 + u) * D + t] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ll[u] > 0.f) {
        const float ms = mm[u] * a.inv_sqrt_d;
        const float x = ms + __logf(ll[u]);
        if (x > top) {
          const float sc = __expf(top - x);
          tot = tot * sc + 1.f;
          acc = acc * sc + __expf(ms - x) * oo[u];
          top = x;
        } else {
          tot += __expf(x - top);
          acc += __expf(ms - top) * oo[u];
        }
      }
    }
  }
  const float lse = (tot > 0.f) ? top + __logf(tot) : -INFINITY;
  const float r = tot > 0.f ? acc / tot : 0.f;
  const __bf16 rb = (__bf16)r;
  a.out[((size_t)b * a.Hq + hq) * D + t] = __builtin_bit_cast(uint16_t, rb);
  if (a.lse && t == 0) a.lse[(size_t)b * a.Hq + hq] = lse;
}

template <int D, int G>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  dim3 g1(a.Hkv, a.B, a.nS);
  hipLaunchKernelGGL((decode_split_kernel<D, G>), g1, dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(a.Hq, a.B);
  hipLaunchKernelGGL((decode_combine_kernel<D>), g2, dim3(D), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_g(const DecodeArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch<D, 1>(a, stream);
    case 2: return launch<D, 2>(a, stream);
    case 4: return launch<D, 4>(a, stream);
    case 8: return launch<D, 8>(a, stream);
    case 16: return launch<D, 16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Scratch of the allocation-free decode entry point: the split partials
// live in this file-scope device array instead of a caller workspace. Every
// GPU the library runs on holds its own copy for the life of the process;
// all such calls on one GPU share it (calls that overlap on a GPU race).
__device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_addr[dev] == nullptr) {
    // The array's name is a host-side stand-in; its device address on the
    // current device comes from the runtime, once per device.
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_addr[dev] = addr;
  }
  *ptr = scratch_addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  DecodeArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.kc = static_cast<const uint16_t*>(p.k_cache);
  a.vc = static_cast<const uint16_t*>(p.v_cache);
  a.seqlens = p.seqlens;
  a.out = static_cast<uint16_t*>(p.out);
  a.lse = p.lse;
  a.skip_counts = p.skip_counts;
  a.tile_state = p.tile_state;
  a.tile_margin = p.tile_margin;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.S_max = p.S_max;
  a.T = p.split_tiles;
  a.nT = (p.S_max + BC - 1) / BC;
  a.nS = (int)decode_num_splits(p.S_max, p.Bc, p.split_tiles);
  a.ws_o = static_cast<float*>(p.workspace);
  a.ws_ml = a.ws_o + (size_t)p.B * p.Hq * a.nS * p.d;
  const float sd = sqrtf((float)p.d);
  a.lam_raw = p.lambda * sd;
  a.c_log2 = kLog2e / sd;
  a.inv_sqrt_d = 1.f / sd;
  const int G = p.Hq / p.Hkv;
  if (p.d == 128) return launch_g<128>(a, G, stream);
  if (p.d == 64) return launch_g<64>(a, G, stream);
  return hipErrorInvalidValue;
}

}  // namespace ssa
