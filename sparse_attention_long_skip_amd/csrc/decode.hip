// Skip-Softmax split-K decode and log-sum-exp combine for gfx950.
//
// Operation (TRT-LLM "Skip Softmax" page: decode is bound by reading the KV
// cache, and a skipped tile's V block is never loaded): one new query token
// per sequence; the G query heads sharing a KV head are the rows of every
// tile decision; the cache is cut into splits of T key tiles, each with its
// own running max; partial (m, l, o) per split are merged with the
// log-sum-exp identity.
//
// Design: each split (sequence, KV head, split) is run by one wave, so the
// vote and the softmax never need a workgroup barrier. The split kernel is
// persistent: one wave per resident wave slot takes splits from a work
// counter in split-major order (every first split, then every second one,
// ...: the short last splits come at the end) and, during the last tile of
// a split, already loads the query rows and first K tile of its next one.
// A wave slot thus never waits for a new wave to be dispatched and for its
// first loads to arrive, which with one wave per split cost about a fifth
// of the slot time. Scores use 16x16x32 bf16 MFMA (S^T = K Q^T, K rows read
// straight from HBM as the A operand, the G query rows as B-operand
// columns). The K tile for step j+1 is prefetched into registers while step
// j runs; the V tile is issued only after the vote, and its P.V waits until
// the scores and vote of the next tile are done. P.V runs on the vector
// units: V rows are read with coalesced 16-byte loads (each row is 16 lanes
// x 16 B at d = 128) and the probabilities come from a small per-wave LDS
// table.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "common.h"
#include "launch.h"

namespace ssa {

namespace {

constexpr int BC = 64;

// Buffer resource from wave-uniform values that the compiler cannot prove
// uniform (they pass through the work-item loop): read from the first lane,
// so the resource is built in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void* base, int nbytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo),
                   __builtin_amdgcn_readfirstlane(nbytes));
}

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
  uint32_t* queue;  // work counter, set by decode_queue_reset before each split launch
  int B, Hq, Hkv, S_max, T, nS, nT;
  float lam_raw;
  float c_log2;
  float inv_sqrt_d;
};

// One wave per SIMD: the cache streams are read faster with fewer of them
// in flight (on the 32-sequence, 16K-32K workload: 0.453 ms with one wave
// per SIMD, 0.478 ms with two), and each wave may then use the whole
// register file.
template <int D, int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1)))
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

  // Work items: every (sequence, KV head, split), in that order, taken from
  // the work counter. Consecutive tickets are consecutive splits of one
  // cache, so the waves in flight at any time stream a compact window of
  // the caches. A split at or past the end of its sequence holds no keys:
  // the wave that draws one zeroes the skip counts of the cache's remaining
  // splits and moves the counter on to the next cache.
  // The lengths are read through the constant address space: a scalar load,
  // wave-uniform, outside the vector load queue (the kernel never writes
  // them).
  const __attribute__((address_space(4))) int32_t* seqlens_c =
      (const __attribute__((address_space(4))) int32_t*)a.seqlens;
  const int total = a.B * a.Hkv * a.nS;
  struct Item {
    int b, kvh, sp, n, j0, j1;
  };
  uint32_t ticket = 0;  // lane 0: the ticket taken last
  auto take = [&]() { if (lane == 0) ticket = atomicAdd(a.queue, 1u); };
  // The first item with a key at or after ticket k (sp = -1: none left).
  auto next_item = [&](int k) -> Item {
    Item it;
    it.sp = -1;
    while (k < total) {
      const int bh = k / a.nS;
      const int sp = k - bh * a.nS;
      const int bb = bh / a.Hkv;
      const int n = min(max(seqlens_c[bb], 0), a.S_max);
      const int ntiles = (n + BC - 1) / BC;
      if (sp * a.T < ntiles) {
        it.b = bb;
        it.kvh = bh - bb * a.Hkv;
        it.sp = sp;
        it.n = n;
        it.j0 = sp * a.T;
        it.j1 = min(ntiles, it.j0 + a.T);
        break;
      }
      // Splits sp .. nS-1 of this cache hold no keys (any wave that draws
      // one of them writes the same zeros). Ticket `next` (the next cache's
      // first split) is this wave's if the counter had not passed it;
      // otherwise a fresh ticket is taken.
      if (a.skip_counts)
        for (int s2 = sp + lane; s2 < a.nS; s2 += kWave) a.skip_counts[(size_t)bh * a.nS + s2] = 0;
      const uint32_t next = (uint32_t)(bh + 1) * (uint32_t)a.nS;
      if (lane == 0) ticket = atomicMax(a.queue, next + 1u);
      if ((uint32_t)__builtin_amdgcn_readfirstlane(ticket) <= next) {
        k = (int)next;
      } else {
        take();
        k = (int)__builtin_amdgcn_readfirstlane(ticket);
      }
    }
    return it;
  };
  // Wave w starts with item w; the counter starts at the number of waves.
  Item cur = next_item((int)blockIdx.x);
  if (cur.sp < 0) return;

  auto kv_base = [&](const Item& it) -> size_t { return ((size_t)it.b * a.Hkv + it.kvh) * a.S_max * D; };

  // S^T = K Q^T with 16x16x32 products: K rows (16 keys per block) are the
  // A operand, the G query rows the B-operand columns (columns >= G zero).
  // A lane then holds 4 consecutive keys of each 16-key block for one query
  // row, and each K load covers 16 rows x 64 contiguous bytes.
  // All loads go through buffer resources that end at the last valid row:
  // query rows past G and keys past the sequence read as zeros, with
  // 32-bit per-lane offsets and no per-lane masks. Lane offset of row c16,
  // chunk q4 (the K rows of a 16-key block use the same one).
  const uint32_t row_off = (uint32_t)(c16 * D + q4 * 8) * 2u;
  bf16x8 qf[NDS];
  auto load_q = [&](const Item& it) {
    const auto rs = wave_rsrc(a.q + ((size_t)it.b * a.Hq + it.kvh * G) * D, G * D * 2);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qf[ds] = as_bf16x8(load16_buf(rs, row_off + ds * 64));
  };

  u32x4 kreg[4][NDS];
  auto load_k = [&](const uint16_t* kptr, int nn, int j) {
    const int k0 = j * BC;
    const auto rs = wave_rsrc(kptr + (size_t)k0 * D, max(0, min(nn - k0, BC)) * D * 2);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) kreg[kb][ds] = load16_buf(rs, row_off + kb * 16 * D * 2 + ds * 64);
  };

  const int rg = lane / CPR;
  const int cc = lane % CPR;
  // V rows rg * KPG + m, chunk cc of a tile
  const uint32_t v_off = (uint32_t)(rg * KPG * D + cc * 8) * 2u;
  float o[G][8];
  u32x4 vreg[KPG];
  int pb = 0;

  load_q(cur);
  load_k(a.kc + kv_base(cur), cur.n, cur.j0);
  for (;;) {
    const int b = cur.b;
    const int kvh = cur.kvh;
    const int sp = cur.sp;
    const int n = cur.n;
    const int j0 = cur.j0;
    const int j1 = cur.j1;
    const uint16_t* kp = a.kc + kv_base(cur);
    const uint16_t* vp = a.vc + kv_base(cur);
    const int hq0 = kvh * G;
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
    bool pend = false;  // a kept tile awaits its P.V (V in vreg, P and alpha in LDS buffer pb)
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

    // During the last tile, after its scores, the next ticket is taken and
    // the next item's query rows and first K tile are loaded into the
    // registers this item no longer needs.
    Item nxt;
    nxt.sp = -1;
    for (int j = j0; j < j1; ++j) {
      f32x4 s[4];  // keys kb * 16 + 4 q4 + i of query row c16
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) s[kb] = mfma16(as_bf16x8(kreg[kb][ds]), qf[ds], s[kb]);
      }
      if (j + 1 < j1) {
        load_k(kp, n, j + 1);
      } else {
        take();
        nxt = next_item((int)__builtin_amdgcn_readfirstlane(ticket));
        if (nxt.sp >= 0) {
          load_q(nxt);
          load_k(a.kc + kv_base(nxt), nxt.n, nxt.j0);
        }
      }
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
      const auto rsv = wave_rsrc(vp + (size_t)kbase * D, max(0, min(n - kbase, BC)) * D * 2);
#pragma unroll
      for (int m = 0; m < KPG; ++m) vreg[m] = load16_buf(rsv, v_off + m * D * 2);
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
    if (a.skip_counts && lane == 0) a.skip_counts[((size_t)b * a.Hkv + kvh) * a.nS + sp] = skipped;
    if (__builtin_amdgcn_readfirstlane(nxt.sp) < 0) break;
    cur.b = __builtin_amdgcn_readfirstlane(nxt.b);
    cur.kvh = __builtin_amdgcn_readfirstlane(nxt.kvh);
    cur.sp = __builtin_amdgcn_readfirstlane(nxt.sp);
    cur.n = __builtin_amdgcn_readfirstlane(nxt.n);
    cur.j0 = __builtin_amdgcn_readfirstlane(nxt.j0);
    cur.j1 = __builtin_amdgcn_readfirstlane(nxt.j1);
  }
}

// One wave per (query head, sequence) merges the split partials, 64 splits
// per batch: lane s holds split s's log-sum-exp lse_s = m_s / sqrt(d) +
// ln l_s (splits with l_s = 0 hold no kept key and are left out); with
// top = max lse_s, tot = sum exp(lse_s - top) and out = sum exp(m_s /
// sqrt(d) - top) o_s / tot, lse = top + ln tot. A lane owns D / 64 output
// elements; a batch's partial loads are all issued before the first use,
// and each split's weight reaches every lane by a scalar read.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  constexpr int E = D / kWave;  // output elements per lane
  constexpr int U = 32;         // partial rows in flight per lane
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int n = min(max(a.seqlens[b], 0), a.S_max);
  const int ntiles = (n + BC - 1) / BC;
  const int nsp = (ntiles + a.T - 1) / a.T;
  const size_t base = ((size_t)b * a.Hq + hq) * a.nS;
  float top = -INFINITY, tot = 0.f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < nsp; s0 += kWave) {
    const int s = s0 + lane;
    float x = -INFINITY, ms = -INFINITY;
    if (s < nsp) {
      const float m = a.ws_ml[(base + s) * 2];
      const float l = a.ws_ml[(base + s) * 2 + 1];
      if (l > 0.f) {
        ms = m * a.inv_sqrt_d;
        x = ms + __logf(l);
      }
    }
    const float bt = wave_max(x);
    if (bt > top) {
      // rescale what the earlier batches summed (nothing if top = -inf)
      const float sc = __expf(top - bt);
      tot *= sc;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] *= sc;
      top = bt;
    }
    if (top == -INFINITY) continue;  // no kept key so far
    tot += wave_sum(x == -INFINITY ? 0.f : __expf(x - top));
    const float wo = ms == -INFINITY ? 0.f : __expf(ms - top);
    const int cnt = min(kWave, nsp - s0);
    for (int u0 = 0; u0 < cnt; u0 += U) {
      float oo[U][E];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < E; ++e)
          oo[u][e] = u0 + u < cnt ? a.ws_o[(base + s0 + u0 + u) * D + e * kWave + lane] : 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float w = __builtin_amdgcn_readlane(__float_as_int(wo), (u0 + u) & (kWave - 1));
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(__int_as_float(w), oo[u][e], acc[e]);
      }
    }
  }
  const float lse = (tot > 0.f) ? top + __logf(tot) : -INFINITY;
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const __bf16 rb = (__bf16)(acc[e] * inv);
    a.out[((size_t)b * a.Hq + hq) * D + e * kWave + lane] = __builtin_bit_cast(uint16_t, rb);
  }
  if (a.lse && lane == 0) a.lse[(size_t)b * a.Hq + hq] = lse;
}

// The split kernel's work counter is set before every launch (a kernel, not
// a memset, so that the launch sequence can be captured in a graph): wave w
// starts with item w, so the first ticket handed out is the wave count.
__global__ void decode_queue_reset(uint32_t* queue, uint32_t first) {
  if (threadIdx.x == 0) *queue = first;
}

// Waves of the persistent split kernel on the current device: one per SIMD
// (four per CU), the CU count looked up once per device.
int split_waves() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDev) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const int r = 4 * cus;
  if (r > 0 && dev < kMaxDev) cache[dev].store(r, std::memory_order_relaxed);
  return r;
}

template <int D, int G>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  const int slots = split_waves();
  if (slots <= 0) return hipErrorInvalidDevice;
  const long long items_max = (long long)a.B * a.Hkv * a.nS;
  const int waves = (int)std::min<long long>(slots, items_max);
  hipLaunchKernelGGL(decode_queue_reset, dim3(1), dim3(64), 0, stream, a.queue, (uint32_t)waves);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_split_kernel<D, G>), dim3(waves), dim3(64), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(a.Hq, a.B);
  hipLaunchKernelGGL((decode_combine_kernel<D>), g2, dim3(kWave), 0, stream, a);
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
  a.queue = reinterpret_cast<uint32_t*>(a.ws_ml + (size_t)p.B * p.Hq * a.nS * 2);
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
