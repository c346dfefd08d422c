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
// persistent: three waves per CU take splits from a work counter in
// (sequence, KV head, split) order and, during the last tile of a split,
// already loads the query rows and first K tile of its next one. A wave
// slot thus never waits for a new wave to be dispatched and for its first
// loads to arrive, which with one wave per split cost about a fifth of the
// slot time. Scores use 16x16x32 bf16 MFMA (S^T = K Q^T, K rows read
// straight from HBM as the A operand, the G query rows as B-operand
// columns). The K tile for step j+1 is prefetched into registers while step
// j runs; the V tile is issued only after the vote, and its P.V waits until
// the scores and vote of the next tile are done. P.V also runs on 16x16x32
// MFMA (O^T = V^T P^T): V rows arrive with coalesced 16-byte loads (each row
// is 16 lanes x 16 B at d = 128), pass through a swizzled LDS tile and come
// back through transposing reads as the A operand, while each lane's own
// exponentials are its B operand.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

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

// At most one wave per SIMD: the cache streams are read faster with fewer
// of them in flight (on the 32-sequence, 16K-32K workload with vector P.V:
// 0.453 ms with one wave per SIMD, 0.478 ms with two), and each wave may
// then use the whole register file.
template <int D, int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_split_kernel(DecodeArgs a) {
  constexpr int NDS = D / 32;    // 32-wide reduction steps of the 16x16x32 products
  constexpr int CPR = D / 8;     // 16-byte chunks per V row
  constexpr int RG = 64 / CPR;   // row groups across the wave
  constexpr int KPG = BC / RG;   // keys per row group and tile

  constexpr int NDB = D / 16;    // 16-row blocks of O^T (d) in the P.V products
  // The V tile of the pending P.V, row-major with 16-byte chunks XOR-swizzled
  // by row (chunk c of row r at c ^ (r % CPR)), read back transposed.
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[BC * D];

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
  // V rows rg * KPG + m, chunk cc of a tile (KPG = CPR, so row % CPR = m)
  const uint32_t v_off = (uint32_t)(rg * KPG * D + cc * 8) * 2u;
  const int vw_base = rg * KPG * D;
  // O^T += V^T P^T on 16x16x32 products: rows d (16 per block), columns the
  // query rows g, reduction over the tile's keys, 32 per product. Reduction
  // slot 8 q + t of k-step ks is key 32 ks + 16 (t / 4) + 4 q + t % 4: for
  // the B operand (P^T) these are exactly the keys a lane's own scores hold
  // (s[2 ks][t], s[2 ks + 1][t - 4]), and for the A operand (V^T) two
  // transposing LDS reads of four rows each. Lane (q4, c16 = 4 e + j)
  // addresses row 4 q4 + e (+ 32 ks + 16 h), columns 16 db + 4 j .. + 3, and
  // receives column 16 db + c16 of those four rows.
  const int tr_e = c16 >> 2, tr_j = c16 & 3;
  const int tr_row = 4 * q4 + tr_e;
  const int tr_sw = tr_row & (CPR - 1);
  int trd[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    trd[db] = tr_row * D + (((2 * db + (tr_j >> 1)) ^ tr_sw) * 8) + (tr_j & 1) * 4;
  f32x4 oacc[NDB];  // O^T rows 16 db + 4 q4 + i, column (query row) c16
  u32x4 vreg[KPG];

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
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_prev = -INFINITY;
    float l_acc = 0.f;
    int skipped = 0;

    // The V rows of a kept tile are loaded right after its vote, and its P.V
    // runs one step later, after the scores and the vote of the next tile:
    // the V load has the next tile's matrix work to land behind. Its P (bf16
    // B operands) and rescale factor wait in registers meanwhile.
    bool pend = false;  // a kept tile awaits its P.V (V in vreg, P in p_pend)
    bf16x8 p_pend[2];
    float alpha_pend = 1.f;
    auto pv_pending = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[db][i] *= alpha_pend;
      // (one wave: its LDS accesses complete in order, so the reads below
      // see these writes, and the writes follow the previous tile's reads)
#pragma unroll
      for (int m = 0; m < KPG; ++m) store16(v_lds + vw_base + m * D + ((cc ^ m) * 8), vreg[m]);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint64_t lo = lds_read_tr16(v_lds + trd[db] + (32 * ks) * D);
          const uint64_t hi = lds_read_tr16(v_lds + trd[db] + (32 * ks + 16) * D);
          const u32x4 va = {(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
          oacc[db] = mfma16(as_bf16x8(va), p_pend[ks], oacc[db]);
        }
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
      // Exponentials of this tile (bf16 B operands, zero in the padding
      // columns c16 >= G), the P.V of the pending tile, then this tile's V
      // rows -- keys kbase + rg*KPG + m, d chunk cc -- into the registers
      // it freed.
      const float m_new = fmaxf(m_prev, mloc);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2((m_prev - m_use) * a.c_log2);
      const float mc = m_use * a.c_log2;
      float psum = 0.f;
      bf16x8 p_new[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 w;
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
          const f32x4& sk = s[2 * ks + t / 4];
          float x0 = fast_exp2(fmaf(sk[t % 4], a.c_log2, -mc));
          float x1 = fast_exp2(fmaf(sk[t % 4 + 1], a.c_log2, -mc));
          if (c16 >= G) x0 = x1 = 0.f;
          psum += x0 + x1;
          w[t / 2] = cvt_pk_bf16(x0, x1);
        }
        p_new[ks] = as_bf16x8(w);
      }
      l_acc = l_acc * alpha + psum;
      m_prev = m_new;
      if (pend) pv_pending();
      p_pend[0] = p_new[0];
      p_pend[1] = p_new[1];
      alpha_pend = alpha;
      const auto rsv = wave_rsrc(vp + (size_t)kbase * D, max(0, min(n - kbase, BC)) * D * 2);
#pragma unroll
      for (int m = 0; m < KPG; ++m) vreg[m] = load16_buf(rsv, v_off + m * D * 2);
      pend = true;
    }
    if (pend) pv_pending();

    float l_tot = l_acc + __shfl_xor(l_acc, 16, kWave);
    l_tot += __shfl_xor(l_tot, 32, kWave);
    const size_t base = ((size_t)b * a.Hq + hq0) * a.nS + sp;
    if (c16 < G) {
      float* dst = a.ws_o + (base + (size_t)c16 * a.nS) * D + q4 * 4;
#pragma unroll
      for (int db = 0; db < NDB; ++db) *reinterpret_cast<f32x4*>(dst + db * 16) = oacc[db];
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
// sqrt(d) - top) o_s / tot, lse = top + ln tot. A lane owns D / 64
// adjacent output elements (one 4- or 8-byte load per partial row); the
// first U partial rows of a batch are loaded together with the batch's
// (m, l) pairs, since neither depends on the other, and each split's
// weight reaches every lane by a scalar read.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  constexpr int E = D / kWave;  // output elements per lane
  constexpr int U = 32;         // partial rows in flight per lane
  using Vec = typename std::conditional<E == 2, float2, float>::type;
  static_assert(E == 1 || E == 2, "head dim 64 or 128");
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int n = min(max(a.seqlens[b], 0), a.S_max);
  const int ntiles = (n + BC - 1) / BC;
  const int nsp = (ntiles + a.T - 1) / a.T;
  const size_t base = ((size_t)b * a.Hq + hq) * a.nS;
  const Vec* po = reinterpret_cast<const Vec*>(a.ws_o + base * D) + lane;
  const float2* pml = reinterpret_cast<const float2*>(a.ws_ml) + base;
  float top = -INFINITY, tot = 0.f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < nsp; s0 += kWave) {
    const int s = s0 + lane;
    const int cnt = min(kWave, nsp - s0);
    const float2 ml = s < nsp ? pml[s] : make_float2(0.f, 0.f);
    Vec oo[U];
#pragma unroll
    for (int u = 0; u < U; ++u) oo[u] = u < cnt ? po[(size_t)(s0 + u) * kWave] : Vec{};
    float x = -INFINITY, ms = -INFINITY;
    if (ml.y > 0.f) {
      ms = ml.x * a.inv_sqrt_d;
      x = ms + __logf(ml.y);
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
    for (int u0 = 0; u0 < cnt; u0 += U) {
      if (u0 > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          oo[u] = u0 + u < cnt ? po[(size_t)(s0 + u0 + u) * kWave] : Vec{};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float w = __int_as_float(
            __builtin_amdgcn_readlane(__float_as_int(wo), (u0 + u) & (kWave - 1)));
        const float* o = reinterpret_cast<const float*>(&oo[u]);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(w, o[e], acc[e]);
      }
    }
  }
  const float lse = (tot > 0.f) ? top + __logf(tot) : -INFINITY;
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  uint16_t ob[E];
#pragma unroll
  for (int e = 0; e < E; ++e) ob[e] = __builtin_bit_cast(uint16_t, (__bf16)(acc[e] * inv));
  uint16_t* dst = a.out + ((size_t)b * a.Hq + hq) * D + lane * E;
  if constexpr (E == 2)
    *reinterpret_cast<uint32_t*>(dst) = (uint32_t)ob[0] | ((uint32_t)ob[1] << 16);
  else
    *dst = ob[0];
  if (a.lse && lane == 0) a.lse[(size_t)b * a.Hq + hq] = lse;
}

// The split kernel's work counter is set before every launch (a kernel, not
// a memset, so that the launch sequence can be captured in a graph): wave w
// starts with item w, so the first ticket handed out is the wave count.
__global__ void decode_queue_reset(uint32_t* queue, uint32_t first) {
  if (threadIdx.x == 0) *queue = first;
}

// Waves of the persistent split kernel on the current device: three per CU
// (fewer cache streams in flight read faster: with MFMA P.V on the
// 32-sequence decode, 512 waves 0.445 ms, 640 0.441, 768 0.437, 1024
// 0.440), the CU count looked up once per device.
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
  const int r = 3 * cus;
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
