// Skip-Softmax prefill kernel for gfx950.
//
// Operation (TRT-LLM "Skip Softmax" page, three-step algorithm; SpargeAttn
// page, stage two): FlashAttention tiled attention; per (query tile, key
// tile) the tile is skipped -- no exp, no P.V, no V load -- when every row's
// block-local max is more than |lambda| below its running max.
//
// Design:
//  * One workgroup per (batch, query head, query tile of BR rows); BR/32
//    waves, each owning 32 query rows; two workgroups per CU so that one
//    workgroup's exponentials overlap the other's matrix work. The decision
//    unit is the whole query tile, or, with Br = 32, each wave (SpargeAttn's
//    warp-granular variant). A tile that some unit keeps is loaded and run
//    through every wave of the workgroup; in a wave whose unit skips it the
//    exponentials are forced to zero, so the result is that of the per-unit
//    rule.
//  * Scores are computed transposed, S^T = K Q^T, with 32x32x16 bf16 MFMA:
//    K rows come from LDS (A operand), Q stays in registers (B operand). The
//    accumulator then gives every lane ONE query row (lane % 32) and 16 keys
//    per 32-key block, so row max / row sum / rescale are lane-local plus one
//    half-wave swap.
//  * The output is accumulated transposed as well, O^T = V^T P^T: the P
//    registers are already the B operand (same lane = query), and the V^T
//    A operand comes straight from the row-major V tile in LDS through the
//    transposing LDS read (ds_read_b64_tr_b16).
//  * K and V tiles go from HBM to LDS with LDS-direct 16-byte loads (no
//    staging registers), into XOR-swizzled rows so that both the K row reads
//    and the transposing V reads are free of bank conflicts. K and V are
//    double-buffered (V alternates per kept tile).
//  * Software pipeline over the visited tiles, ONE barrier per step t:
//      wait for this wave's loads; barrier (K(t), the last kept V, flags(t-1)
//      visible); workgroup vote of tile t-1 (OR of the per-wave ballots); if
//      tile t-1 is kept: P.V of the previous kept tile interleaved with
//      exp -> P(t-1) (bf16 registers), chunk by chunk, with the K(t+1)
//      loads, then the V(t-1) loads and the scores of tile t; otherwise the
//      scores of tile t, then the K(t+1) loads; row max, gap against the
//      running max, wave ballot.
//    So V is fetched only for kept tiles and has at least a whole step to
//    land, and the exponentials run in the shadow of the matrix work.
//  * The exponentials use a reference max that lags the running max: O and
//    the row sum are rescaled only when a row max exceeds the reference by
//    more than 2^8 in the exp2 domain (softmax is exact for any reference;
//    P stays <= 256).
//  * Workgroups are mapped so that every XCD (own L2) works through whole KV
//    heads, heaviest causal query tiles first, the G query heads of one KV
//    head on consecutive slots: the K/V tiles they stream stay L2-resident.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace ssa {

namespace {

constexpr int BC = 64;

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;
  int32_t* skip_counts;
  uint8_t* tile_state;
  float* tile_margin;
  int B, Hq, Hkv, L, nQ, nK, G;
  int tasks, per_xcd;  // B*Hq*nQ work items; workgroup slots per XCD
  int xcd_rr;          // deal groups of G items round-robin over the XCDs
  float lam_raw;       // lambda * sqrt(d): threshold on raw q.k differences
  float c_log2;        // log2(e) / sqrt(d)
  float inv_sqrt_d;
  int causal;
  const int32_t* block_idx;
  const int32_t* block_cnt;
  int max_blocks;
  int nm_n, nm_m, dense_sink, dense_recent;  // N:M sparse softmax (NM instances)
  int nQ_unit;    // decision units (query tiles of Br rows) per (batch, head)
};

// 16-byte chunk swizzles of a tile row (physical chunk = logical ^ swz(row)).
// K rows are read 16 rows x one chunk at a time; V rows 4 rows x 4 chunks.
template <int D>
__device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

template <int N>
struct StepParity {
  static constexpr int value = N;
};


// BR: query rows per workgroup (BR / 32 waves). UW: waves per decision unit
// (the query tile of Br = 32 * UW rows); a workgroup holds BR / (32 UW)
// units that vote separately and share the K/V tiles (V is loaded when any
// unit keeps the tile). STATS: write per-tile decisions / margins (a
// separate instance, so the hot instance carries none of that code).
// SPARSE: visit a per-tile block list (one unit per workgroup). NM: N:M
// sparse softmax on the scores before the tile rule.
template <int D, int BR, bool STATS, bool SPARSE, bool NM, int UW>
__global__ __launch_bounds__(BR * 2) __attribute__((amdgpu_waves_per_eu(D == 64 && BR == 64 ? 3 : 2)))
void prefill_kernel(PrefillArgs a) {
  constexpr int NW = BR / 32;
  constexpr int NU = NW / UW;  // decision units per workgroup
  static_assert(NU * UW == NW && (!SPARSE || NU <= 2), "unit layout");
  constexpr int NT = NW * kWave;
  constexpr int CPR = D / 8;                   // 16-byte chunks per row
  constexpr int TILE = BC * D;                 // bf16 elements per K or V tile
  constexpr int LPW = TILE * 2 / 1024 / NW;    // 1 KiB LDS-direct loads per wave per tile
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;

  __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[TILE];
  // d = 64 with 64-row tiles: one V buffer (24 KiB of LDS per workgroup, six
  // workgroups -- three waves per SIMD -- per CU); the V load of a kept tile
  // then waits for a second barrier, after every wave's P.V of the tile
  // before it.
  constexpr bool VSINGLE = D == 64 && BR == 64;
  // The two K buffers are separate LDS objects and every step names its K
  // buffers at compile time (the loop below is unrolled by two); the V
  // buffers alternate per kept tile. The compiler then sees that the reads
  // of one buffer cannot alias the LDS-direct loads into another (V is
  // loaded after the P.V reads of a step), and does not wait for loads in
  // flight before the P.V or the scores.
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[VSINGLE ? 1 : 2][TILE];
  __shared__ float flag_lds[2][NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int r32 = lane & 31;

  // XCD-aware work mapping (workgroups are dealt to the XCDs round-robin by
  // index). Items are ordered (batch, KV head), heaviest query tile first,
  // the G heads of a tile adjacent. When the (batch, KV head) pairs divide
  // evenly over the XCDs, XCD x takes the contiguous items
  // [x*per_xcd, (x+1)*per_xcd): whole KV heads, so K/V stay in its L2.
  // Otherwise the groups of G items (one query tile of one KV head) are
  // dealt round-robin to the XCDs, which balances the causal work.
  const int xcd = blockIdx.x % kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  int task;
  if (a.xcd_rr) {
    const int kq = slot / a.G;
    const int grp = kq * kNumXcd + xcd;
    if (grp >= a.tasks / a.G) return;
    task = grp * a.G + (slot - kq * a.G);
  } else {
    task = xcd * a.per_xcd + slot;
    if (slot >= a.per_xcd || task >= a.tasks) return;
  }
  const int per_bkv = a.G * a.nQ;
  const int bkv = task / per_bkv;
  const int rem = task - bkv * per_bkv;
  const int i = a.nQ - 1 - rem / a.G;  // heaviest query tiles first
  const int hq = (bkv % a.Hkv) * a.G + rem % a.G;
  const int b = bkv / a.Hkv;
  const int kvh = hq / a.G;
  const int L = a.L;
  const int q0 = i * BR;
  const int row = q0 + w * 32 + r32;
  const bool row_ok = row < L;
  const int last_row = min(q0 + BR, L) - 1;
  // This wave's decision unit u covers rows [q0 + 32 UW u, q0 + 32 UW (u + 1)).
  const int u = w / UW;
  const bool unit_rows = q0 + u * UW * 32 < L;
  const int unit_last = min(q0 + (u + 1) * UW * 32 - 1, L - 1);
  const size_t unit_id = (size_t)(b * a.Hq + hq) * a.nQ_unit + (size_t)i * NU + u;

  const uint16_t* qp = a.q + ((size_t)(b * a.Hq + hq) * L) * D;
  const uint16_t* kp = a.k + ((size_t)(b * a.Hkv + kvh) * L) * D;
  const uint16_t* vp = a.v + ((size_t)(b * a.Hkv + kvh) * L) * D;
  const size_t unit = ((size_t)(b * a.Hq + hq) * a.nQ + i);

  // Query rows as the B operand: lane holds row (lane % 32), d chunk 16*kk + 8h.
  bf16x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row_ok) x = load16(qp + (size_t)row * D + kk * 16 + h * 8);
    qf[kk] = as_bf16x8(x);
  }

  // Visit sequence: (tile j, mask of the units that visit it), j = -1 at the
  // end. Dense: ascending tiles up to the causal limit, every unit (a unit
  // whose rows cannot see a tile skips its vote through uvis below). Block
  // lists: each unit visits the valid entries of its own list in list order.
  // With two units per workgroup (64-row units of a block list) the two
  // lists are merged by tile index when both are ascending -- a tile on both
  // lists is visited once for both, and each unit still sees its own tiles
  // in its own order -- and otherwise visited one after the other.
  constexpr int kEnd = 0x7fffffff;
  int cur_t = 0;  // dense cursor
  const int n_dense = a.causal ? (last_row / BC + 1) : a.nK;
  const int32_t* lp[NU];
  int nl[NU], ulim[NU], pos[NU], head[NU], cbase[NU], cval[NU];
  bool merge = true;
  if (SPARSE) {
#pragma unroll
    for (int uu = 0; uu < NU; ++uu) {
      const size_t uid = (size_t)(b * a.Hq + hq) * a.nQ_unit + (size_t)i * NU + uu;
      const bool exists = i * NU + uu < a.nQ_unit;
      lp[uu] = a.block_idx + (exists ? uid : 0) * a.max_blocks;
      nl[uu] = exists ? min(max(a.block_cnt[uid], 0), a.max_blocks) : 0;
      ulim[uu] = min(q0 + (uu + 1) * UW * 32 - 1, L - 1);
      pos[uu] = 0;
      cbase[uu] = -64;
      cval[uu] = 0;
    }
  }
  // A block list is read 64 entries at a time, one per lane, and entry t is
  // taken from lane t % 64: one vector load per 64 tiles instead of a load
  // (and a wait behind the tile loads in flight) per tile.
  auto entry = [&](int uu, int t) -> int {
    const int blk = t & ~63;
    if (blk != cbase[uu]) {
      cbase[uu] = blk;
      cval[uu] = blk + lane < nl[uu] ? lp[uu][blk + lane] : -1;
    }
    return __builtin_amdgcn_readlane(cval[uu], t & 63);
  };
  auto valid_u = [&](int uu, int j) -> bool {
    return j >= 0 && j < a.nK && (!a.causal || j * BC <= ulim[uu]);
  };
  // head[uu]: the tile at the first valid position >= pos[uu] (kEnd if none).
  auto seek = [&](int uu) {
    for (; pos[uu] < nl[uu]; ++pos[uu]) {
      const int j = entry(uu, pos[uu]);
      if (valid_u(uu, j)) {
        head[uu] = j;
        return;
      }
    }
    head[uu] = kEnd;
  };
  if (SPARSE) {
#pragma unroll
    for (int uu = 0; uu < NU; ++uu) {
      if (NU > 1) {
        // strictly ascending valid entries? (each valid entry above the
        // largest valid entry before it: a prefix max across the lanes)
        int before = -1;
        for (int t0 = 0; t0 < nl[uu]; t0 += 64) {
          const int j = t0 + lane < nl[uu] ? lp[uu][t0 + lane] : -1;
          const bool v = valid_u(uu, j);
          int pm = v ? j : -1;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(pm, o, kWave);
            if (lane >= o) pm = max(pm, y);
          }
          int ex = __shfl_up(pm, 1, kWave);
          ex = max(lane == 0 ? -1 : ex, before);
          if (__ballot(v && j <= ex) != 0ull) merge = false;
          before = max(before, __shfl(pm, 63, kWave));
        }
      }
      seek(uu);
    }
  }
  auto next_tile = [&](int& j, int& m) {
    if (!SPARSE) {
      j = cur_t < n_dense ? cur_t++ : -1;
      m = (1 << NU) - 1;
      return;
    }
    if (NU == 1) {
      j = head[0] == kEnd ? -1 : head[0];
      m = 1;
      if (j >= 0) {
        ++pos[0];
        seek(0);
      }
      return;
    }
    const int h0 = head[0], h1 = head[NU - 1];
    if (merge) {
      const int jm = min(h0, h1);
      j = jm == kEnd ? -1 : jm;
      m = (h0 == jm ? 1 : 0) | (h1 == jm ? 2 : 0);
      if (j < 0) m = 0;
    } else {
      j = h0 != kEnd ? h0 : (h1 != kEnd ? h1 : -1);
      m = j < 0 ? 0 : (h0 != kEnd ? 1 : 2);
    }
#pragma unroll
    for (int uu = 0; uu < NU; ++uu)
      if ((m >> uu) & 1) {
        ++pos[uu];
        seek(uu);
      }
  };

  // LDS-direct tile loads: this wave fills LPW consecutive 1 KiB blocks; LDS
  // slot s (16 B) holds row s / CPR, logical chunk (s % CPR) ^ swz(row).
  // Per-lane source offsets are fixed; a tile is read through a buffer
  // resource that ends at row L, so rows past L (last tile only) land as
  // zeros (their scores are masked and their P is 0), with no per-lane
  // clamp and no branch.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // Source offsets are in bytes from the tile's first row.
  uint32_t koff[LPW], voff[LPW];
#pragma unroll
  for (int r = 0; r < LPW; ++r) {
    const int s = (w * LPW + r) * 64 + lane;
    const int rr = s / CPR;
    koff[r] = (uint32_t)(rr * D + ((s % CPR) ^ swz_k<D>(rr)) * 8) * 2u;
    voff[r] = (uint32_t)(rr * D + ((s % CPR) ^ swz_v<D>(rr)) * 8) * 2u;
  }
  // The resource is built per tile with scalar instructions only.
  auto load_tile = [&](const uint16_t* src, int j, uint16_t* dst, const uint32_t* off) __attribute__((always_inline)) {
    const int kb0 = j * BC;
    const auto rs = make_rsrc(src + (size_t)kb0 * D, min(L - kb0, BC) * D * 2);
#pragma unroll
    for (int r = 0; r < LPW; ++r) load_lds16_buf(rs, off[r], dst + (wu * LPW + r) * 512);
  };

  float m_run = -INFINITY;  // running max of raw q.k over visited tiles (the vote)
  float m_ref = -INFINITY;  // reference max of the exponentials (lags m_run)
  float l_acc = 0.f;        // partial row sum over this lane's keys, relative to m_ref
  // Rescale O only when a row max exceeds the reference by more than 2^8 in
  // the exp2 domain; P <= 256 otherwise. Softmax is exact for any reference.
  const float tau_raw = 8.f / a.c_log2;
  f32x16 o[NDB];
#pragma unroll
  for (int nb = 0; nb < NDB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[nb][e] = 0.f;
  f32x16 s[2];  // scores of the latest tile
  // P of the last kept tile, awaiting its P.V (V in buffer vpar). Before
  // the first kept tile it is zero against a zeroed V buffer.
  bf16x8 p[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) p[c] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  int vpar = 0;
  bool pend = false;  // 32-row units: this wave's P awaits its P.V
#pragma unroll
  for (int x = tid; x < TILE / 8; x += NT) store16(v_lds[0] + x * 8, u32x4{0u, 0u, 0u, 0u});
  int skipped = 0;

  // Per-lane element offsets of the transposing V reads of rows 0..15, one
  // per 32-column block; rows kc + 0..15 (kc a multiple of 8) add kc * D,
  // since the V swizzle depends only on row bits that kc leaves unchanged.
  // The empty asm keeps each offset opaque, so every read address is one
  // offset from the buffer: the compiler then keeps the alias information
  // that tells it the read cannot touch the buffer being loaded.
  int vrd[NDB];
#pragma unroll
  for (int nb = 0; nb < NDB; ++nb) {
    const int g16 = lane >> 4;
    const int jj = lane & 15;
    const int c = nb * 4 + (g16 & 1) * 2 + ((jj & 3) >> 1);
    const int ra = 4 * h + (jj >> 2);
    vrd[nb] = ra * D + ((c ^ swz_v<D>(ra)) * 8) + (jj & 1) * 4;
    asm("" : "+v"(vrd[nb]));
  }

  // Per-lane element offsets of the K row reads for the scores, one per
  // 16-wide reduction slice kk (key row r32; rows 32 + r32 add 32 * D, the K
  // swizzle depending only on the low row bits), opaque for the same reason.
  int krd[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    krd[kk] = r32 * D + (((2 * kk + h) ^ swz_k<D>(r32)) * 8);
    asm("" : "+v"(krd[kk]));
  }

  // O^T += V^T P^T from the V tile at vt. A operand for (nb, kb, gp): element
  // e of lane (h, r32) = V[kc + 8*(e/4) + 4h + e%4][32 nb + r32].
  // P chunk c (keys 16c .. 16c + 15 of a tile) is p[c]; it comes from the
  // scores s[c / 2][8 (c % 2) .. 8 (c % 2) + 7].
  auto pv_chunk = [&](const uint16_t* vt, int c) __attribute__((always_inline)) {
    const int kc = c * 16;
#pragma unroll
    for (int nb = 0; nb < NDB; ++nb) {
      const uint64_t lo = lds_read_tr16(vt + vrd[nb] + kc * D);
      const uint64_t hi = lds_read_tr16(vt + vrd[nb] + (kc + 8) * D);
      u32x4 va = {(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
      o[nb] = mfma32(as_bf16x8(va), p[c], o[nb]);
    }
  };
  // S^T = K Q^T, keys 32 kb .. 32 kb + 31 of the K tile at kl, for this
  // wave's 32 rows (one accumulator chain).
  auto scores_half = [&](const uint16_t* kl, int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const bf16x8 ka = as_bf16x8(load16(kl + krd[kk] + kb * 32 * D));
      s[kb] = mfma32(ka, qf[kk], s[kb]);
    }
  };
  // exp2 of chunk c of the latest scores, with 1/sqrt(d) and log2(e) folded
  // in, against the scaled reference mc; packed to bf16 into p[c].
  auto exp_chunk = [&](int c, float mc, float& psum) __attribute__((always_inline)) {
    const int kb = c >> 1, gp = c & 1;
    u32x4 pk;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float x0 = fast_exp2(fmaf(s[kb][gp * 8 + e], a.c_log2, -mc));
      const float x1 = fast_exp2(fmaf(s[kb][gp * 8 + e + 1], a.c_log2, -mc));
      psum += x0 + x1;
      pk[e >> 1] = cvt_pk_bf16(x0, x1);
    }
    p[c] = as_bf16x8(pk);
  };

  // N:M sparse softmax (Model Optimizer tutorial, step 2; FAQ on sink and
  // recent tokens): in every aligned group of M consecutive keys a row keeps
  // its top-N allowed scores (ties: lower key), plus keys below dense_sink
  // and keys in (row - dense_recent, row]; the rest become -inf. A lane
  // holds, per 8-key block, 4 consecutive keys (8q + 4h + 0..3), so groups
  // of 2 or 4 are lane-local.
  auto nm_sparsify = [&](int kbase) __attribute__((always_inline)) {
    const bool exempt_here = (kbase < a.dense_sink) ||
        (a.dense_recent > 0 && kbase + BC - 1 > q0 + wu * 32 - a.dense_recent);
    // e is dropped when at least N members of its group beat it (a higher
    // score, or an equal score at a lower key). For e < f one comparison
    // decides the pair: f beats e iff x[f] > x[e], else e beats f (scores
    // are never NaN). With M = 4, "at least N of e's three possible
    // beaters" is their OR (N = 1), majority (N = 2) or AND (N = 3), taken
    // on the comparisons' wave-wide lane masks by the scalar unit.
    // MODE 1, 2, 3: M = 4 with N = 1, 2, 3; MODE 4: M = 2 with N = 1.
    auto groups = [&](auto mode_c) __attribute__((always_inline)) {
      constexpr int MODE = decltype(mode_c)::value;
      auto atleast = [&](uint64_t p, uint64_t q, uint64_t r) __attribute__((always_inline)) -> uint64_t {
        if constexpr (MODE == 1) return p | q | r;
        else if constexpr (MODE == 2) return (p & q) | (r & (p | q));
        else return p & q & r;
      };
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = s[kb][q4 * 4 + e];
          const uint64_t c01 = __builtin_amdgcn_ballot_w64(x[1] > x[0]);
          const uint64_t c23 = __builtin_amdgcn_ballot_w64(x[3] > x[2]);
          uint64_t drop[4];
          if constexpr (MODE == 4) {
            drop[0] = c01;
            drop[1] = ~c01;
            drop[2] = c23;
            drop[3] = ~c23;
          } else {
            const uint64_t c02 = __builtin_amdgcn_ballot_w64(x[2] > x[0]);
            const uint64_t c03 = __builtin_amdgcn_ballot_w64(x[3] > x[0]);
            const uint64_t c12 = __builtin_amdgcn_ballot_w64(x[2] > x[1]);
            const uint64_t c13 = __builtin_amdgcn_ballot_w64(x[3] > x[1]);
            drop[0] = atleast(c01, c02, c03);
            drop[1] = atleast(~c01, c12, c13);
            drop[2] = atleast(~c02, ~c12, c23);
            drop[3] = atleast(~c03, ~c13, ~c23);
          }
          if (exempt_here) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int key = kbase + kb * 32 + q4 * 8 + h * 4 + e;
              drop[e] &= ~__builtin_amdgcn_ballot_w64(key < a.dense_sink ||
                                                       (row - a.dense_recent < key && key <= row));
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[kb][q4 * 4 + e] = __builtin_amdgcn_inverse_ballot_w64(drop[e]) ? -INFINITY : x[e];
        }
    };
    // N >= M keeps every key.
    if (a.nm_m == 4) {
      if (a.nm_n == 2) groups(std::integral_constant<int, 2>{});
      else if (a.nm_n == 1) groups(std::integral_constant<int, 1>{});
      else if (a.nm_n == 3) groups(std::integral_constant<int, 3>{});
    } else if (a.nm_n == 1) {
      groups(std::integral_constant<int, 4>{});
    }
  };

  // tiles (and unit masks) of the current, next and previous positions
  int jcur, mcur, jnext, mnext;
  next_tile(jcur, mcur);
  if (jcur >= 0) load_tile(kp, jcur, k_lds0, koff);
  next_tile(jnext, mnext);
  int jprev = -1, mprev = 0;
  // One pipeline step per list position t (the loop runs t = 0 .. n, one
  // barrier each): vote of tile t-1; if kept, P.V of the previous kept tile
  // with the exponentials of tile t-1 and the K(t+1) loads, then V(t-1);
  // scores of tile t (K(t+1) after them when nothing was kept); row max and
  // wave flag of tile t. buf = step parity selects the K buffers.
  auto step = [&](auto buf_c) __attribute__((always_inline)) -> bool {
    constexpr int buf = decltype(buf_c)::value;
    uint16_t* const k_cur = buf == 0 ? k_lds0 : k_lds1;  // K(t), read by the scores
    uint16_t* const k_nxt = buf == 0 ? k_lds1 : k_lds0;  // K(t+1), loaded now
    const bool have_cur = jcur >= 0;
    const bool have_prev = jprev >= 0;
    if (!have_cur && !have_prev) return false;
    // K(t) and the last kept V (LDS-direct loads) and the flags of tile t-1
    // (LDS writes of the previous step, across the loop's back edge) must be
    // complete before the barrier: one wait covers both counters.
    wait_vmem_lds();
    __syncthreads();
    bool keep1 = false;     // some unit keeps tile jprev: exponentials, P.V, V load
    bool keep_mine = false;  // this wave's unit keeps it
    if (have_prev) {
      // keep1: some decision unit of the workgroup keeps the tile;
      // keep_mine: this wave's unit keeps it. A unit whose rows cannot see
      // the tile (causal), or whose list does not hold it, does not count it
      // as visited.
      const bool uvis = SPARSE ? (((mprev >> u) & 1) != 0)
                               : (unit_rows && (!a.causal || jprev * BC <= unit_last));
      if (STATS) {
        float gu = flag_lds[buf ^ 1][u * UW];
#pragma unroll
        for (int ww = 1; ww < UW; ++ww) gu = fmaxf(gu, flag_lds[buf ^ 1][u * UW + ww]);
        float g = gu;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) g = fmaxf(g, flag_lds[buf ^ 1][ww]);
        keep1 = !(g < a.lam_raw);
        keep_mine = !(gu < a.lam_raw);
        if (lane == 0 && w % UW == 0 && uvis) {
          const size_t ti = unit_id * a.nK + jprev;
          if (a.tile_state) a.tile_state[ti] = keep_mine ? 1 : 2;
          if (a.tile_margin) a.tile_margin[ti] = gu * a.inv_sqrt_d;
        }
      } else {
        float fu = 0.f, f = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
          const float x = flag_lds[buf ^ 1][ww];
          f += x;
          if (ww / UW == u) fu += x;
        }
        keep1 = f > 0.f;
        keep_mine = fu > 0.f;
      }
      if (uvis && !keep_mine) ++skipped;
    }
    if (keep1) {
      // Every wave of the workgroup takes a tile that some unit keeps (the
      // V tile and the P.V pipeline are shared); in a wave whose unit
      // skips it the exponentials are exp2(-inf) = 0, so the tile adds
      // nothing to its rows.
      // A reference max that grew is taken first: O, the row sum and the
      // pending P (still to be multiplied into O) move to the new reference.
      // Then the P.V of the previous kept tile and the exponentials of this
      // one run in one block: chunk c of the old P feeds the matrix cores
      // while the exponentials refill chunk c - 1.
      const bool grow = keep_mine && ((m_run > m_ref + tau_raw) || (m_ref == -INFINITY && m_run != -INFINITY));
      if (__ballot(grow) != 0ull) {
        float alpha = 1.f;
        if (grow) {
          alpha = (m_ref == -INFINITY) ? 0.f : fast_exp2((m_ref - m_run) * a.c_log2);
          m_ref = m_run;
        }
#pragma unroll
        for (int nb = 0; nb < NDB; ++nb)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[nb][e] *= alpha;
        l_acc *= alpha;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          u32x4 w4 = as_u32x4(p[c]);
#pragma unroll
          for (int x = 0; x < 4; ++x) w4[x] = cvt_pk_bf16(bf16_lo(w4[x]) * alpha, bf16_hi(w4[x]) * alpha);
          p[c] = as_bf16x8(w4);
        }
      }
      const float mc = !keep_mine ? INFINITY : (m_ref == -INFINITY ? 0.f : m_ref * a.c_log2);
      const uint16_t* vt = v_lds[VSINGLE ? 0 : vpar];
      float psum = 0.f;
      // The K(t+1) loads go out one share after each P.V chunk, so they
      // queue while the matrix cores work. Past the last position the
      // resource is empty and the loads write zeros into the free buffer
      // (no branch splits the block).
      const bool kn = jnext >= 0;
      const int kb0n = kn ? jnext * BC : 0;
      const auto rsk = make_rsrc(kp + (size_t)kb0n * D, kn ? min(L - kb0n, BC) * D * 2 : 0);
      auto k_share = [&](int c) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < LPW; ++r)
          if (r * 4 / LPW == c) load_lds16_buf(rsk, koff[r], k_nxt + (wu * LPW + r) * 512);
      };
      if constexpr (UW == 1) {
        // Every wave is a decision unit of its own (32-row units): the P.V
        // of its pending P runs only if its unit kept the last kept tile,
        // and the exponentials only if its unit keeps this one (branches
        // uniform per wave), so the matrix and exponential work follow the
        // unit's own decisions; the V tile is still shared.
        if (pend) pv_chunk(vt, 0);
        k_share(0);
#pragma unroll
        for (int c = 0; c < 3; ++c) {
          if (pend) pv_chunk(vt, c + 1);
          k_share(c + 1);
          if (keep_mine) exp_chunk(c, mc, psum);
        }
      } else {
        pv_chunk(vt, 0);
        k_share(0);
#pragma unroll
        for (int c = 0; c < 3; ++c) {
          pv_chunk(vt, c + 1);
          k_share(c + 1);
          exp_chunk(c, mc, psum);
        }
      }
      if constexpr (VSINGLE) {
        // Every wave is done reading the V buffer before any wave loads
        // V(t-1) into it: this wave's LDS reads have returned (lgkmcnt 0;
        // vmcnt and expcnt left at their maximum), then a plain barrier (a
        // full __syncthreads() would also wait for the K(t+1) loads).
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        load_tile(vp, jprev, v_lds[0], voff);
      } else {
        vpar ^= 1;
        load_tile(vp, jprev, v_lds[vpar], voff);
      }
      // The scores of tile t (run even past the last tile, where they are
      // not used) overlap the last exponential chunk: keys 0..31 go to s[0],
      // already consumed, while chunk 3 reads s[1].
      scores_half(k_cur, 0);
      if (UW > 1 || keep_mine) exp_chunk(3, mc, psum);
      scores_half(k_cur, 1);
      l_acc += psum;
      if constexpr (UW == 1) pend = keep_mine;
    }
    if (have_cur && !keep1) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 ka = as_bf16x8(load16(k_cur + krd[kk] + kb * 32 * D));
          s[kb] = mfma32(ka, qf[kk], s[kb]);
        }
    }
    // Without a kept tile, K(t+1) is issued after the scores of tile t: the
    // loads queue behind the other waves' loads while the matrix cores work
    // (measured ~1% faster than issuing them right after the vote).
    if (!keep1 && jnext >= 0) load_tile(kp, jnext, k_nxt, koff);
    jprev = -1;
    if (have_cur) {
      const int j = jcur;
      const int kbase = j * BC;
      const bool need_mask = (kbase + BC > L) || (a.causal && kbase + BC - 1 > q0 + w * 32);
      if (need_mask) {
        // key = kbase + 4h + off(kb, e) with a compile-time off; it is masked
        // when key > min(row, L - 1) (causal) or key > L - 1. One per-lane
        // limit instead of a per-element key index keeps registers free.
        const int lim = (a.causal ? min(row, L - 1) : L - 1) - kbase - 4 * h;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (kb * 32 + (e >> 2) * 8 + (e & 3) > lim) s[kb][e] = -INFINITY;
      }
      if (NM) nm_sparsify(kbase);
      if (SPARSE && NU > 1 && ((mcur >> u) & 1) == 0) {
        // the tile is on the other unit's list only: no score of this unit
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) s[kb][e] = -INFINITY;
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, s[kb][e]);
      mloc = max_halves(mloc);
      float gap;
      if (!row_ok || mloc == -INFINITY) gap = -INFINITY;
      else if (m_run == -INFINITY) gap = INFINITY;
      else gap = mloc - m_run;
      if (STATS) {
        const float gw = wave_max(gap);
        if (lane == 0) flag_lds[buf][w] = gw;
      } else {
        const bool wk = __ballot(gap >= a.lam_raw) != 0ull;
        if (lane == 0) flag_lds[buf][w] = wk ? 1.f : 0.f;
      }
      m_run = fmaxf(m_run, mloc);
      jprev = j;
      mprev = mcur;
      jcur = jnext;
      mcur = mnext;
      next_tile(jnext, mnext);
    }
    return true;
  };
  while (step(StepParity<0>{}) && step(StepParity<1>{})) {
  }
  // P.V of the last kept tile (of zeros if none was kept).
  wait_vmem_lds();
  __syncthreads();
  if (UW > 1 || pend) {
#pragma unroll
    for (int c = 0; c < 4; ++c) pv_chunk(v_lds[VSINGLE ? 0 : vpar], c);
  }

  // Epilogue: normalise, write out (bf16) and lse.
  const float l_tot = sum_halves(l_acc);
  if (row_ok) {
    const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = a.out + ((size_t)(b * a.Hq + hq) * L + row) * D;
#pragma unroll
    for (int nb = 0; nb < NDB; ++nb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 st;
        st[0] = cvt_pk_bf16(o[nb][g4 * 4 + 0] * inv_l, o[nb][g4 * 4 + 1] * inv_l);
        st[1] = cvt_pk_bf16(o[nb][g4 * 4 + 2] * inv_l, o[nb][g4 * 4 + 3] * inv_l);
        *reinterpret_cast<u32x2*>(op + nb * 32 + g4 * 8 + h * 4) = st;
      }
    if (a.lse && h == 0)
      a.lse[(size_t)(b * a.Hq + hq) * L + row] =
          l_tot > 0.f ? m_ref * a.inv_sqrt_d + __logf(l_tot) : -INFINITY;
  }
  if (a.skip_counts && lane == 0 && w % UW == 0 && unit_rows) a.skip_counts[unit_id] = skipped;
}

template <int D, int BR, int UW>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)(a.per_xcd * kNumXcd));
  dim3 block(BR * 2);
  const bool stats = a.tile_state || a.tile_margin;
  const bool nm = a.nm_m > 0 && a.nm_n < a.nm_m;
#define SSA_LAUNCH(ST, SP, NMF) \
  hipLaunchKernelGGL((prefill_kernel<D, BR, ST, SP, NMF, UW>), grid, block, 0, stream, a)
  if (a.block_idx != nullptr) {
    if constexpr (BR / 32 == UW || (BR == 128 && UW == 2)) {
      if (stats) SSA_LAUNCH(true, true, false);
      else SSA_LAUNCH(false, true, false);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (nm) {
    if (stats) SSA_LAUNCH(true, false, true);
    else SSA_LAUNCH(false, false, true);
  } else {
    if (stats) SSA_LAUNCH(true, false, false);
    else SSA_LAUNCH(false, false, false);
  }
#undef SSA_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  PrefillArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.out = static_cast<uint16_t*>(p.out);
  a.lse = p.lse;
  a.skip_counts = p.skip_counts;
  a.tile_state = p.tile_state;
  a.tile_margin = p.tile_margin;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.L = p.L;
  // Workgroup rows: Br = 32 units run four to a 128-row workgroup (per-wave
  // votes); at d = 128, Br = 64 units run two to a 128-row workgroup (a
  // 64-row workgroup holds the same 64 KiB of K/V tiles, so only one of its
  // waves would fit per SIMD; with block lists the two lists are merged, so
  // a tile on both is loaded once for 128 rows); otherwise one unit per
  // workgroup. (At d = 64 the 64-row workgroups with one V buffer fit six
  // to a CU, and pairing their block lists measured 12-27% slower on the
  // 32K block-sparse legs.)
  const bool pair64 = p.Br == 64 && p.d == 128;
  const int br_wg = (p.Br == 32 || pair64) ? 128 : p.Br;
  a.nQ = (p.L + br_wg - 1) / br_wg;
  a.nQ_unit = (p.L + p.Br - 1) / p.Br;
  a.nK = (p.L + p.Bc - 1) / p.Bc;
  a.G = p.Hq / p.Hkv;
  a.tasks = p.B * p.Hq * a.nQ;
  a.xcd_rr = (p.B * p.Hkv) % kNumXcd != 0;
  if (a.xcd_rr) {
    const int groups = p.B * p.Hkv * a.nQ;
    a.per_xcd = (groups + kNumXcd - 1) / kNumXcd * a.G;
  } else {
    a.per_xcd = (a.tasks + kNumXcd - 1) / kNumXcd;
  }
  const float sd = sqrtf((float)p.d);
  a.lam_raw = p.lambda * sd;
  a.c_log2 = kLog2e / sd;
  a.inv_sqrt_d = 1.f / sd;
  a.causal = p.causal;
  a.block_idx = p.block_idx;
  a.block_cnt = p.block_cnt;
  a.max_blocks = p.max_blocks;
  a.nm_n = p.nm_n;
  a.nm_m = p.nm_m;
  a.dense_sink = p.dense_sink;
  a.dense_recent = p.dense_recent;
  if (p.Br == 32) {
    if (p.d == 128) return launch<128, 128, 1>(a, stream);
    if (p.d == 64) return launch<64, 128, 1>(a, stream);
  } else if (p.Br == 128) {
    if (p.d == 128) return launch<128, 128, 4>(a, stream);
    if (p.d == 64) return launch<64, 128, 4>(a, stream);
  } else if (p.Br == 64) {
    if (p.d == 128) return launch<128, 128, 2>(a, stream);
    if (p.d == 64) return launch<64, 64, 2>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace ssa
