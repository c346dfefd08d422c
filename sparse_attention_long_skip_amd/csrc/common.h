// Device-side helpers shared by the Skip-Softmax kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// 32x32x16 bf16 matrix-core product, fp32 accumulate.
// Operand layout (lane l, half h = l / 32): A supplies row (l % 32) and
// reduction indices 8h..8h+7; B supplies column (l % 32) and the same
// reduction indices; the accumulator holds column (l % 32) and rows
// 8*(i/4) + 4h + (i%4) for element i.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 matrix-core product, fp32 accumulate. Operand layout (lane
// l, group q = l / 16): A supplies row (l % 16) and reduction indices
// 8q..8q+7; B supplies column (l % 16) and the same reduction indices; the
// accumulator holds column (l % 16) and rows 4q + i for element i.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 x) { return __builtin_bit_cast(u32x4, x); }

// Two fp32 -> packed bf16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo;
  __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max across all 64 lanes of a wave.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

// Value held by lane (l ^ 32).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, kWave); }

// max(x[l], x[l ^ 32]) for every lane, through the half-wave swap
// (v_permlane32_swap): after swapping, one result holds the lane's own value
// and the other the opposite half's, in either order.
__device__ __forceinline__ float max_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Number of XCDs; workgroups are dealt to them round-robin by id.
constexpr int kNumXcd = 8;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Two fp32 -> one packed bf16 pair with a single conversion (RNE).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Asynchronous 16-byte global -> LDS copy: lane i's chunk lands at
// lds_base + 16 * i (lds_base must be wave-uniform).
__device__ __forceinline__ void load_lds16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)gsrc,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// Buffer resource over [base, base + nbytes): loads through it return zero
// (and an LDS-direct load writes zero) for every dword at or past nbytes.
// The last dword holds the gfx9 buffer format word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, 0x00020000);
}

// Asynchronous 16-byte buffer -> LDS copy: lane i's chunk at byte offset
// voff of the buffer lands at lds_base + 16 * i (lds_base wave-uniform);
// out-of-range chunks land as zeros.
__device__ __forceinline__ void load_lds16_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_base, 16, (int)voff, 0,
                                           0, 0);
}

// Wait until every global load of this wave (including LDS-direct ones) is
// done: s_waitcnt with vmcnt = 0 and the other counters at their maximum
// (expcnt 7, lgkmcnt 15). Issued through the builtin rather than inline asm
// so that the compiler's own wait insertion knows the loads have landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until every global load (LDS-direct ones included) AND every LDS
// access of this wave is done: vmcnt 0, lgkmcnt 0 (expcnt at its maximum).
__device__ __forceinline__ void wait_vmem_lds() { __builtin_amdgcn_s_waitcnt(0x0070); }

// Workgroup barrier for LDS hand-offs between waves. The release fence of
// __syncthreads() is meant to wait for this wave's LDS writes, but where the
// barrier heads a loop the compiler has been seen to drop that wait on the
// back edge (an LDS write at the end of one iteration, the barrier at the
// top of the next): the write could then land after another wave's read.
// This barrier first waits for all of this wave's LDS operations (lgkmcnt 0)
// with a wait the compiler keeps.
__device__ __forceinline__ void sync_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __syncthreads();
}

// LDS transpose read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane li receives element (li % 4) of the 8-byte chunks addressed by lanes
// 4e + li / 4, for e = 0..3.
__device__ __forceinline__ uint64_t lds_read_tr16(const void* lds_addr) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(lds_addr));
  return __builtin_bit_cast(uint64_t, v);
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// 16-byte buffer load at byte offset voff: zero when the chunk lies at or
// past the resource's end. Only the vector and immediate offsets take part
// in that range check (a scalar offset would not), so the whole offset
// goes in voff.
__device__ __forceinline__ u32x4 load16_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)voff, 0, 0));
}
__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace ssa
