// Device helpers shared by the gfx950 kernels of the DSA path (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// 16 raw bytes as a native vector (HIP's uint4 is a struct, whose copies become memcpy)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 64;  // positions per page
constexpr int kWave = 64;   // CDNA wavefront width

#define DSA_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// 16x16x32 bf16 MFMA, fp32 accumulate.
// A: lane l holds row l%16, 8 k-values; B: lane l holds column l%16, 8 k-values (the
// same 8 k-slots as A for lanes of the same l/16 group).  C: lane l holds
// rows 4*(l/16) + j (j = 0..3) of column l%16.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16 MFMA.  A: lane l holds row l%32; B: column l%32; 8 k-values each.
// C: lane l, slot j holds row 8*(j/4) + 4*(l/32) + (j%4) of column l%32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int mfma32_row(int lane, int j) {
  return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
}

// Transposed LDS read of 16-bit data (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives in slot j the element (i % 4) of the 4-element (8-byte) run
// addressed by lane 4*j + i/4 of the same group.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* lds_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(DSA_LDS(s16x4, const_cast<void*>(lds_addr)));
}

__device__ __forceinline__ bf16x8 as_bf8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint16_t f2bf_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}


// Compiler-level ordering point for LDS traffic exchanged between lanes of one wave
// (LDS operations of a wave execute in order in hardware).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

// Wave-wide scans and reductions on DPP (VALU lane moves, no LDS round trip): row_shr
// steps scan each 16-lane row, then row_bcast:15 / row_bcast:31 carry the row totals
// into the rows above.  Out-of-row sources read as 0 (bound_ctrl), the identity of both
// add and unsigned max.  All 64 lanes must be active.
#define DSA_DPP(v, ctrl, rows, bc) \
  ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(v), (ctrl), (rows), 0xf, (bc)))

__device__ __forceinline__ uint32_t wave_incl_add(uint32_t v) {
  v += DSA_DPP(v, 0x111, 0xf, true);   // row_shr:1
  v += DSA_DPP(v, 0x112, 0xf, true);   // row_shr:2
  v += DSA_DPP(v, 0x114, 0xf, true);   // row_shr:4
  v += DSA_DPP(v, 0x118, 0xf, true);   // row_shr:8
  v += DSA_DPP(v, 0x142, 0xa, false);  // row_bcast:15 into rows 1 and 3
  v += DSA_DPP(v, 0x143, 0xc, false);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Maximum over the wave, in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, DSA_DPP(v, 0x111, 0xf, true));
  v = max(v, DSA_DPP(v, 0x112, 0xf, true));
  v = max(v, DSA_DPP(v, 0x114, 0xf, true));
  v = max(v, DSA_DPP(v, 0x118, 0xf, true));
  v = max(v, DSA_DPP(v, 0x142, 0xa, false));
  v = max(v, DSA_DPP(v, 0x143, 0xc, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// max(x, 0) for finite x as a single v_med3_f32 (clamp to [0, FLT_MAX]).  fmaxf costs two
// instructions in IEEE mode: the compiler first quiets a possible signalling NaN.
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.4028235e38f); }

// Reductions over the four 16-lane rows of a wave, per column (lanes c, c+16, c+32, c+48),
// with gfx950's row-swap instructions: permlane16_swap pairs rows (0,1) and (2,3),
// permlane32_swap pairs the two halves; every lane ends with the column's result, and the
// lanes of one column add in the same order.
__device__ __forceinline__ float rows4_max(float v) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two floats as packed bf16 (round to nearest even): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), h2));
}

__device__ __forceinline__ float max2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); }

// Max / sum of a lane's value and the same lane's in the other half of the wave (lanes l and
// l ^ 32 hold the same row of an MFMA tile), in both: one permlane32 swap.  Both halves add
// or compare the same two values, so they end with the same result.
__device__ __forceinline__ float half_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Minimum over the wave, in every lane (min a = ~max ~a keeps 0 the identity).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }

// Makes `v` available in registers at this point: its loads complete here rather than
// wherever the scheduler would sink them (e.g. into a loop whose waits it would then
// count against loads issued outside its view).
template <typename T>
__device__ __forceinline__ void settle(const T& v) {
  asm volatile("" ::"v"(v));
}

// s_waitcnt immediate waiting for LDS/scalar operations only (gfx9 encoding: vmcnt[3:0]
// and [15:14] all ones, expcnt[6:4] all ones, lgkmcnt[11:8] zero)
#define DSA_LGKMCNT0 0xc07f

// Workgroup barrier for LDS traffic only: waits for the wave's own LDS operations, not for
// global loads still in flight into registers (prefetched tiles stay in flight across it).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(DSA_LGKMCNT0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace dsa
