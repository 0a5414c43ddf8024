// Device-side building blocks shared by the gfx950 attention kernels.
//
// Lane layouts used throughout (wave64, lane l, r = l & 31, half = l >> 5):
//   v_mfma_f32_32x32x16_bf16  A (32 x 16): lane holds A[r][8*half .. 8*half+7]
//                             B (16 x 32): lane holds B[8*half .. 8*half+7][r]
//                             C (32 x 32): lane holds C[8*i + 4*half + j][r] at acc[4*i + j]
//   ds_read_b64_tr_b16        within each group of 16 lanes, output lane j element e is
//                             element (j & 3) of what input lane 4*e + (j >> 2) addressed:
//                             if input lane i reads row (base + i/4), columns
//                             (col + 4*(i%4) .. +3) of a row-major bf16 tile, output lane j
//                             receives column (col + j) of rows base .. base+3.
//   v_permlane32_swap         with both operands equal to x, the two results hold
//                             x[l & 31] and x[(l & 31) + 32].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Workgroup and work-item ids read from the hardware registers. The HIP built-in index
// variables go through device-library functions built with packed fp32 enabled; with that
// feature switched off for this code they are not inlined but called, and their results lose
// the compiler's knowledge that they are the same in every lane of a wave.
__device__ __forceinline__ int group_id_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int thread_id_x() { return (int)__builtin_amdgcn_workitem_id_x(); }

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16: A (16 x 32): lane holds A[l%16][8*(l/16) .. +7]; B (32 x 16):
// lane holds B[8*(l/16) .. +7][l%16]; C (16 x 16): lane holds C[4*(l/16) + i][l%16] at acc[i].
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Value held by the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float pair_max(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(s[0]), __int_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(s[0]) + __int_as_float(s[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 -> bf16 of two values (one v_cvt_pk_bf16_f32), lo first.
__device__ __forceinline__ bf16x2 cvt_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_convertvector(v, bf16x2);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, cvt_bf16x2(lo, hi));
}

// Eight fp32 values -> bf16x8 MFMA operand; `sum` accumulates the eight *rounded* values
// (v_dot2_f32_bf16 of each pair against (1, 1)), i.e. exactly the weights the MFMA uses.
__device__ __forceinline__ bf16x8 pack_bf16x8_sum(const float* a, float& sum) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const bf16x2 p0 = cvt_bf16x2(a[0], a[1]);
  const bf16x2 p1 = cvt_bf16x2(a[2], a[3]);
  const bf16x2 p2 = cvt_bf16x2(a[4], a[5]);
  const bf16x2 p3 = cvt_bf16x2(a[6], a[7]);
  sum = __builtin_amdgcn_fdot2_f32_bf16(p0, ones, sum, false);
  sum = __builtin_amdgcn_fdot2_f32_bf16(p1, ones, sum, false);
  sum = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, sum, false);
  sum = __builtin_amdgcn_fdot2_f32_bf16(p3, ones, sum, false);
  return __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                 __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

// acc + the sum of the eight bf16 values (v_dot2_f32_bf16 of each pair against (1, 1)).
// The pairs are taken with shufflevector: extracting them through an integer bitcast of the
// vector has been seen to make the compiler feed the same register to every dot2.
__device__ __forceinline__ float sum_bf16x8(const bf16x8& x, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), ones, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), ones, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), ones, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), ones, acc, false);
  return acc;
}

__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3,
                                              float a4, float a5, float a6, float a7) {
  const bf16x2 p0 = cvt_bf16x2(a0, a1), p1 = cvt_bf16x2(a2, a3);
  const bf16x2 p2 = cvt_bf16x2(a4, a5), p3 = cvt_bf16x2(a6, a7);
  return __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                 __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Transposing 8-byte LDS read (see the layout note at the top of this file).
__device__ __forceinline__ i16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_u16*)p);
}

__device__ __forceinline__ bf16x8 join_tr(const i16x4& lo, const i16x4& hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, x);
}

typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over `bytes` bytes at `base` (raw addressing, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// One wave-wide copy of 16 bytes per lane from a buffer into LDS (buffer_load_dwordx4 with
// the LDS destination): lane i's bytes land at lds_wave_base + 16*i. The lane reads at byte
// offset `off` of the buffer; offsets at or past the buffer's size read as zero.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t src, unsigned off, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void*)lds_wave_base, 16, off, 0, 0, 0);
}

}  // namespace fa
