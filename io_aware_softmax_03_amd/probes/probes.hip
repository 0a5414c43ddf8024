// Hardware probes for gfx950 (MI355X): the figures the kernels' design is measured against.
// Not part of the attention library: built into a separate shared library and run by
// probes/run.py, which prints the table kept with the profiles.
//
//   probe_mfma      bf16 v_mfma_f32_32x32x16 throughput: every wave keeps eight independent
//                   accumulators busy for `iters` rounds (operands in registers); the template
//                   occupancy is one or two waves per SIMD.
//   probe_mfma_exp  the same with one v_exp_f32 and four v_fma_f32 on independent values
//                   issued between consecutive MFMAs (the forward kernel's per-score work),
//                   at one wave per SIMD or with several waves sharing a SIMD.
//   probe_read      streaming read of a buffer (16 bytes per lane, grid-stride).
//   probe_copy      streaming copy between two buffers.
//   probe_xcc       the XCD (XCC id hardware register) each workgroup runs on.
// Every loop has a fixed trip count or a bound checked against the buffer size.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int OCC>
__global__ __launch_bounds__(256, OCC) void mfma_kernel(float* out, int iters, float seed) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed + 0.001f * e);
    b[e] = (__bf16)(seed - 0.002f * e);
  }
  f32x16 acc[8];
  for (int k = 0; k < 8; ++k)
    for (int i = 0; i < 16; ++i) acc[k][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
  for (int k = 0; k < 8; ++k)
    for (int i = 0; i < 16; ++i) s += acc[k][i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// NACC independent accumulators per wave: 8 at one wave per SIMD; 4 lets two or three waves
// share a SIMD (the other waves' VALU work then runs beside a wave's MFMAs)
template <int OCC, int NACC>
__global__ __launch_bounds__(256, OCC) void mfma_exp_kernel(float* out, int iters, float seed) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed + 0.001f * e);
    b[e] = (__bf16)(seed - 0.002f * e);
  }
  f32x16 acc[NACC];
  for (int k = 0; k < NACC; ++k)
    for (int i = 0; i < 16; ++i) acc[k][i] = 0.f;
  float x[NACC], y[NACC];
  for (int k = 0; k < NACC; ++k) {
    x[k] = seed * (k + 1) * 1e-3f;
    y[k] = 0.f;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < NACC; ++k) {
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
      // independent of the MFMAs: one exponential and four FMAs per MFMA
      y[k] += __builtin_amdgcn_exp2f(x[k]);
      x[k] = __builtin_fmaf(x[k], 0.999f, 1e-6f);
      x[k] = __builtin_fmaf(x[k], 1.0001f, -1e-6f);
      y[k] = __builtin_fmaf(y[k], 0.5f, x[k]);
    }
  }
  float s = 0.f;
  for (int k = 0; k < NACC; ++k) {
    s += y[k];
    for (int i = 0; i < 16; ++i) s += acc[k][i];
  }
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void read_kernel(const u32x4* src, size_t n16, unsigned* out) {
  const size_t stride = (size_t)gridDim.x * 256;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v;
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* src, u32x4* dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// XCC_ID hardware register (id 20), bits [3:0]: s_getreg encoding id | offset << 6 | (size - 1) << 11
__global__ void xcc_kernel(int* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = (int)(__builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & 15);
}

}  // namespace

extern "C" {

// grid: workgroups of 256 threads; out: grid * 256 floats. Returns a hipError_t.
int probe_mfma(float* out, int grid, int iters, int waves_per_simd, void* stream) {
  if (!out || grid <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  if (waves_per_simd == 2)
    hipLaunchKernelGGL(mfma_kernel<2>, dim3(grid), dim3(256), 0, (hipStream_t)stream, out, iters, 0.5f);
  else
    hipLaunchKernelGGL(mfma_kernel<1>, dim3(grid), dim3(256), 0, (hipStream_t)stream, out, iters, 0.5f);
  return (int)hipGetLastError();
}

// waves_per_simd 1: eight accumulators per wave; otherwise four (two or three waves per SIMD)
int probe_mfma_exp(float* out, int grid, int iters, int waves_per_simd, void* stream) {
  if (!out || grid <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  if (waves_per_simd == 1)
    hipLaunchKernelGGL((mfma_exp_kernel<1, 8>), dim3(grid), dim3(256), 0, (hipStream_t)stream, out, iters, 0.5f);
  else
    hipLaunchKernelGGL((mfma_exp_kernel<2, 4>), dim3(grid), dim3(256), 0, (hipStream_t)stream, out, iters, 0.5f);
  return (int)hipGetLastError();
}

// src: n16 16-byte elements; out: grid * 256 unsigned
int probe_read(const void* src, size_t n16, unsigned* out, int grid, void* stream) {
  if (!src || !out || grid <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, n16, out);
  return (int)hipGetLastError();
}

int probe_copy(const void* src, void* dst, size_t n16, int grid, void* stream) {
  if (!src || !dst || grid <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, (u32x4*)dst, n16);
  return (int)hipGetLastError();
}

// out: grid ints
int probe_xcc(int* out, int grid, void* stream) {
  if (!out || grid <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(xcc_kernel, dim3(grid), dim3(64), 0, (hipStream_t)stream, out);
  return (int)hipGetLastError();
}

}  // extern "C"
