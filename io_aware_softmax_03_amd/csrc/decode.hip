// Single-token decode against a contiguous KV cache, split over the keys (Flash-Decoding,
// "FlashAttention-2 and -3", section "Decoding needs a different split").
//
// Kernel 1 (split): one workgroup per (batch, chunk, head), head fastest so that the
// workgroups in flight together read whole [H, d] rows of the cache. Each group of D/8
// lanes owns one key at a time (16 bytes per lane), forms the score with an in-row DPP
// reduction, and keeps its own running max / sum / partial output over the keys it
// visits. The groups are merged in LDS and the chunk's (max, sum, unnormalised output)
// goes to the workspace. Bandwidth-bound: every cache byte is read exactly once, with
// non-temporal loads, eight keys in flight per lane.
// Kernel 2 (combine): per (batch, head), weights chunk c by exp(m_c - M) (its softmax
// mass relative to the largest), O = sum_c w_c o~_c / sum_c w_c l_c, LSE = M + ln sum.
//
// Paged caches ("Paged KV caches, a preview of serving"): the same kernels, except that
// key n of sequence b is read from page block_table[b][n / page_size], slot
// n % page_size, of a page pool. Each sequence has its own length and is cut into
// num_splits chunks of ceil(L_b / num_splits) keys. The page ids of a window of up to
// 256 pages are staged in LDS, so a key's address costs an LDS read; every page is still
// read as whole, coalesced [H, d] rows. Table entries and lengths are clamped to the pool
// and the table, so no input can send a read outside the buffers.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBatchKeys = 8;  // keys in flight per lane

struct SplitArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* part_m;
  float* part_l;
  float* part_o;
  int heads, cache_len, num_splits, chunk;
  float scale_log2;
  // paged cache only
  const int* block_table;
  const int* seqlens;
  int page_shift, num_pages, max_pages;
};

constexpr int kPageWindow = 256;  // page ids staged in LDS at a time

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the G consecutive lanes of a group (G = 8 or 16, groups aligned in DPP rows).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror: other quad of the 8-lane half
  if constexpr (G == 16) x += dpp<0x140>(x);  // row_mirror: other half of the row
  return x;
}

template <int D, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(SplitArgs p) {
  constexpr int CH = D / 8;             // lanes per key
  constexpr int KPP = kThreads / CH;    // keys per pass over the workgroup
  const int h = group_id_x() % p.heads;
  const int c = (group_id_x() / p.heads) % p.num_splits;
  const int b = group_id_x() / (p.heads * p.num_splits);
  int kbeg, kend;
  if constexpr (PAGED) {
    const int cap = p.max_pages << p.page_shift;
    const int len = min(max(p.seqlens[b], 0), cap);
    const int chunk = (len + p.num_splits - 1) / p.num_splits;
    kbeg = min(c * chunk, len);
    kend = min(kbeg + chunk, len);
  } else {
    kbeg = c * p.chunk;
    kend = min(kbeg + p.chunk, p.cache_len);
  }
  const int tid = thread_id_x();
  const int sub = tid % CH, grp = tid / CH;

  float qv[8];
  {
    const u32x4 x = *(const u32x4*)(p.q + ((size_t)b * p.heads + h) * D + sub * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[2 * e] = bf16_lo(x[e]) * p.scale_log2;
      qv[2 * e + 1] = bf16_hi(x[e]) * p.scale_log2;
    }
  }
  const size_t rs = (size_t)p.heads * D;
  // contiguous: row n of sequence b; paged: row page*page_size + slot of the pool
  const size_t off = PAGED ? (size_t)h * D + sub * 8 : ((size_t)b * p.cache_len * p.heads + h) * D + sub * 8;
  const uint16_t* __restrict__ kg = p.k + off;
  const uint16_t* __restrict__ vg = p.v + off;

  float m = -1e30f, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;

  __shared__ int sm_page[PAGED ? kPageWindow : 1];
  const int wkeys = PAGED ? (kPageWindow << p.page_shift) : 0;
  for (int wbeg = kbeg, wend; wbeg < kend; wbeg = wend) {
  wend = PAGED && kend - wbeg > wkeys ? wbeg + wkeys : kend;
  int p0 = 0;
  if constexpr (PAGED) {
    // stage the page ids of keys wbeg .. wend-1 (clamped into the pool)
    p0 = wbeg >> p.page_shift;
    const int np = ((wend - 1) >> p.page_shift) - p0 + 1;
    __syncthreads();
    if (tid < np) sm_page[tid] = min(max(p.block_table[(size_t)b * p.max_pages + p0 + tid], 0), p.num_pages - 1);
    __syncthreads();
  }
  for (int n0 = wbeg; n0 < wend; n0 += KPP * kBatchKeys) {
    u32x4 kx[kBatchKeys], vx[kBatchKeys];
#pragma unroll
    for (int i = 0; i < kBatchKeys; ++i) {
      const int n = n0 + i * KPP + grp;
      u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
      if (n < wend) {
        size_t row = (size_t)n;
        if constexpr (PAGED)
          row = ((size_t)sm_page[(n >> p.page_shift) - p0] << p.page_shift) + (n & ((1 << p.page_shift) - 1));
        zk = __builtin_nontemporal_load((const u32x4*)(kg + row * rs));
        zv = __builtin_nontemporal_load((const u32x4*)(vg + row * rs));
      }
      kx[i] = zk;
      vx[i] = zv;
    }
    float s[kBatchKeys];
    float mb = -INFINITY;
#pragma unroll
    for (int i = 0; i < kBatchKeys; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(qv[2 * e], bf16_lo(kx[i][e]), acc);
        acc = __builtin_fmaf(qv[2 * e + 1], bf16_hi(kx[i][e]), acc);
      }
      acc = group_sum<CH>(acc);
      const int n = n0 + i * KPP + grp;
      s[i] = n < wend ? acc : -INFINITY;
      mb = fmaxf(mb, s[i]);
    }
    const float m_new = fmaxf(m, mb);
    const float alpha = exp2_fast(m - m_new);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
    for (int i = 0; i < kBatchKeys; ++i) {
      const float pr = exp2_fast(s[i] - m_new);
      l += pr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = __builtin_fmaf(pr, bf16_lo(vx[i][e]), o[2 * e]);
        o[2 * e + 1] = __builtin_fmaf(pr, bf16_hi(vx[i][e]), o[2 * e + 1]);
      }
    }
    m = m_new;
  }
  }

  // merge the KPP key groups of the workgroup
  __shared__ float sm_m[KPP], sm_l[KPP];
  __shared__ __attribute__((aligned(16))) float sm_o[KPP * D];
  if (sub == 0) {
    sm_m[grp] = m;
    sm_l[grp] = l;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sm_o[grp * D + sub * 8 + e] = o[e];
  __syncthreads();
  if (tid < D) {
    float M = -1e30f;
    for (int g = 0; g < KPP; ++g) M = fmaxf(M, sm_m[g]);
    float L = 0.f, acc = 0.f;
    for (int g = 0; g < KPP; ++g) {
      const float wgt = exp2_fast(sm_m[g] - M);
      L += wgt * sm_l[g];
      acc += wgt * sm_o[g * D + tid];
    }
    const size_t pc = ((size_t)b * p.heads + h) * p.num_splits + c;
    p.part_o[pc * D + tid] = acc;
    if (tid == 0) {
      p.part_m[pc] = M;
      p.part_l[pc] = L;
    }
  }
}

struct CombineArgs {
  const float* part_m;
  const float* part_l;
  const float* part_o;
  uint16_t* o;
  float* lse;
  int num_splits;
};

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(CombineArgs p) {
  const size_t bh = group_id_x();
  const int d = thread_id_x();
  const float* pm = p.part_m + bh * p.num_splits;
  const float* pl = p.part_l + bh * p.num_splits;
  const float* po = p.part_o + bh * p.num_splits * D;
  float M = -1e30f;
  for (int c = 0; c < p.num_splits; ++c) M = fmaxf(M, pm[c]);
  float L = 0.f, acc = 0.f;
  for (int c = 0; c < p.num_splits; ++c) {
    const float wgt = exp2_fast(pm[c] - M);
    L += wgt * pl[c];
    acc += wgt * po[(size_t)c * D + d];
  }
  const float out = L > 0.f ? acc / L : 0.f;
  const __bf16 ob = (__bf16)out;
  p.o[bh * D + d] = __builtin_bit_cast(uint16_t, ob);
  if (d == 0 && p.lse) p.lse[bh] = L > 0.f ? (M + log2_fast(L)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const size_t nbh = (size_t)a.batch * a.heads;
  float* part_m = a.partials;
  float* part_l = part_m + nbh * a.num_splits;
  float* part_o = part_l + nbh * a.num_splits;
  SplitArgs s;
  s.q = (const uint16_t*)a.q;
  s.k = (const uint16_t*)a.k_cache;
  s.v = (const uint16_t*)a.v_cache;
  s.part_m = part_m;
  s.part_l = part_l;
  s.part_o = part_o;
  s.heads = a.heads;
  s.cache_len = a.cache_len;
  s.num_splits = a.num_splits;
  s.chunk = (a.cache_len + a.num_splits - 1) / a.num_splits;
  s.scale_log2 = a.scale * kLog2e;
  s.block_table = a.block_table;
  s.seqlens = a.seqlens;
  s.page_shift = 0;
  while ((1 << s.page_shift) < a.page_size) ++s.page_shift;
  s.num_pages = a.num_pages;
  s.max_pages = a.max_pages;
  const size_t blocks = nbh * a.num_splits;
  if (blocks > 0x7fffffffu || nbh > 0x7fffffffu) return hipErrorInvalidConfiguration;
  if (a.block_table)
    hipLaunchKernelGGL((decode_split_kernel<D, true>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, s);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, false>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CombineArgs c;
  c.part_m = part_m;
  c.part_l = part_l;
  c.part_o = part_o;
  c.o = (uint16_t*)a.o;
  c.lse = a.lse;
  c.num_splits = a.num_splits;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)nbh), dim3(D), 0, stream, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_t<128>(a, stream);
  if (a.head_dim == 64) return launch_t<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
