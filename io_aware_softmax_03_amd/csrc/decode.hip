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
//
// Grouped-query caches (Hkv < H key-value heads, query heads in Hkv consecutive groups of
// g = H / Hkv; "Using it, the real way"): kernel 1 is replaced by a matrix-core kernel in
// which one wave serves all g query heads of a key-value head (up to 16 per wave), so each
// cached key and value is read from memory once per group instead of once per query head.
// Per 32-key tile: S^T = K Q^T (16 keys x 16 query heads per v_mfma_f32_16x16x32_bf16, K
// straight from memory into the A operand), online softmax per query head, then
// O^T += V^T P^T with P^T taken from the score registers and V^T read from an LDS copy of
// the tile by the transposing LDS read. The combine kernel is shared.
#include "fa_device.hpp"
#include "fa_launch.hpp"

#include <mutex>

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

struct GqaArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* part_m;
  float* part_l;
  float* part_o;
  int heads, kv_heads, group, nhb;  // nhb: blocks of up to 16 query heads per group
  int cache_len, num_splits, chunk;
  float scale_log2;
  const int* block_table;  // paged cache only
  const int* seqlens;
  int page_shift, num_pages, max_pages;
};

// Chunk (16-byte) swizzle of the LDS copy of a V tile: the transposing read takes 8 rows x
// 32 bytes per half wave; the XOR puts those 8 rows on distinct 32-byte bank groups.
template <int D>
__device__ __forceinline__ int swz_vt(int row) {
  return D == 128 ? ((row & 7) << 1) : (((row >> 1) & 3) << 1);
}

// One wave per (batch, key-value head, block of up to 16 query heads of its group, split).
// Lane l: r = l % 16, G = l / 16. Layouts (v_mfma_f32_16x16x32_bf16, see fa_device.hpp):
//   S^T = K Q^T:  A = K rows (key 16*kh + r, dims 32*ks + 8G ..+7), B = Q^T (query head r,
//                 same dims), C: lane holds S^T[key 16*kh + 4G + i][query head r].
//   O^T += V^T P^T: k-slot 8G + j of the MFMA is key 4G + j (j < 4) or 16 + 4G + j - 4, so
//                 B = P^T is the lane's own eight probabilities and A = V^T comes from two
//                 transposing reads (rows 4G.., 16 + 4G..). C: lane holds
//                 O^T[dim 16*nb + 4G + i][query head r].
// Every value a lane needs for its query head's softmax lives in the lanes r, r+16, r+32,
// r+48; the running max is shared by them, the running sums are per lane until the end.
template <int D, bool PAGED>
__global__ __launch_bounds__(64) void decode_gqa_split_kernel(GqaArgs p) {
  constexpr int KS = D / 32;             // k-steps of S^T over the head dim
  constexpr int NB = D / 16;             // 16-dim blocks of O^T
  constexpr int CPR = D / 8;             // 16-byte chunks per key row
  constexpr int VL = 32 * CPR / 64;      // V chunks per lane per tile
  constexpr int kWin = 256;              // page ids staged at a time
  __shared__ __attribute__((aligned(16))) uint16_t vt[32 * D];
  __shared__ int sm_page[PAGED ? kWin : 1];

  const int w = group_id_x();
  const int c = w % p.num_splits;
  int rest = w / p.num_splits;
  const int hb = rest % p.nhb;
  rest /= p.nhb;
  const int hk = rest % p.kv_heads;
  const int b = rest / p.kv_heads;
  const int lane = thread_id_x();
  const int r = lane & 15, G = lane >> 4;

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

  // query heads h0 .. h0 + nq - 1 of this wave; lane rows r >= nq are zero padding
  const int h0 = hk * p.group + hb * 16;
  const int nq = min(16, p.group - hb * 16);
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (r < nq) x = *(const u32x4*)(p.q + ((size_t)b * p.heads + h0 + r) * D + 32 * ks + 8 * G);
    qf[ks] = __builtin_bit_cast(bf16x8, x);
  }

  const size_t rsk = (size_t)p.kv_heads * D;
  const uint16_t* __restrict__ kg = p.k + (size_t)hk * D;
  const uint16_t* __restrict__ vg = p.v + (size_t)hk * D;
  int p0 = -(1 << 30);  // first page of the staged window
  // cache row of key n (contiguous: row b*L + n; paged: through the staged page ids)
  auto row_of = [&](int n) -> size_t {
    if constexpr (PAGED)
      return ((size_t)sm_page[(n >> p.page_shift) - p0] << p.page_shift) + (n & ((1 << p.page_shift) - 1));
    else
      return (size_t)b * p.cache_len + n;
  };
  u32x4 kx[2][KS], vx[VL];
  auto load_tile = [&](int kt0) {
    if constexpr (PAGED) {
      const int last = min(kt0 + 31, kend - 1);
      if ((kt0 >> p.page_shift) < p0 || (last >> p.page_shift) - p0 >= kWin) {
        __syncthreads();  // earlier reads of the window are done
        p0 = kt0 >> p.page_shift;
        for (int i = lane; i < kWin; i += 64)
          if (p0 + i < p.max_pages)
            sm_page[i] = min(max(p.block_table[(size_t)b * p.max_pages + p0 + i], 0), p.num_pages - 1);
        __syncthreads();
      }
    }
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int n = kt0 + 16 * kh + r;
      const bool ok = n < kend;
      const size_t row = ok ? row_of(n) : 0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (ok) x = __builtin_nontemporal_load((const u32x4*)(kg + row * rsk + 32 * ks + 8 * G));
        kx[kh][ks] = x;
      }
    }
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int ci = i * 64 + lane;
      const int n = kt0 + ci / CPR;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (n < kend) x = __builtin_nontemporal_load((const u32x4*)(vg + row_of(n) * rsk + (ci % CPR) * 8));
      vx[i] = x;
    }
  };

  // per-lane LDS element offsets of the transposing reads: row 4G + r/4 (+16 for keys
  // 16..31), columns 16*nb + 4*(r%4) .. +3
  int tr_off[2][NB];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int row = 16 * kh + 4 * G + (r >> 2);
      const int col = 16 * nb + 4 * (r & 3);
      tr_off[kh][nb] = row * D + ((((col >> 3) ^ swz_vt<D>(row)) << 3) | (col & 7));
    }

  float m = -1e30f, lsum = 0.f;
  f32x4 oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (kbeg < kend) load_tile(kbeg);
  for (int kt0 = kbeg; kt0 < kend; kt0 += 32) {
    // V tile into LDS (row-major, swizzled chunks); the previous tile's transposing reads
    // have returned (their MFMAs consumed them) before these writes
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int ci = i * 64 + lane;
      const int row = ci / CPR;
      *(u32x4*)(vt + row * D + (((ci % CPR) ^ swz_vt<D>(row)) << 3)) = vx[i];
    }
    __syncthreads();  // one wave: a wait for the writes (this tile's loads have landed anyway)
    bf16x8 kc[2][KS];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kc[kh][ks] = __builtin_bit_cast(bf16x8, kx[kh][ks]);
    if (kt0 + 32 < kend) load_tile(kt0 + 32);  // next tile in flight during this one

    float s[8];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) st = mfma16(kc[kh][ks], qf[ks], st);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = kt0 + 16 * kh + 4 * G + i;
        s[4 * kh + i] = n < kend ? st[i] * p.scale_log2 : -INFINITY;
      }
    }
    float tmax = s[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, s[i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m, tmax);
    const float alpha = exp2_fast(m - m_new);
    m = m_new;
    float pv[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = exp2_fast(s[i] - m);
      ps += pv[i];
    }
    lsum = lsum * alpha + ps;
    const bf16x8 pb = pack_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      oacc[nb] *= alpha;
      const bf16x8 va = join_tr(lds_read_tr(vt + tr_off[0][nb]), lds_read_tr(vt + tr_off[1][nb]));
      oacc[nb] = mfma16(va, pb, oacc[nb]);
    }
  }

  // query head r's sum over its four lanes; write the chunk partials of the valid heads
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (r < nq) {
    const size_t pc = ((size_t)b * p.heads + h0 + r) * p.num_splits + c;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) *(f32x4*)(p.part_o + pc * D + 16 * nb + 4 * G) = oacc[nb];
    if (G == 0) {
      p.part_m[pc] = m;
      p.part_l[pc] = lsum;
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
  if (a.kv_heads == a.heads) {
    const size_t blocks = nbh * a.num_splits;
    if (blocks > 0x7fffffffu || nbh > 0x7fffffffu) return hipErrorInvalidConfiguration;
    if (a.block_table)
      hipLaunchKernelGGL((decode_split_kernel<D, true>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, s);
    else
      hipLaunchKernelGGL((decode_split_kernel<D, false>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, s);
  } else {
    GqaArgs g;
    g.q = s.q;
    g.k = s.k;
    g.v = s.v;
    g.part_m = part_m;
    g.part_l = part_l;
    g.part_o = part_o;
    g.heads = a.heads;
    g.kv_heads = a.kv_heads;
    g.group = a.heads / a.kv_heads;
    g.nhb = (g.group + 15) / 16;
    g.cache_len = a.cache_len;
    g.num_splits = a.num_splits;
    g.chunk = s.chunk;
    g.scale_log2 = s.scale_log2;
    g.block_table = a.block_table;
    g.seqlens = a.seqlens;
    g.page_shift = s.page_shift;
    g.num_pages = a.num_pages;
    g.max_pages = a.max_pages;
    const size_t blocks = (size_t)a.batch * a.kv_heads * g.nhb * a.num_splits;
    if (blocks > 0x7fffffffu || nbh > 0x7fffffffu) return hipErrorInvalidConfiguration;
    if (a.block_table)
      hipLaunchKernelGGL((decode_gqa_split_kernel<D, true>), dim3((unsigned)blocks), dim3(64), 0, stream, g);
    else
      hipLaunchKernelGGL((decode_gqa_split_kernel<D, false>), dim3((unsigned)blocks), dim3(64), 0, stream, g);
  }
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

// Scratch of fa_decode_noalloc, for callers that cannot allocate device memory: the chunk
// partials (running max, sum and d-wide output per (batch, head, split), the fa_decode
// workspace layout) live in this fixed array instead of a caller workspace. Each GPU the
// library runs on holds its own copy until the process ends. Every partial is written by
// its split kernel before the combine kernel reads it, so nothing needs clearing between
// calls; calls that overlap on one GPU share the array and race.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of `scratch` on the current device. The host-side name of the array is
// only a handle for the symbol lookup; kernels get this address.
hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_t<128>(a, stream);
  if (a.head_dim == 64) return launch_t<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
