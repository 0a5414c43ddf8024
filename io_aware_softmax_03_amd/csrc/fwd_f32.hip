// Forward attention in fp32 throughout (inputs, products, softmax, output).
//
// The exact-precision path: same tiled online softmax as the bf16 kernel ("Tile
// decomposition", "Online softmax"), but the products use fp32 FMAs rather than reduced
// precision matrix cores, so results stay within fp32 rounding of the exact value.
// Each query row is owned by 8 consecutive lanes (D/8 head dims each), so a dot product is
// a short per-lane FMA chain plus a three-step butterfly; K and V blocks of 32 keys are
// staged in LDS. It takes the same general mask as the bf16 kernel (query i sees key j
// when i + lo_off <= j <= i + hi_off) and grouped key-value heads.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kKT = 32;     // keys per block
constexpr int kThreads = 256;

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  const int* cu_seqlens;
  int heads, kv_heads, group, seqlen, seqlen_k, total_rows, nqb;
  int lo_off, hi_off;  // visible keys of query i: i + lo_off <= j (and j <= i + hi_off if CAUSAL)
  float scale_log2;
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(F32Args p) {
  constexpr int TPR = 8;                 // lanes per query row
  constexpr int DPL = D / TPR;           // head dims per lane
  constexpr int RPB = kThreads / TPR;    // query rows per workgroup
  __shared__ __attribute__((aligned(16))) float ks[kKT * D];
  __shared__ __attribute__((aligned(16))) float vs[kKT * D];

  const int qb_first = p.nqb - 1 - (int)(group_id_x() % p.nqb);
  const int bh = group_id_x() / p.nqb;
  const int h = bh % p.heads, bs = bh / p.heads;
  int seq_start, seq_start_k, L, Lk;  // L: query rows, Lk: keys
  if constexpr (VARLEN) {
    // offsets clamped into the packed tensor: a sequence starts in [0, T] and ends in
    // [its start, T], so no access leaves the buffers whatever cu_seqlens holds
    seq_start = min(max(p.cu_seqlens[bs], 0), p.total_rows);
    L = min(max(p.cu_seqlens[bs + 1], seq_start), p.total_rows) - seq_start;
    seq_start_k = seq_start;
    Lk = L;
  } else {
    seq_start = bs * p.seqlen;
    L = p.seqlen;
    seq_start_k = bs * p.seqlen_k;
    Lk = p.seqlen_k;
  }
  // query blocks qb_first, qb_first + nqb, ...: a packed sequence longer than the grid was
  // sized for (max_seqlen understated) is still computed in full
  for (int qb = qb_first; qb * RPB < L; qb += p.nqb) {
  const int q0 = qb * RPB;
  const size_t rs = (size_t)p.heads * D;      // Q / O row stride
  const size_t rsk = (size_t)p.kv_heads * D;  // K / V row stride
  const size_t base = ((size_t)seq_start * p.heads + h) * D;
  const size_t base_kv = ((size_t)seq_start_k * p.kv_heads + h / p.group) * D;
  const int tid = thread_id_x();
  const int part = tid % TPR;
  const int myq = q0 + tid / TPR;
  const bool valid = myq < L;

  float qv[DPL], ov[DPL];
#pragma unroll
  for (int c = 0; c < DPL; ++c) {
    qv[c] = valid ? p.q[base + (size_t)myq * rs + part * DPL + c] : 0.f;
    ov[c] = 0.f;
  }
  float m = -1e30f, l = 0.f;

  // keys any row of the block can see: from the first row's lowest to the last row's highest
  int kv_end = Lk;
  if constexpr (CAUSAL) kv_end = min(Lk, min(q0 + RPB, L) + p.hi_off);
  const int kv_begin = max(0, q0 + p.lo_off) / kKT * kKT;
  for (int k0 = kv_begin; k0 < kv_end; k0 += kKT) {
    __syncthreads();
    for (int e = tid; e < kKT * D; e += kThreads) {
      const int row = e / D, col = e % D;
      const int key = k0 + row;
      const bool in = key < Lk;
      ks[e] = in ? p.k[base_kv + (size_t)key * rsk + col] : 0.f;
      vs[e] = in ? p.v[base_kv + (size_t)key * rsk + col] : 0.f;
    }
    __syncthreads();
    float s[kKT];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKT; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < DPL; ++c) acc = __builtin_fmaf(qv[c], ks[j * D + part * DPL + c], acc);
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) acc += __shfl_xor(acc, off);
      const int key = k0 + j;
      const bool keep = key < Lk && (!CAUSAL || key <= myq + p.hi_off) && key >= myq + p.lo_off;
      s[j] = keep ? acc * p.scale_log2 : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float m_new = fmaxf(m, mt);
    const float alpha = exp2_fast(m - m_new);
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < kKT; ++j) {
      s[j] = exp2_fast(s[j] - m_new);
      ls += s[j];
    }
    l = l * alpha + ls;
#pragma unroll
    for (int c = 0; c < DPL; ++c) {
      float acc = ov[c] * alpha;
#pragma unroll
      for (int j = 0; j < kKT; ++j) acc = __builtin_fmaf(s[j], vs[j * D + part * DPL + c], acc);
      ov[c] = acc;
    }
    m = m_new;
  }
  if (valid) {
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int c = 0; c < DPL; ++c) p.o[base + (size_t)myq * rs + part * DPL + c] = ov[c] * inv;
  if (part == 0) {
    const float lse = l > 0.f ? (m + log2_fast(l)) * kLn2 : -INFINITY;
    if constexpr (VARLEN)
      p.lse[(size_t)h * p.total_rows + seq_start + myq] = lse;
    else
      p.lse[((size_t)bs * p.heads + h) * p.seqlen + myq] = lse;
  }
  }  // valid
  }  // query blocks
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  constexpr int RPB = kThreads / 8;
  F32Args p;
  p.q = (const float*)a.q;
  p.k = (const float*)a.k;
  p.v = (const float*)a.v;
  p.o = (float*)a.o;
  p.lse = a.lse;
  p.cu_seqlens = a.cu_seqlens;
  p.heads = a.heads;
  p.kv_heads = a.kv_heads;
  p.group = a.heads / a.kv_heads;
  p.seqlen = a.seqlen;
  p.seqlen_k = a.seqlen_k;
  p.lo_off = a.lo_off;
  p.hi_off = a.hi_off;
  p.total_rows = a.total_rows;
  p.nqb = (a.seqlen + RPB - 1) / RPB;
  p.scale_log2 = a.scale * kLog2e;
  const long long blocks = (long long)p.nqb * a.heads * a.batch;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, VARLEN>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  const bool varlen = a.cu_seqlens != nullptr;
  if (a.banded) return varlen ? launch_t<D, true, true>(a, stream) : launch_t<D, true, false>(a, stream);
  return varlen ? launch_t<D, false, true>(a, stream) : launch_t<D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  if (a.head_dim == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
