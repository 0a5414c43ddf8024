// Forward attention, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Method ("FlashAttention: IO-aware exact attention", "Tile decomposition" and "Online
// softmax"; "FlashAttention-2 and -3", "Fewer non-matmul FLOPs", "Parallelism over the
// sequence", "Split the queries, not the keys"):
//   * one workgroup per (query block of BR rows, batch*head); the query block stays in
//     registers while 64-key blocks of K and V stream through LDS (double buffered);
//   * each wave owns 32 whole query rows, so the running max, running sum and output
//     accumulator of a row never leave the wave;
//   * scores are computed transposed, S^T = K Q^T, so the 32 keys x 32 queries MFMA
//     output leaves one query per lane (16 scores, the other 16 in the lane 32 away) and
//     the row max / row sum are in-lane plus one swap between wave halves;
//   * O^T += V^T P^T on MFMA, with P^T taken straight from the score registers and V^T
//     read from the row-major V tile with the LDS transpose read;
//   * online softmax in base 2 on scaled scores; the pivot is only moved when a block's
//     maximum exceeds it by more than kRescaleThreshold (exact for any shared pivot,
//     "And on Blackwell"), so most blocks skip the accumulator rescale;
//   * key blocks entirely above the causal diagonal are never loaded; within a block, a
//     wave skips 32-key halves its rows cannot see.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kBC = 64;                    // keys per streamed block
constexpr float kRescaleThreshold = 8.0f;  // log2 units: P stays <= 256

struct FwdKernelArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int* cu_seqlens;
  int heads;
  int seqlen;      // dense sequence length (unused for packed)
  int total_rows;  // LSE row stride for packed, N for dense
  int nqb;         // query blocks per (sequence, head)
  float scale_log2;
};

// XOR swizzles of 16-byte chunks inside a tile row, chosen so that the MFMA operand reads
// (K: 32 rows at one chunk; V: 8 rows x 4 chunks through the transpose read) and the
// row-wise staging writes spread over all LDS banks.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? ((row & 7) << 1) : (((row >> 1) & 3) << 1);
}

template <int D, int NW, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16_kernel(FwdKernelArgs p) {
  constexpr int NT = NW * 64;
  constexpr int BR = 32 * NW;
  constexpr int CH = D / 8;               // 16-byte chunks per row
  constexpr int KK = D / 16;              // MFMA k-steps over the head dim
  constexpr int DB = D / 32;              // 32-wide output blocks over the head dim
  constexpr int TILE = kBC * D;           // elements per K or V tile
  constexpr int LOADS = kBC * CH / NT;    // 16-byte chunks per thread per tile
  static_assert(kBC * CH % NT == 0, "tile must split evenly over threads");

  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE];  // K[2], V[2]

  // ---- work decode: XCD-aware remap, heavy (late) query blocks first
  const int total = gridDim.x;
  const int w = blockIdx.x;
  const int logical = (total % 8 == 0) ? (w % 8) * (total / 8) + (w / 8) : w;
  const int qb = p.nqb - 1 - (logical % p.nqb);
  const int bh = logical / p.nqb;
  const int h = bh % p.heads;
  const int bs = bh / p.heads;
  int seq_start, L;
  if constexpr (VARLEN) {
    seq_start = p.cu_seqlens[bs];
    L = p.cu_seqlens[bs + 1] - seq_start;
  } else {
    seq_start = bs * p.seqlen;
    L = p.seqlen;
  }
  const int q0 = qb * BR;
  if (q0 >= L) return;

  const int tid = threadIdx.x;
  const int wid = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 31;
  const int hh = lane >> 5;
  const size_t rs = (size_t)p.heads * D;  // row stride in elements
  const size_t base = ((size_t)seq_start * p.heads + h) * D;
  const uint16_t* __restrict__ qg = p.q + base;
  const uint16_t* __restrict__ kg = p.k + base;
  const uint16_t* __restrict__ vg = p.v + base;

  const int qw = q0 + 32 * wid;  // first query row of this wave
  const int myq = qw + r;
  const bool wave_active = qw < L;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds Q[myq][16*kk + 8*hh .. +7]
  bf16x8 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (myq < L) x = *(const u32x4*)(qg + (size_t)myq * rs + 16 * kk + 8 * hh);
    qf[kk] = __builtin_bit_cast(bf16x8, x);
  }

  int ntiles = (L + kBC - 1) / kBC;
  if constexpr (CAUSAL) {
    const int last_q = min(q0 + BR, L) - 1;
    ntiles = min(ntiles, last_q / kBC + 1);
  }

  // ---- staging: thread t moves chunks t, t+NT, ... of each tile (16 lanes per row)
  u32x4 kreg[LOADS], vreg[LOADS];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int ci = tid + it * NT;
      const int row = ci / CH, c = ci % CH;
      const int key = kt * kBC + row;
      u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
      if (key < L) {
        zk = *(const u32x4*)(kg + (size_t)key * rs + c * 8);
        zv = *(const u32x4*)(vg + (size_t)key * rs + c * 8);
      }
      kreg[it] = zk;
      vreg[it] = zv;
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* ks = smem + buf * TILE;
    uint16_t* vs = smem + (2 + buf) * TILE;
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int ci = tid + it * NT;
      const int row = ci / CH, c = ci % CH;
      *(u32x4*)(ks + row * D + ((c ^ swz_k<D>(row)) << 3)) = kreg[it];
      *(u32x4*)(vs + row * D + ((c ^ swz_v<D>(row)) << 3)) = vreg[it];
    }
  };

  float m_ref = -1e30f;  // pivot (log2 units of scaled score), shared by both wave halves
  float l_part = 0.f;    // this lane's half of the running sum of P (fp32, for the LSE)
  float lr_part = 0.f;   // the same sum over P as rounded to bf16 for the MFMA (normalises O)
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ntiles) load_tile(kt + 1);
    const int k0 = kt * kBC;
    const bool need0 = wave_active && (!CAUSAL || k0 <= qw + 31);
    if (need0) {
      const bool need1 = !CAUSAL || (k0 + 32 <= qw + 31);
      const uint16_t* ks = smem + buf * TILE;
      const uint16_t* vs = smem + (2 + buf) * TILE;

      // S^T = K Q^T for the two 32-key halves of the block
      f32x16 s0, s1;
#pragma unroll
      for (int i = 0; i < 16; ++i) { s0[i] = 0.f; s1[i] = 0.f; }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int c = 2 * kk + hh;
        const int row0 = r, row1 = 32 + r;
        bf16x8 a0 = __builtin_bit_cast(bf16x8, *(const u32x4*)(ks + row0 * D + ((c ^ swz_k<D>(row0)) << 3)));
        s0 = mfma32(a0, qf[kk], s0);
        if (need1) {
          bf16x8 a1 = __builtin_bit_cast(bf16x8, *(const u32x4*)(ks + row1 * D + ((c ^ swz_k<D>(row1)) << 3)));
          s1 = mfma32(a1, qf[kk], s1);
        }
      }

      // masking: causal diagonal block, ragged tail, skipped half
      const bool edge = (CAUSAL && k0 + kBC - 1 > qw) || (k0 + kBC > L);
      if (edge || !need1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kl = 8 * (i >> 2) + 4 * hh + (i & 3);
          const int key0 = k0 + kl, key1 = k0 + 32 + kl;
          if ((CAUSAL && key0 > myq) || key0 >= L) s0[i] = -INFINITY;
          if (!need1 || (CAUSAL && key1 > myq) || key1 >= L) s1[i] = -INFINITY;
        }
      }

      // online softmax (base 2). Row max over this lane's 32 scores, then the other half.
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
      mx = pair_max(mx);
      const float mt = mx * p.scale_log2;
      if (wave_any(mt > m_ref + kRescaleThreshold)) {
        const float m_new = fmaxf(m_ref, mt);
        const float alpha = exp2_fast(m_ref - m_new);
        l_part *= alpha;
        lr_part *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        m_ref = m_new;
      }
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] = exp2_fast(__builtin_fmaf(s0[i], p.scale_log2, -m_ref));
        s1[i] = exp2_fast(__builtin_fmaf(s1[i], p.scale_log2, -m_ref));
        ls += s0[i] + s1[i];
      }
      l_part += ls;

      // O^T += V^T P^T. k-step ks covers block keys 16ks..16ks+15; its B operand is
      // P^T from score half ks/2, registers 8*(ks%2)..+7 (keys 16ks + 8(e/4) + 4hh + e%4).
      const int nh = r >> 4, gi = lane & 15;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks >= 2 && !need1) break;
        const f32x16& sp = (ks < 2) ? s0 : s1;
        const int o8 = 8 * (ks & 1);
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = sp[o8 + e];
        const bf16x8 pb = pack_bf16x8_sum(pv, lr_part);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int col = db * 32 + 16 * nh + 4 * (gi & 3);
          const int row_a = 16 * ks + 4 * hh + (gi >> 2);
          const int row_b = row_a + 8;
          const i16x4 lo = lds_read_tr(vs + row_a * D + (((col >> 3) ^ swz_v<D>(row_a)) << 3) + (col & 7));
          const i16x4 hi = lds_read_tr(vs + row_b * D + (((col >> 3) ^ swz_v<D>(row_b)) << 3) + (col & 7));
          oacc[db] = mfma32(join_tr(lo, hi), pb, oacc[db]);
        }
      }
    }
    if (kt + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: one division by l, single bf16 rounding, natural-log LSE
  if (!wave_active) return;
  // O is normalised by the sum of the weights it was accumulated with (bf16-rounded P), so
  // the output is an exact convex combination of the rounded weights; the LSE uses the
  // unrounded sum.
  const float l_tot = pair_sum(l_part);
  const float lr_tot = pair_sum(lr_part);
  const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
  if (myq < L) {
    uint16_t* og = p.o + base + (size_t)myq * rs;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 wv;
        wv[0] = pack_bf16x2(oacc[db][4 * i + 0] * inv, oacc[db][4 * i + 1] * inv);
        wv[1] = pack_bf16x2(oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv);
        *(u32x2*)(og + db * 32 + 8 * i + 4 * hh) = wv;
      }
    if (hh == 0) {
      const float lse = l_tot > 0.f ? (m_ref + log2_fast(l_tot)) * kLn2 : -INFINITY;
      if constexpr (VARLEN)
        p.lse[(size_t)h * p.total_rows + seq_start + myq] = lse;
      else
        p.lse[((size_t)bs * p.heads + h) * p.seqlen + myq] = lse;
    }
  }
}

template <int D, int NW, bool CAUSAL, bool VARLEN>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  constexpr int BR = 32 * NW;
  FwdKernelArgs p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.o = (uint16_t*)a.o;
  p.lse = a.lse;
  p.cu_seqlens = a.cu_seqlens;
  p.heads = a.heads;
  p.seqlen = a.seqlen;
  p.total_rows = a.total_rows;
  p.nqb = (a.seqlen + BR - 1) / BR;
  p.scale_log2 = a.scale * kLog2e;
  const long long blocks = (long long)p.nqb * a.heads * a.batch;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, CAUSAL, VARLEN>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  constexpr int NW = 4;
  const bool varlen = a.cu_seqlens != nullptr;
  if (a.causal) return varlen ? launch_t<D, NW, true, true>(a, stream) : launch_t<D, NW, true, false>(a, stream);
  return varlen ? launch_t<D, NW, false, true>(a, stream) : launch_t<D, NW, false, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  if (a.head_dim == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
