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
// gfx950 specifics: K and V tiles go from global memory straight into LDS
// (global_load_lds_dwordx4, lane i -> bytes 16i of a wave's 1 KB slice), each lane picking
// the source chunk that lands it at its swizzled position; every LDS operand address is a
// per-lane register plus an immediate, and switching buffers flips one bit of those registers.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kBC = 64;                    // keys per streamed block
constexpr float kRescaleThreshold = 8.0f;  // log2 units: P stays <= 256

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glob_void;

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

// XOR swizzles of 16-byte chunks inside a tile row. K is read 32 rows x one chunk per
// ds_read_b128 (16 lanes = 16 consecutive rows must hit distinct chunks); V is read by the
// transpose read, 8 rows x 4 chunks per instruction, 32 lanes covering 4 rows (the row's
// two low bits must move the chunk's two high bits). Both keep row-wise fills conflict-free.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

__device__ __forceinline__ void copy16_to_lds(const uint16_t* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((glob_void*)src, (lds_void*)lds_wave_base, 16, 0, 0);
}

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

template <int D, int NW, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16_kernel(FwdKernelArgs p) {
  constexpr int BR = 32 * NW;
  constexpr int CH = D / 8;                 // 16-byte chunks per row
  constexpr int KK = D / 16;                // MFMA k-steps over the head dim
  constexpr int DB = D / 32;                // 32-wide output blocks over the head dim
  constexpr int TILE_B = kBC * D * 2;       // bytes of one K or V tile
  constexpr int ROWS_PER_KB = 1024 / (2 * D);
  constexpr int LOADS = TILE_B / 1024 / NW; // 1 KB wave-loads per tile per wave
  static_assert(TILE_B % (1024 * NW) == 0, "tile must split evenly over waves");

  // [K buf0 | K buf1 | V buf0 | V buf1]
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE_B];

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
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r = lane & 31;
  const int hh = lane >> 5;
  const int nh = r >> 4, gi = lane & 15;
  const int rs = p.heads * D;  // row stride in elements (< 2^31 by the host checks)
  const size_t base = ((size_t)seq_start * p.heads + h) * D;
  const uint16_t* __restrict__ qg = p.q + base;
  const uint16_t* __restrict__ kg = p.k + base;
  const uint16_t* __restrict__ vg = p.v + base;

  const int qw = q0 + 32 * wid;  // first query row of this wave
  const int myq = qw + r;
  const bool wave_active = qw < L;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds Q[myq][16*kk + 8*hh .. +7].
  // Rows past the end read the last row (finite values, never stored).
  bf16x8 qf[KK];
  {
    const uint16_t* qrow = qg + (size_t)min(myq, L - 1) * rs + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * kk));
  }

  int ntiles = (L + kBC - 1) / kBC;
  if constexpr (CAUSAL) {
    const int last_q = min(q0 + BR, L) - 1;
    ntiles = min(ntiles, last_q / kBC + 1);
  }

  // ---- staging: wave-load `it` of this wave fills tile rows
  // lrow = (wid*LOADS + it) * ROWS_PER_KB + lane / CH at physical chunk lane % CH; the lane
  // fetches the logical chunk that the swizzle puts there. Sources are a uniform tile base
  // plus a 32-bit per-lane offset (loop invariant except in a ragged last tile, where rows
  // past the end re-read the last row; they are masked later).
  auto lane_src = [&](int it, int last_row, int& koff, int& voff) {
    const int lrow = (wid * LOADS + it) * ROWS_PER_KB + lane / CH;
    const int phys = lane % CH;
    const int row = min(lrow, last_row);
    koff = row * rs + (phys ^ swz_k<D>(lrow)) * 8;
    voff = row * rs + (phys ^ swz_v<D>(lrow)) * 8;
  };
  int k_src[LOADS], v_src[LOADS];
#pragma unroll
  for (int it = 0; it < LOADS; ++it) lane_src(it, kBC - 1, k_src[it], v_src[it]);
  auto issue_tile = [&](int kt, int buf) {
    const int k0 = kt * kBC;
    const uint16_t* kt_base = kg + (size_t)k0 * rs;
    const uint16_t* vt_base = vg + (size_t)k0 * rs;
    const bool full = k0 + kBC <= L;
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      int ko = k_src[it], vo = v_src[it];
      if (!full) lane_src(it, L - 1 - k0, ko, vo);
      char* kdst = smem + buf * TILE_B + (wid * LOADS + it) * 1024;
      char* vdst = smem + (2 + buf) * TILE_B + (wid * LOADS + it) * 1024;
      copy16_to_lds(kt_base + (unsigned)ko, kdst);
      copy16_to_lds(vt_base + (unsigned)vo, vdst);
    }
  };

  // ---- per-lane LDS operand offsets, absolute bytes into smem for buffer 0; the loop
  // flips bit log2(TILE_B) of every offset to switch buffers (buffer bases are TILE_B aligned).
  // K (A operand of S^T): row r (+32 for the second half), chunk 2*kk + hh.
  int k_off[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) k_off[kk] = r * D * 2 + (((2 * kk + hh) ^ swz_k<D>(r)) << 4);
  // V (A operand of O^T, transpose read): rows 16ks + 8t + 4hh + gi/4, columns db*32 + 16nh + 4(gi%4).
  int v_off[DB];
  {
    const int vrow = 4 * hh + (gi >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = db * 32 + 16 * nh + 4 * (gi & 3);
      v_off[db] = 2 * TILE_B + vrow * D * 2 + ((((col >> 3) ^ swz_v<D>(vrow)) << 3) + (col & 7)) * 2;
    }
  }

  float m_ref = -1e30f;  // pivot (log2 units of scaled score), shared by both wave halves
  float l_part = 0.f;    // this lane's half of the running sum of P (fp32, for the LSE)
  float lr_part = 0.f;   // the same sum over P as rounded to bf16 for the MFMA (normalises O)
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

  const float c2 = p.scale_log2;

  issue_tile(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    if (kt + 1 < ntiles) issue_tile(kt + 1, (kt + 1) & 1);
    const int k0 = kt * kBC;
    if (wave_active && (!CAUSAL || k0 <= qw + 31)) {
      // S^T = K Q^T for the two 32-key halves of the block
      f32x16 s0, s1;
#pragma unroll
      for (int i = 0; i < 16; ++i) { s0[i] = 0.f; s1[i] = 0.f; }
      // operands read two k-steps ahead of their MFMAs
      bf16x8 a0[2], a1[2];
      a0[0] = __builtin_bit_cast(bf16x8, *(const u32x4*)(smem + k_off[0]));
      a1[0] = __builtin_bit_cast(bf16x8, *(const u32x4*)(smem + k_off[0] + 32 * D * 2));
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) {
          a0[(kk + 1) & 1] = __builtin_bit_cast(bf16x8, *(const u32x4*)(smem + k_off[kk + 1]));
          a1[(kk + 1) & 1] = __builtin_bit_cast(bf16x8, *(const u32x4*)(smem + k_off[kk + 1] + 32 * D * 2));
        }
        s0 = mfma32(a0[kk & 1], qf[kk], s0);
        s1 = mfma32(a1[kk & 1], qf[kk], s1);
      }
      // causal diagonal block or ragged tail: mask (wave-uniform branch)
      if ((CAUSAL && k0 + kBC - 1 > qw) || (k0 + kBC > L)) {
        const int lim = CAUSAL ? min(myq, L - 1) : L - 1;  // last visible key of this row
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kl = k0 + 8 * (i >> 2) + 4 * hh + (i & 3);
          s0[i] = kl > lim ? -INFINITY : s0[i];
          s1[i] = kl + 32 > lim ? -INFINITY : s1[i];
        }
      }

      // row max over this lane's 32 scores (raw), then across the two wave halves
      float ma = max3(s0[0], s0[1], s1[0]), mb = max3(s1[1], s0[2], s1[2]);
#pragma unroll
      for (int i = 3; i < 16; i += 2) {
        ma = max3(ma, s0[i], s1[i]);
        if (i + 1 < 16) mb = max3(mb, s0[i + 1], s1[i + 1]);
      }
      const float mt = pair_max(fmaxf(ma, mb)) * c2;
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
      const float mneg = -m_ref;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] = exp2_fast(__builtin_fmaf(s0[i], c2, mneg));
        s1[i] = exp2_fast(__builtin_fmaf(s1[i], c2, mneg));
      }
      // tree sum of the 32 values
      float t[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) t[i] = s0[i] + s1[i];
#pragma unroll
      for (int n = 8; n >= 1; n >>= 1)
#pragma unroll
        for (int i = 0; i < n; ++i) t[i] += t[i + n];
      l_part += t[0];

      // O^T += V^T P^T. k-step ks covers block keys 16ks..16ks+15; its B operand is P^T from
      // score half ks/2, registers 8*(ks%2)..+7 (keys 16ks + 8(e/4) + 4hh + e%4).
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f32x16& sp = (ks < 2) ? s0 : s1;
        const int o8 = 8 * (ks & 1);
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = sp[o8 + e];
        const bf16x8 pb = pack_bf16x8_sum(pv, lr_part);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const char* va = smem + v_off[db] + 16 * ks * D * 2;
          const i16x4 lo = lds_read_tr((const uint16_t*)va);
          const i16x4 hi = lds_read_tr((const uint16_t*)(va + 8 * D * 2));
          oacc[db] = mfma32(join_tr(lo, hi), pb, oacc[db]);
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) k_off[kk] ^= TILE_B;
#pragma unroll
    for (int db = 0; db < DB; ++db) v_off[db] ^= TILE_B;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next tile have landed
    __syncthreads();
  }

  // ---- epilogue: one division, single bf16 rounding, natural-log LSE.
  // O is normalised by the sum of the weights it was accumulated with (bf16-rounded P), so
  // the output is an exact convex combination of the rounded weights; the LSE uses the
  // unrounded sum.
  if (!wave_active || myq >= L) return;
  const float l_tot = pair_sum(l_part);
  const float lr_tot = pair_sum(lr_part);
  const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
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
