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
// the source chunk that lands it at its swizzled position. Within a wave the loop is software
// pipelined: the MFMAs of the next block's scores run beside the exponentials of this one,
// and this block's P V MFMAs beside the next block's row maximum.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kBC = 64;                    // keys per streamed block
// instruction classes for __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedVmem = 0x010, kSchedDsRead = 0x100;
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
  int nqb;         // workgroups per (sequence, head): query blocks, or pairs of them if causal
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

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glob_void;

// One wave-wide global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane i's
// bytes land at lds_wave_base + 16*i. The source is a uniform tile base plus a per-lane
// 32-bit element offset.
__device__ __forceinline__ void copy16_to_lds(const uint16_t* tile_base, unsigned elem_off, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((glob_void*)(tile_base + elem_off), (lds_void*)lds_wave_base, 16, 0, 0);
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

  // Double-buffered K and V tiles, as four separate LDS objects: every access names its
  // buffer at compile time, so the compiler can tell a copy into one buffer from reads of
  // another and does not make those reads wait for the copy.
  __shared__ __attribute__((aligned(1024))) char k_lds0[TILE_B];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILE_B];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILE_B];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILE_B];

  // ---- work decode: XCD-aware remap (workgroup w runs on XCD w % 8; each XCD gets a
  // contiguous range of (batch*head, block pair)). Causal: workgroup p of a sequence takes
  // query blocks nb-1-p and p (nb blocks in the sequence), so all workgroups do the same
  // number of key blocks; non-causal: one block each.
  const int total = gridDim.x;
  const int w = blockIdx.x;
  const int logical = (total % 8 == 0) ? (w % 8) * (total / 8) + (w / 8) : w;
  const int pi = logical % p.nqb;  // p.nqb counts work items per (sequence, head)
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
  const int nb = (L + BR - 1) / BR;

  auto run_block = [&](int qb) {
    const int q0 = qb * BR;

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
    // copy key block kt of K (IS_K) or V into buffer BUF
    auto issue = [&](auto is_kc, auto bufc, int kt) {
      constexpr bool IS_K = decltype(is_kc)::value;
      constexpr int BUF = decltype(bufc)::value;
      const int k0 = kt * kBC;
      const uint16_t* t_base = (IS_K ? kg : vg) + (size_t)k0 * rs;
      char* dst = (IS_K ? (BUF ? k_lds1 : k_lds0) : (BUF ? v_lds1 : v_lds0)) + wid * LOADS * 1024;
      const int last_row = min(kBC - 1, L - 1 - k0);
  #pragma unroll
      for (int it = 0; it < LOADS; ++it) {
        int ko, vo;
        lane_src(it, last_row, ko, vo);
        copy16_to_lds(t_base, (unsigned)(IS_K ? ko : vo), dst + it * 1024);
      }
    };

    // ---- per-lane LDS operand offsets, bytes within a tile buffer
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
        v_off[db] = vrow * D * 2 + ((((col >> 3) ^ swz_v<D>(vrow)) << 3) + (col & 7)) * 2;
      }
    }
    // keep these per-block values from being hoisted out of the block loop, where they
    // would stay live across both causal passes and be spilled
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(k_off[kk]));
#pragma unroll
    for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(v_off[db]));

    float m_ref = -1e30f;  // pivot (log2 units of scaled score), shared by both wave halves
    float l_part = 0.f;    // this lane's half of the running sum of P (fp32, for the LSE)
    float lr_part = 0.f;   // the same sum over P as rounded to bf16 for the MFMA (normalises O)
    f32x16 oacc[DB];
  #pragma unroll
    for (int db = 0; db < DB; ++db)
  #pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

    const float c2 = p.scale_log2;

    // Tiles this wave computes (causal: those with a key its rows can see). All waves take
    // part in every tile's loads and barriers.
    int wtiles = 0;
    if (wave_active) wtiles = CAUSAL ? min(ntiles, min(qw + 31, L - 1) / kBC + 1) : ntiles;

    // S^T = K Q^T for one key block from the K buffer the offsets currently point at
    auto qk = [&](f32x16& s0, f32x16& s1, auto bufc) {
      const char* kb = decltype(bufc)::value ? k_lds1 : k_lds0;
  #pragma unroll
      for (int i = 0; i < 16; ++i) { s0[i] = 0.f; s1[i] = 0.f; }
      bf16x8 a0[2], a1[2];
      a0[0] = __builtin_bit_cast(bf16x8, *(const u32x4*)(kb + k_off[0]));
      a1[0] = __builtin_bit_cast(bf16x8, *(const u32x4*)(kb + k_off[0] + 32 * D * 2));
  #pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) {
          a0[(kk + 1) & 1] = __builtin_bit_cast(bf16x8, *(const u32x4*)(kb + k_off[kk + 1]));
          a1[(kk + 1) & 1] = __builtin_bit_cast(bf16x8, *(const u32x4*)(kb + k_off[kk + 1] + 32 * D * 2));
        }
        s0 = mfma32(a0[kk & 1], qf[kk], s0);
        s1 = mfma32(a1[kk & 1], qf[kk], s1);
      }
    };
    // mask a causal-diagonal or ragged block (wave-uniform test)
    auto mask = [&](f32x16& s0, f32x16& s1, int k0) {
      if ((CAUSAL && k0 + kBC - 1 > qw) || (k0 + kBC > L)) {
        const int lim = CAUSAL ? min(myq, L - 1) : L - 1;  // last visible key of this row
  #pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kl = k0 + 8 * (i >> 2) + 4 * hh + (i & 3);
          s0[i] = kl > lim ? -INFINITY : s0[i];
          s1[i] = kl + 32 > lim ? -INFINITY : s1[i];
        }
      }
    };
    // the block's row maximum (log2 units), over this lane's 32 scores and the other half's
    auto rowmax = [&](const f32x16& s0, const f32x16& s1) {
      float ma = max3(s0[0], s0[1], s1[0]), mb = max3(s1[1], s0[2], s1[2]);
  #pragma unroll
      for (int i = 3; i < 16; i += 2) {
        ma = max3(ma, s0[i], s1[i]);
        if (i + 1 < 16) mb = max3(mb, s0[i + 1], s1[i + 1]);
      }
      return pair_max(fmaxf(ma, mb)) * c2;
    };
    // move the pivot when the block maximum exceeds it by more than the threshold (rare),
    // rescaling O and both sums to the new pivot
    auto repivot = [&](bool apply, float mt) {
      if (wave_any(apply && mt > m_ref + kRescaleThreshold)) {
        const float m_new = apply ? fmaxf(m_ref, mt) : m_ref;
        const float alpha = exp2_fast(m_ref - m_new);
        l_part *= alpha;
        lr_part *= alpha;
  #pragma unroll
        for (int db = 0; db < DB; ++db)
  #pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        m_ref = m_new;
      }
    };
    // P = exp2(S*c - pivot), in place, and as four bf16x8 MFMA operands (k-step ks holds
    // score half ks/2, registers 8*(ks%2)..+7, i.e. keys 16ks + 8(e/4) + 4hh + e%4)
    auto exp_pack = [&](f32x16& s0, f32x16& s1, bf16x8* pb) {
      const float mneg = -m_ref;
      float la = 0.f, lb = 0.f;  // fp32 sum of P (for the LSE), two chains
  #pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] = exp2_fast(__builtin_fmaf(s0[i], c2, mneg));
        s1[i] = exp2_fast(__builtin_fmaf(s1[i], c2, mneg));
        la += s0[i];
        lb += s1[i];
      }
      l_part += la + lb;
  #pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f32x16& sp = (ks < 2) ? s0 : s1;
        const int o = 8 * (ks & 1);
        pb[ks] = pack_bf16x8(sp[o], sp[o + 1], sp[o + 2], sp[o + 3], sp[o + 4], sp[o + 5], sp[o + 6], sp[o + 7]);
      }
    };
    // running sum of the bf16-rounded P the MFMA used (normalises O)
    auto sums = [&](const bf16x8* pb) {
  #pragma unroll
      for (int ks = 0; ks < 4; ++ks) lr_part = sum_bf16x8(pb[ks], lr_part);
    };
    // O^T += V^T P^T from the V buffer the offsets currently point at
    auto pv = [&](const bf16x8* pb, auto bufc) {
      const char* vb = decltype(bufc)::value ? v_lds1 : v_lds0;
  #pragma unroll
      for (int ks = 0; ks < 4; ++ks)
  #pragma unroll
        for (int db = 0; db < DB; ++db) {
          const char* va = vb + v_off[db] + 16 * ks * D * 2;
          const i16x4 lo = lds_read_tr((const uint16_t*)va);
          const i16x4 hi = lds_read_tr((const uint16_t*)(va + 8 * D * 2));
          oacc[db] = mfma32(join_tr(lo, hi), pb[ks], oacc[db]);
        }
    };
    // Software pipeline, per wave: iteration j computes P(j) (VALU) while the MFMAs of
    // S(j+1) = K(j+1) Q^T run, then O += V(j) P(j) (MFMA) while S(j+1) is masked and its
    // maximum folded into the pivot (VALU). K is loaded one block ahead of V: during
    // iteration j the loads of K(j+2) and V(j+1) go to the buffers K(j) and V(j-1) left.
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using KT = std::integral_constant<bool, true>;
    using VT = std::integral_constant<bool, false>;
    issue(KT(), B0(), 0);
    issue(VT(), B0(), 0);
    if (ntiles > 1) issue(KT(), B1(), 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 sA0, sA1, sB0, sB1;
    auto edge = [&](int k0) { return (CAUSAL && k0 + kBC - 1 > qw) || (k0 + kBC > L); };
    if (wtiles > 0) {
      qk(sA0, sA1, B0());
      if (!edge(0)) repivot(true, rowmax(sA0, sA1));
    }
    __syncthreads();   // every wave is done with K(0): its buffer takes K(2)

    auto iteration = [&](auto parity, int j) {
      constexpr bool ODD = decltype(parity)::value;
      f32x16& c0 = ODD ? sB0 : sA0;  // S(j)
      f32x16& c1 = ODD ? sB1 : sA1;
      f32x16& n0 = ODD ? sA0 : sB0;  // S(j+1)
      f32x16& n1 = ODD ? sA1 : sB1;
      // iteration j reads K(j+1) from K buffer !ODD and V(j) from V buffer ODD, and refills
      // K buffer ODD with K(j+2) and V buffer !ODD with V(j+1)
      using Pc = std::integral_constant<int, ODD ? 1 : 0>;
      using Qc = std::integral_constant<int, ODD ? 0 : 1>;
      // Loads of K(j+2) and V(j+1); past the last block the last block is loaded again (its
      // buffer is free and the copy is never read), which keeps phase B free of branches.
      const int kt_next = min(j + 2, ntiles - 1), vt_next = min(j + 1, ntiles - 1);
      if (j < wtiles) {
        // a diagonal or ragged block is masked, and its pivot taken, only now
        if (edge(j * kBC)) {
          mask(c0, c1, j * kBC);
          repivot(true, rowmax(c0, c1));
        }
        // S(j+1) is formed even past this wave's last block (stale LDS, never used) so that
        // phase A and phase B each stay one basic block the scheduler can interleave
        const bool more = j + 1 < wtiles && !edge((j + 1) * kBC);
        bf16x8 pb[4];
        // phase A: 16 MFMAs of S(j+1) interleaved with the 32 exponentials, 32 FMAs, 32 adds
        // and 16 conversions of P(j)
        exp_pack(c0, c1, pb);
        qk(n0, n1, Qc());
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
  #pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedValu, 7, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // phase B: 16 MFMAs of O += V(j) P(j) interleaved with the rounded-P sum, the row
        // maximum of S(j+1) and the copies of the next K and V blocks
        issue(KT(), Pc(), kt_next);
        issue(VT(), Qc(), vt_next);
        pv(pb, Pc());
        sums(pb);
        const float mt = rowmax(n0, n1);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 1);
  #pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
          if (i % 2 == 0 && i / 2 < 2 * LOADS) __builtin_amdgcn_sched_group_barrier(kSchedVmem, 1, 1);
          __builtin_amdgcn_sched_group_barrier(kSchedValu, 5, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        repivot(more, mt);
      } else {
        issue(KT(), Pc(), kt_next);
        issue(VT(), Qc(), vt_next);
      }
      __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of K(j+2), V(j+1) have landed
      __syncthreads();
    };
    for (int j = 0; j < ntiles; j += 2) {
      iteration(std::integral_constant<bool, false>(), j);
      if (j + 1 < ntiles) iteration(std::integral_constant<bool, true>(), j + 1);
    }

    // ---- epilogue: one division, single bf16 rounding, natural-log LSE.
    // O is normalised by the sum of the weights it was accumulated with (bf16-rounded P), so
    // the output is an exact convex combination of the rounded weights; the LSE uses the
    // unrounded sum.
    if (wave_active && myq < L) {
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
  };

  // (one inlined copy of the block body: the second pass reuses its registers)
  const int heavy = CAUSAL ? nb - 1 - pi : pi;
  const int passes = CAUSAL ? (pi < heavy ? 2 : pi == heavy ? 1 : 0) : (pi < nb ? 1 : 0);
  for (int pass = 0; pass < passes; ++pass) {
    if (pass) __syncthreads();  // every wave is done with the LDS tiles of the first block
    run_block(pass ? pi : heavy);
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
  const int nqb = (a.seqlen + BR - 1) / BR;
  p.nqb = CAUSAL ? (nqb + 1) / 2 : nqb;  // causal workgroups take a pair of query blocks
  p.scale_log2 = a.scale * kLog2e;
  const long long blocks = (long long)p.nqb * a.heads * a.batch;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, CAUSAL, VARLEN>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                     stream, p);
  return hipGetLastError();
}

#ifndef FA_FWD_WAVES
#define FA_FWD_WAVES 4
#endif
template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  constexpr int NW = FA_FWD_WAVES;
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
