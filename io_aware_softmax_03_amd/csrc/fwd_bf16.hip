// Forward attention, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Method ("FlashAttention: IO-aware exact attention", "Tile decomposition" and "Online
// softmax"; "FlashAttention-2 and -3", "Fewer non-matmul FLOPs", "Parallelism over the
// sequence", "Split the queries, not the keys"):
//   * one workgroup per (query block of 256 rows, batch*head), two waves per SIMD: for
//     d = 128 eight waves of 32 rows (one workgroup per CU), for d = 64 four waves of 64 rows
//     (two workgroups per CU, each with its own barriers); the query block stays in
//     registers while 32-key blocks of K and V stream through LDS and are shared by the
//     workgroup's waves (four buffers each: every other step copies the tiles of the next
//     pair of steps, and the workgroup synchronises once per pair; with a sliding window two
//     buffers and a barrier every step);
//   * each wave owns whole query rows, so the running max, running sum and output
//     accumulator of a row never leave the wave (NG = kQW / 32 query groups per wave, each
//     K or V operand read from LDS feeding NG MFMAs);
//   * scores are computed transposed, S^T = K Q^T, so the 32 keys x 32 queries MFMA output
//     leaves one query per lane (16 scores, the other 16 in the lane 32 away) and the row
//     max / row sum are in-lane plus one swap between wave halves;
//   * O^T += V^T P^T on MFMA, with P^T taken straight from the score registers and V^T read
//     from the row-major V tile with the LDS transpose read;
//   * online softmax in base 2 on scaled scores against a pivot that moves only when a
//     block's values exceed it by more than a threshold (exact for any shared pivot,
//     "And on Blackwell"): a wave's first block sets it from its row maximum (plus a headroom
//     of 16 in log2 units); after that no row maximum is taken, P is formed against the
//     current pivot and a lane sum above kPMax = 2^16 (rare) sends the block through a path
//     that forms its scores again, moves the pivot to their maximum (plus the headroom) and
//     rescales O and the sums;
//   * key blocks entirely above the causal diagonal are never loaded, and a wave stops at the
//     last key block its rows can see. The mask is general: query i sees key j when
//     i + lo_off <= j <= i + hi_off (bottom-right causal for Nq != Nk, sliding windows;
//     "Using it, the real way"); a query block loads only the key blocks between its first
//     row's lowest and last row's highest visible key, and with a window each wave starts
//     at its own first block;
//   * grouped-query attention: query head h reads key-value head h / (H / Hkv).
// gfx950 specifics: two waves per SIMD (256 registers each: output accumulators, Q
// operands and score tiles all in VGPRs), so one wave's exponentials and LDS reads issue
// beside the other wave's MFMAs (a lone wave issues a VALU instruction only every ~6 cycles,
// an exponential every ~12, against 32 cycles per MFMA); K and V tiles go from global memory
// straight into LDS (buffer loads with an LDS destination, lane i -> bytes 16i of a wave's
// 1 KB slice), each lane picking the source chunk that lands it at its swizzled position.
// Within a wave the loop is a three-stage software pipeline: while the MFMAs of the next
// block's scores and of the previous block's P V run, the VALU turns this block's scores
// into probabilities.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kBC = 32;       // keys per streamed block
// Waves per workgroup and query rows per wave. d = 128: eight waves of 32 rows, one
// workgroup per CU (the 32 x 128 output accumulator of a wave takes 64 of its 256
// registers). d = 64: four waves of 64 rows (two query groups per wave, so each K or V
// operand read from LDS feeds two MFMAs), two workgroups per CU; on the packed d = 64
// workload 0.40 ms against 0.51 ms for eight 32-row waves, whose barriers coupled all the
// waves of a CU.
template <int D>
struct FwdShape {
  static constexpr int NW = D == 64 ? 4 : 8;
  static constexpr int QW = D == 64 ? 64 : 32;
  static constexpr int BR = NW * QW;            // query rows per block
};
constexpr float kRescaleThreshold = 8.0f;  // log2 units, for a wave's first block: P <= 256
// Bound on P after the first block. The result is exact for any pivot; the bound only keeps
// the fp32 accumulators far from overflow (O <= 2^16 * keys * max|V|). A larger bound than
// the first block's 2^8 matters: a pivot taken from a block with few visible keys (first
// rows of a causal or windowed sequence) or on large-magnitude scores is often exceeded by 8,
// and every such block would go through the rescue path.
constexpr float kPMax = 65536.0f;
// A pivot is placed this far (log2 units) above the maximum it is taken from (a wave's first
// block, or a block sent through the rescue path): its P start at most 2^-16, so later scores
// can pass that maximum by about 16 + 16 before a block needs the rescue path again (the
// packed workload's Q x 4 heads, whose first blocks of a sequence see few keys, otherwise
// went through it often). The result is exact for any pivot; weights that matter stay far
// above the fp32 / bf16 underflow (2^-126).
constexpr float kPivotHeadroom = 16.0f;

struct FwdKernelArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int* cu_seqlens;
  int heads;
  int kv_heads;    // K and V heads; query head h reads kv head h / group
  int group;       // heads / kv_heads
  int seqlen;      // dense query sequence length (unused for packed)
  int seqlen_k;    // dense key sequence length (unused for packed: queries and keys coincide)
  // visible keys of query i: i + lo_off <= j (and j <= i + hi_off with CAUSAL), j < Lk
  int lo_off, hi_off;
  int total_rows;  // LSE row stride for packed, N for dense
  int nqb;         // workgroups per (sequence, head): query blocks, or pairs of them if causal
  int grid;        // workgroups launched
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

// x * alpha, element-wise, rounded back to bf16
__device__ __forceinline__ bf16x8 scale_bf16x8(const bf16x8& x, float alpha) {
  const u32x4 w = __builtin_bit_cast(u32x4, x);
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]) * alpha;
    f[2 * i + 1] = bf16_hi(w[i]) * alpha;
  }
  return pack_bf16x8(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]);
}

// The sequence (of n <= 64) that comes r-th in order of decreasing length, ties by index:
// lane i ranks sequence i against all others (lengths clamped into the packed tensor as the
// kernel clamps them), and the lane of rank r names it. Wave-uniform.
__device__ __forceinline__ int sequence_of_rank(const int* cu, int n, int total, int r) {
  const int i = thread_id_x() & 63;
  int len = -1;
  if (i < n) {
    const int s = min(max(cu[i], 0), total);
    len = min(max(cu[i + 1], s), total) - s;
  }
  int rank = 0;
  for (int j = 0; j < n; ++j) {
    const int lj = __builtin_amdgcn_readlane(len, j);
    rank += (lj > len || (lj == len && j < i)) ? 1 : 0;
  }
  const unsigned long long m = __builtin_amdgcn_ballot_w64(i < n && rank == r);
  return m ? (int)__builtin_ctzll(m) : r;
}

template <int D, bool CAUSAL, bool VARLEN, bool WINDOW>
// (the second bound is the minimum number of waves per SIMD: two, 256 registers each)
__global__ __launch_bounds__(FwdShape<D>::NW * 64, 2) void fwd_bf16_kernel(FwdKernelArgs p) {
  constexpr int kNW = FwdShape<D>::NW;  // waves per workgroup
  constexpr int kQW = FwdShape<D>::QW;  // query rows per wave
  constexpr int NG = kQW / 32;          // 32-row query groups per wave
  constexpr int kBR = FwdShape<D>::BR;
  constexpr int KK = D / 16;                 // MFMA k-steps over the head dim
  constexpr int DB = D / 32;                 // 32-wide output blocks over the head dim
  constexpr int KS = kBC / 16;               // MFMA k-steps over a key block
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int TILE_B = kBC * D * 2;        // bytes of one K or V tile
  constexpr int ROWS_PER_KB = 1024 / (2 * D);
  // 1 KB wave-loads per tile: LOADS per wave for the first CPW waves (the others copy nothing)
  constexpr int CPW = TILE_B / 1024 < kNW ? TILE_B / 1024 : kNW;
  constexpr int LOADS = TILE_B / 1024 / CPW;
  static_assert(TILE_B % (1024 * CPW) == 0, "tile must split evenly over the copying waves");
  static_assert(KS == 2, "the score layout below assumes 32-key blocks");
  // K and V tile buffers each: four (steps go in pairs with one barrier a pair: the even
  // step of a pair copies the four tiles the next pair reads, a step ahead of the wait for
  // them), two with a window (waves start at different blocks, so the four-buffer rotation
  // would need a run-time phase: see the loop)
  constexpr int NBUF = WINDOW ? 2 : 4;

  // K and V tiles as separate LDS objects: every access names its buffer at compile time,
  // so the compiler can tell a copy into one buffer from reads of another and does not make
  // those reads wait for the copy.
  __shared__ __attribute__((aligned(1024))) char k_lds0[TILE_B];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILE_B];
  __shared__ __attribute__((aligned(1024))) char k_lds2[NBUF == 4 ? TILE_B : 16];
  __shared__ __attribute__((aligned(1024))) char k_lds3[NBUF == 4 ? TILE_B : 16];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILE_B];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILE_B];
  __shared__ __attribute__((aligned(1024))) char v_lds2[NBUF == 4 ? TILE_B : 16];
  __shared__ __attribute__((aligned(1024))) char v_lds3[NBUF == 4 ? TILE_B : 16];
  auto kbuf = [&](auto bc) -> char* {
    constexpr int b = decltype(bc)::value % NBUF;
    return b == 0 ? k_lds0 : (b == 1 ? k_lds1 : (b == 2 ? k_lds2 : k_lds3));
  };
  auto vbuf = [&](auto bc) -> char* {
    constexpr int b = decltype(bc)::value % NBUF;
    return b == 0 ? v_lds0 : (b == 1 ? v_lds1 : (b == 2 ? v_lds2 : v_lds3));
  };
  // Workgroup barrier once this wave's copies into LDS (and, with LGKM, its LDS stores) have
  // landed. The wavefront-scope fences emit nothing; they keep the compiler from moving
  // memory accesses across the barrier.
  auto sync_copies = [](auto lgkmc) {
    constexpr int lgkm = decltype(lgkmc)::value ? 0 : 0xF00;  // lgkmcnt(0), or no LGKM wait
    __builtin_amdgcn_s_waitcnt(0x70 | lgkm);                  // vmcnt(0), no EXP wait
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  using LgkmToo = std::integral_constant<bool, true>;
  using VmOnly = std::integral_constant<bool, false>;

  // ---- work decode, XCD-aware: workgroup w runs on XCD w % 8. With a key-value head count
  // divisible by 8, XCD x takes key-value heads x, x+8, ... of every sequence with every query
  // head that reads them (all query blocks of those heads share that XCD's L2 for K and V,
  // and every XCD gets the same mix of sequence lengths); else, with a query head count
  // divisible by 8, query heads x, x+8, ...; otherwise each XCD takes a contiguous range of
  // (sequence*head, block). Causal: workgroup p of a sequence
  // takes query blocks nb-1-p and p (nb blocks in the sequence), so all workgroups of a
  // sequence do the same number of key blocks; non-causal: one block each.
  const int total = p.grid;
  const int w = group_id_x();
  int pi, h, bs;
  if (p.kv_heads % 8 == 0) {
    const int slot = w / 8, hx = p.kv_heads / 8;
    pi = slot % p.nqb;
    int rest = slot / p.nqb;
    const int j = rest % p.group;
    rest /= p.group;
    h = (w % 8 + 8 * (rest % hx)) * p.group + j;
    bs = rest / hx;
  } else if (p.heads % 8 == 0) {
    const int slot = w / 8, hx = p.heads / 8;
    pi = slot % p.nqb;
    const int rest = slot / p.nqb;
    h = w % 8 + 8 * (rest % hx);
    bs = rest / hx;
  } else {
    const int logical = (total % 8 == 0) ? (w % 8) * (total / 8) + (w / 8) : w;
    pi = logical % p.nqb;
    const int bh = logical / p.nqb;
    h = bh % p.heads;
    bs = bh / p.heads;
  }
  int seq_start, seq_start_k, L, Lk;  // L: query rows
  if constexpr (VARLEN) {
    // packed batches of up to 64 sequences go longest first: the index decoded above is a
    // rank in order of decreasing length, so the last workgroups of the launch are those of
    // the shortest sequences
    const int nseq = total / (p.nqb * p.heads);
    if (nseq <= 64) bs = sequence_of_rank(p.cu_seqlens, nseq, p.total_rows, bs);
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
  const int nb = (L + kBR - 1) / kBR;

  auto run_block = [&](int qb) {
    const int q0 = qb * kBR;

    const int tid = thread_id_x();
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int r = lane & 31;
    const int hh = lane >> 5;
    const int nh = r >> 4, gi = lane & 15;
    const int rs = p.heads * D;     // Q / O row stride in elements (< 2^31 by the host checks)
    const int rsk = p.kv_heads * D; // K / V row stride
    const size_t base = ((size_t)seq_start * p.heads + h) * D;
    const size_t base_kv = ((size_t)seq_start_k * p.kv_heads + h / p.group) * D;
    const uint16_t* __restrict__ qg = p.q + base;
    const uint16_t* __restrict__ kg = p.k + base_kv;
    const uint16_t* __restrict__ vg = p.v + base_kv;

    const int qw = q0 + kQW * wid;  // first query row of this wave
    const bool wave_active = qw < L;

    // ---- Q fragments (B operand of S^T = K Q^T): lane holds, for query group g, row
    // qw + 32g + r, dims 16kk + 8hh .. +7. Rows past the end read the last row (finite
    // values, never stored).
    bf16x8 qf[NG][KK];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const uint16_t* qrow = qg + (size_t)min(qw + 32 * g + r, L - 1) * rs + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qf[g][kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * kk));
    }
    // the Q operands are pinned here, before the block loop, so the loads are not sunk into it
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(qf[g][kk]));

    // key blocks t0 .. t0 + ntiles - 1 of this query block: from the block holding the first
    // row's lowest visible key to the one holding the last row's highest (blocks outside
    // hold no visible key and are skipped)
    const int kfirst = WINDOW ? max(0, q0 + p.lo_off) : 0;
    const int klast = CAUSAL ? min(Lk - 1, min(q0 + kBR, L) - 1 + p.hi_off) : Lk - 1;
    const int t0 = kfirst / kBC;
    const int ntiles = klast >= kfirst ? klast / kBC + 1 - t0 : 0;
    const int kb0 = t0 * kBC;
    // key blocks this wave computes (upper bound: the last one with a key its rows can see);
    // every wave takes part in all of the block's loads and barriers
    int wtiles = 0;
    if (wave_active) {
      const int wlast = CAUSAL ? min(Lk - 1, min(qw + kQW - 1, L - 1) + p.hi_off) : Lk - 1;
      wtiles = wlast >= kb0 ? min(ntiles, wlast / kBC + 1 - t0) : 0;
    }
    // first key block this wave computes (window: the one holding its first row's lowest
    // visible key); before it the wave only takes part in the loads and barriers
    int ws = 0;
    if constexpr (WINDOW) ws = min(wtiles, max(0, qw + p.lo_off) / kBC - t0);

    // ---- staging: wave-load `it` of this wave fills tile rows
    // lrow = (wid*LOADS + it) * ROWS_PER_KB + lane / CH at physical chunk lane % CH; the lane
    // fetches the logical chunk that the swizzle puts there. Each copy goes through a buffer
    // resource that ends with the sequence, so rows past the end arrive as zeros (masked
    // later); the per-lane byte offsets are the same for every tile.
    unsigned k_src[LOADS], v_src[LOADS];
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int lrow = (wid * LOADS + it) * ROWS_PER_KB + lane / CH;
      const int phys = lane % CH;
      k_src[it] = (unsigned)(lrow * rsk + (phys ^ swz_k<D>(lrow)) * 8) * 2u;
      v_src[it] = (unsigned)(lrow * rsk + (phys ^ swz_v<D>(lrow)) * 8) * 2u;
    }
    // copy key block t0 + kt of K (IS_K) or V into buffer BUF
    auto issue = [&](auto is_kc, auto bufc, int kt) {
      constexpr bool IS_K = decltype(is_kc)::value;
      const int k0 = kb0 + kt * kBC;
      const unsigned bytes = (unsigned)(min(kBC - 1, Lk - 1 - k0) * rsk + D) * 2u;
      const __amdgpu_buffer_rsrc_t src = make_rsrc((IS_K ? kg : vg) + (size_t)k0 * rsk, bytes);
      char* dst = (IS_K ? kbuf(bufc) : vbuf(bufc)) + wid * LOADS * 1024;
      if (CPW == kNW || wid < CPW) {
#pragma unroll
        for (int it = 0; it < LOADS; ++it) copy16_to_lds(src, IS_K ? k_src[it] : v_src[it], dst + it * 1024);
      }
    };

    // ---- per-lane LDS operand offsets, bytes within a tile buffer
    // K (A operand of S^T): row r, chunk 2*kk + hh.
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
    // would stay live across both causal passes
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(k_off[kk]));
#pragma unroll
    for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(v_off[db]));
#pragma unroll
    for (int it = 0; it < LOADS; ++it) asm volatile("" : "+v"(k_src[it]), "+v"(v_src[it]));

    // per query group: pivot (log2 units of scaled score, shared by both wave halves), this
    // lane's half of the running fp32 sum of P (for the LSE), and of the sum of P as rounded
    // to bf16 for the MFMA (normalises O)
    float m_ref[NG], l_part[NG], lr_part[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      m_ref[g] = -1e30f;
      l_part[g] = 0.f;
      lr_part[g] = 0.f;
    }
    // Sums of the rounded P formed on the matrix core: v_mfma_f32_16x16x32_bf16 with a 0/1
    // selector as A and a P^T operand as B. Read as a 16x16x32 B operand, the P^T register of
    // lane l is column l%16, k-block l/16; blocks 0 and 2 hold query l%16 (both wave halves),
    // blocks 1 and 3 query l%16 + 16. Selector rows 0-7 take blocks 0 and 2, rows 8-15 blocks
    // 1 and 3, so every output row is a complete 16-key sum; lane l ends up holding the sum
    // of query q16(l) = l%16 + 16*(l/32) (four equal copies).
    f32x4 lsum[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) lsum[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 sel;
    {
      const __bf16 one = (((lane >> 4) & 1) == ((lane & 15) >= 8)) ? (__bf16)1.0f : (__bf16)0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sel[e] = one;
    }
    const int lane_q16 = (lane & 15) + 16 * (lane >> 5);  // query whose sum lane holds in lsum
    f32x16 oacc[NG][DB];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[g][db][i] = 0.f;

    const float c2 = p.scale_log2;

    // score s[g][i] of a block is S^T[key k0 + 8(i/4) + 4hh + i%4][query qw + 32g + r]
    auto edge = [&](int k0) {
      return (CAUSAL && k0 + kBC - 1 > qw + p.hi_off) || (k0 + kBC > Lk) ||
             (WINDOW && k0 < qw + kQW - 1 + p.lo_off);
    };
    auto mask = [&](f32x16 (&s)[NG], int k0) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int row = qw + 32 * g + r;
        const int lim = CAUSAL ? min(row + p.hi_off, Lk - 1) : Lk - 1;  // last visible key
        const int low = row + p.lo_off;                                  // first visible key
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kl = k0 + 8 * (i >> 2) + 4 * hh + (i & 3);
          s[g][i] = (kl > lim || (WINDOW && kl < low)) ? -INFINITY : s[g][i];
        }
      }
    };
    // block row maximum of query group g (log2 units), over both wave halves
    auto rowmax = [&](const f32x16& s) {
      float ma = max3(s[0], s[1], s[2]), mb = max3(s[3], s[4], s[5]);
      ma = max3(ma, s[6], s[7]);
      mb = max3(mb, s[8], s[9]);
      ma = max3(ma, s[10], s[11]);
      mb = max3(mb, s[12], s[13]);
      ma = max3(ma, s[14], s[15]);
      return pair_max(fmaxf(ma, mb)) * c2;
    };
    // O and both sums of group g times alpha (after its pivot moved up by -log2(alpha))
    auto rescale = [&](int g, float alpha) {
      l_part[g] *= alpha;
      lr_part[g] *= alpha;
      lsum[g] *= __int_as_float(__builtin_amdgcn_ds_bpermute(4 * lane_q16, __float_as_int(alpha)));
      // one 16-register block at a time, so this rare path does not raise the kernel's
      // register count
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[g][db][i] *= alpha;
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // Before a wave's first block: move a group's pivot when the block maximum exceeds it by
    // more than the threshold, rescaling the P block not yet multiplied into O as well.
    auto repivot = [&](const float (&mt)[NG], bf16x8 (&pend)[NG][KS]) {
      bool up = false;
#pragma unroll
      for (int g = 0; g < NG; ++g) up = up || mt[g] > m_ref[g] + kRescaleThreshold;
      if (wave_any(up)) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const float m_new = fmaxf(m_ref[g], mt[g] + kPivotHeadroom);
          const float alpha = exp2_fast(m_ref[g] - m_new);
          m_ref[g] = m_new;
          rescale(g, alpha);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) pend[g][ks] = scale_bf16x8(pend[g][ks], alpha);
        }
      }
    };
    // running sums of the bf16-rounded P the MFMA uses
    auto rsums = [&](const bf16x8 (&pb)[NG][KS]) {
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) lr_part[g] = sum_bf16x8(pb[g][ks], lr_part[g]);
    };
    // S^T = K Q^T for both query groups from K buffer BUF
    auto qk = [&](f32x16 (&s)[NG], auto bufc) {
      const char* kb = kbuf(bufc);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(kb + k_off[kk]));
#pragma unroll
        for (int g = 0; g < NG; ++g) s[g] = mfma32(a, qf[g][kk], kk == 0 ? f32x16{} : s[g]);
      }
    };
    // A P block with a value above kPMax (a lane's sum of its 16 values says so, inf
    // included): the block's scores exceed the running pivot by more than the threshold,
    // which is rare. S is formed again from K in global memory (the block's LDS copy has been
    // overwritten by then), the pivot moves to the block's maximum, and the block's P (fp32
    // sums into bs, bf16 operands into pb) is redone with it; the factor O and the running sums
    // must be multiplied by goes to alpha.
    auto rescue = [&](int k0, bf16x8 (&pb)[NG][KS], float (&bs)[NG], float (&alpha)[NG]) {
      const uint16_t* krow = kg + (size_t)min(k0 + r, Lk - 1) * rsk + 8 * hh;
      // one query group at a time and one K operand at a time (scheduling barriers keep the
      // loads from being hoisted), so this path needs few registers beyond the step's own
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        f32x16 sg[1];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(krow + 16 * kk));
          sg[0] = mfma32(a, qf[g][kk], kk == 0 ? f32x16{} : sg[0]);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (edge(k0)) {
          const int row = qw + 32 * g + r;
          const int lim = CAUSAL ? min(row + p.hi_off, Lk - 1) : Lk - 1;
          const int low = row + p.lo_off;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kl = k0 + 8 * (i >> 2) + 4 * hh + (i & 3);
            sg[0][i] = (kl > lim || (WINDOW && kl < low)) ? -INFINITY : sg[0][i];
          }
        }
        const float m_new = fmaxf(m_ref[g], rowmax(sg[0]) + kPivotHeadroom);
        alpha[g] = exp2_fast(m_ref[g] - m_new);
        m_ref[g] = m_new;
        bs[g] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sg[0][i] = exp2_fast(__builtin_fmaf(sg[0][i], c2, -m_ref[g]));
          bs[g] += sg[0][i];
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          pb[g][ks] = pack_bf16x8(sg[0][8 * ks], sg[0][8 * ks + 1], sg[0][8 * ks + 2], sg[0][8 * ks + 3],
                                  sg[0][8 * ks + 4], sg[0][8 * ks + 5], sg[0][8 * ks + 6], sg[0][8 * ks + 7]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // V^T operand of k-step ks, output block db, from V buffer BUF
    auto vread = [&](auto bufc, int ks, int db) {
      const char* va = vbuf(bufc) + v_off[db] + 16 * ks * D * 2;
      return join_tr(lds_read_tr((const uint16_t*)va), lds_read_tr((const uint16_t*)(va + 8 * D * 2)));
    };
    // O^T += V^T P^T for k-step ks of both query groups
    auto pv_step = [&](const bf16x8 (&va)[DB], const bf16x8 (&pb)[NG][KS], int ks) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < NG; ++g) oacc[g][db] = mfma32(va[db], pb[g][ks], oacc[g][db]);
    };
    // the last P block of a wave, multiplied into O on its own
    auto pv_tail = [&](const bf16x8 (&pb)[NG][KS], auto bufc) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 va[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) va[db] = vread(bufc, ks, db);
        pv_step(va, pb, ks);
      }
      rsums(pb);
    };

    // Values a pipeline part produces are pinned in VGPRs at its end, so that neither the IR
    // optimisers (which would sink them past the part, next to their first use) nor the
    // register allocator (AGPRs) move them out of the part they are scheduled in.
    auto pin = [&](bf16x8 (&pb)[KS], float& a) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(pb[ks]));
      asm volatile("" : "+v"(a));
    };

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using KT = std::integral_constant<bool, true>;
    using VT = std::integral_constant<bool, false>;

    // ---- prologue: K(0), K(1) -> K buffers 0, 1 (and with four buffers K(2) -> K buffer 2,
    // V(0) -> V buffer 0: the tiles of the first pair of steps); V buffer NBUF-1 is cleared so
    // the first step's P V (a zero P block times that buffer) adds exact zeros. A block whose
    // rows see no key at all skips to the epilogue (zeros, LSE -inf).
    if (ntiles > 0) {
    issue(KT(), B0(), 0);
    issue(KT(), B1(), min(1, ntiles - 1));
    if constexpr (NBUF == 4) {
      issue(KT(), std::integral_constant<int, 2>(), min(2, ntiles - 1));
      issue(VT(), B0(), 0);
    }
    {
      char* vz = vbuf(std::integral_constant<int, NBUF - 1>());
      u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int o = tid * 16; o < TILE_B; o += kNW * 64 * 16) *(u32x4*)(vz + o) = z;
    }
    f32x16 sA[NG], sB[NG];
    bf16x8 pA[NG][KS], pB[NG][KS];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) pB[g][ks] = bf16x8{};
    sync_copies(LgkmToo());  // the first tiles and the cleared buffer are in place
    if (ws == 0 && wtiles > 0) {
      qk(sA, B0());
#pragma unroll
      for (int g = 0; g < NG; ++g) asm volatile("" : "+v"(sA[g]));
      if (edge(kb0)) mask(sA, kb0);
      float mt[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) mt[g] = rowmax(sA[g]);
      repivot(mt, pB);
    }
    sync_copies(VmOnly());  // every wave is done with K(0)

    // ---- step j (phase PH = j % 4 with four buffers, j % 2 with two; tile t lives in
    // buffer t % NBUF), for j < wtiles: computes S(j+1) = K(j+1) Q^T, P(j) from S(j), and
    // O += V(j-1) P(j-1). Four buffers: an even step j copies K(j+3), K(j+4), V(j+1), V(j+2)
    // (into the buffers of K(j-1), K(j), V(j-3), V(j-2), which every wave finished with in the
    // previous pair) and an odd step j+1 ends the pair: it waits for those copies, issued a
    // step earlier, and the workgroup synchronises; within a pair no wave writes a buffer
    // another may still read (K(j+1), K(j+2), V(j-1), V(j)). Two buffers: every step copies
    // K(j+2), V(j), waits for them and synchronises. Past the last block the copies repeat
    // the last block (into a free buffer, never read), so a step has no branches.
    //
    // The step is laid out by hand as NSLOT slots, one MFMA each (the score MFMAs first, then
    // those of P V), fenced by scheduling barriers. Each slot also carries a fixed share of
    // the VALU work on P(j) (scale-and-shift FMA, exponential, fp32 sum, bf16 packing), the
    // rounded sums of P(j-1), and LDS reads a few slots ahead of the MFMA that consumes them.
    // P(j) is formed with the current pivot; no row maximum is taken. The lane sums of P(j)
    // bound its values: when one exceeds kPMax (rare) the block is redone with a new pivot.
    constexpr int NQK = NG * KK;               // score MFMAs (all query groups)
    constexpr int NSLOT = NQK + NG * KS * DB;  // + P V MFMAs
    constexpr int NV = 16 * NG;                // probabilities of a block per lane
    constexpr int VPS = NV / NSLOT;            // probabilities per slot (1 for D=128, 2 for D=64)
    static_assert(NV % NSLOT == 0, "slot plan");
    // LDS operand reads run a few slots ahead of the MFMAs that consume them (a sweep of both
    // distances over 2..8 slots changed the headline time by less than 1%)
    constexpr int KAH = 4;                     // K operand reads, slots ahead of their MFMA
    constexpr int KR = KAH / NG + 1;           // K operands in flight (ring)
    constexpr int VAH = NG == 1 ? 4 : 6;       // V operand reads, slots ahead of their MFMA
    // slot plan (slot -1 is the preamble before the first MFMA, slot NSLOT the tail after the last)
    auto fma_slot = [](int v) { return v / VPS - 1; };
    auto exp_slot = [](int v) { return v / VPS; };
    auto add_slot = [](int v) { return v / VPS + 1 < NSLOT ? v / VPS + 1 : NSLOT; };
    auto cvt_slot = [](int q) { return (2 * q + 1) / VPS + 1 < NSLOT ? (2 * q + 1) / VPS + 1 : NSLOT; };
    // the row-sum MFMAs need no LDS operand: they fill the matrix pipe at the start of the
    // step while the first K operands are read
    auto lsum_slot = [](int k) { return -1 + 0 * k; };
    auto kread_slot = [](int kk) { return kk * NG - KAH < -1 ? -1 : kk * NG - KAH; };
    auto vread_slot = [](int ks, int db, int hf) {
      const int t = NQK + (ks * DB + db) * NG - VAH + hf;
      return t < -1 ? -1 : t;
    };

    // the copies of step j: K(j+NBUF) -> the buffer of K(j), V(j+NBUF-2) -> that of V(j-2)
    auto issue_step = [&](auto phase, int j) {
      constexpr int PH = decltype(phase)::value;
      if constexpr (NBUF == 4) {
        if constexpr ((PH & 1) == 0) {  // even steps copy the next pair's tiles
          issue(KT(), std::integral_constant<int, PH + 3>(), min(j + 3, ntiles - 1));
          issue(KT(), std::integral_constant<int, PH>(), min(j + 4, ntiles - 1));
          issue(VT(), std::integral_constant<int, PH + 1>(), min(j + 1, ntiles - 1));
          issue(VT(), std::integral_constant<int, PH + 2>(), min(j + 2, ntiles - 1));
        }
      } else {
        issue(KT(), std::integral_constant<int, PH>(), min(j + NBUF, ntiles - 1));
        issue(VT(), std::integral_constant<int, PH + NBUF - 2>(), min(j + NBUF - 2, ntiles - 1));
      }
    };
    // end of step PH: with four buffers only odd steps wait (for the pair's copies) and
    // synchronize; with two, every step
    auto end_step = [&](auto phase) {
      constexpr int PH = decltype(phase)::value;
      if constexpr (NBUF != 4 || (PH & 1) == 1) sync_copies(VmOnly());
    };

    auto step = [&](auto phase, int j) {
      constexpr int PH = decltype(phase)::value;
      constexpr bool ODD = PH & 1;
      f32x16(&c)[NG] = ODD ? sB : sA;       // S(j)
      f32x16(&n)[NG] = ODD ? sA : sB;       // S(j+1)
      bf16x8(&pc)[NG][KS] = ODD ? pB : pA;  // P(j)
      bf16x8(&pp)[NG][KS] = ODD ? pA : pB;  // P(j-1)
      const char* kb = kbuf(std::integral_constant<int, PH + 1>());         // K(j+1)
      const char* vb = vbuf(std::integral_constant<int, PH + NBUF - 1>());  // V(j-1)
      float mneg[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) mneg[g] = -m_ref[g];
      bf16x8 ka[KR];
      i16x4 vlo[KS][DB], vhi[KS][DB];
      float acc[NG][4];  // four partial fp32 sums of P(j) per query group
      bf16x2 pr[NV / 2]; // P(j) pairs: pair q holds values 2q, 2q+1 (value v = 16g + i is c[g][i])

      auto slot = [&](auto tc) {
        constexpr int t = decltype(tc)::value;
        // (plain unrolled loops: with t fixed, every condition below folds at compile time)
        // LDS reads
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          if (kread_slot(kk) == t) ka[kk % KR] = __builtin_bit_cast(bf16x8, *(const u32x4*)(kb + k_off[kk]));
#pragma unroll
        for (int x = 0; x < KS * DB * 2; ++x) {
          const int ks = x / (2 * DB), db = (x / 2) % DB, hf = x % 2;
          if (vread_slot(ks, db, hf) == t) {
            const uint16_t* a = (const uint16_t*)(vb + v_off[db] + 16 * ks * D * 2 + hf * 8 * D * 2);
            if (hf == 0) vlo[ks][db] = lds_read_tr(a);
            else vhi[ks][db] = lds_read_tr(a);
          }
        }
        // the slot's MFMA
        if constexpr (t >= 0 && t < NQK) {
          constexpr int kk = t / NG, g = t % NG;
          n[g] = mfma32(ka[kk % KR], qf[g][kk], kk == 0 ? f32x16{} : n[g]);
        } else if constexpr (t >= NQK && t < NSLOT) {
          constexpr int u = t - NQK, ks = u / (NG * DB), db = (u / NG) % DB, g = u % NG;
          oacc[g][db] = mfma32(join_tr(vlo[ks][db], vhi[ks][db]), pp[g][ks], oacc[g][db]);
        }
        // VALU work on P(j)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int g = v / 16, i = v % 16;
          if ((fma_slot(v) < -1 ? -1 : fma_slot(v)) == t) c[g][i] = __builtin_fmaf(c[g][i], c2, mneg[g]);
          if (exp_slot(v) == t) c[g][i] = exp2_fast(c[g][i]);
          if (add_slot(v) == t) acc[g][i % 4] = i < 4 ? c[g][i] : acc[g][i % 4] + c[g][i];
        }
#pragma unroll
        for (int q = 0; q < NV / 2; ++q) {
          const int g = q / 8, i = 2 * (q % 8);
          if (cvt_slot(q) == t) {
            pr[q] = cvt_bf16x2(c[g][i], c[g][i + 1]);
            asm volatile("" : "+v"(pr[q]));  // keeps the conversion in its slot
          }
        }
        // rounded sums of P(j-1) on the matrix core (one 16x16x32 MFMA per k-step and group)
#pragma unroll
        for (int k = 0; k < NG * KS; ++k)
          if (lsum_slot(k) == t) lsum[k / KS] = mfma16(sel, pp[k / KS][k % KS], lsum[k / KS]);
        // d = 128: issue priority falls in four stages as a wave moves through its step, so
        // that of the two waves of a SIMD (one workgroup) the one behind is issued first (the
        // older wave otherwise wins every tie, runs ahead and waits at the barrier while the
        // younger one issues alone). At d = 64 the two waves of a SIMD belong to different
        // workgroups and the stages made no difference.
        if constexpr (D == 128) {
          if constexpr (t == -1) __builtin_amdgcn_s_setprio(3);
          if constexpr (t == NSLOT / 4) __builtin_amdgcn_s_setprio(2);
          if constexpr (t == NSLOT / 2) __builtin_amdgcn_s_setprio(1);
          if constexpr (t == 3 * NSLOT / 4) __builtin_amdgcn_s_setprio(0);
        }
        __builtin_amdgcn_sched_barrier(0);
      };

      // preamble (slot -1): the first LDS reads, the row-sum MFMAs and the first FMAs; then
      // this step's copies into LDS (their scalar set-up runs while the reads are in flight)
      slot(std::integral_constant<int, -1>());
      issue_step(phase, j);
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, NSLOT + 1>(slot);
      // tail: this lane's sums of P(j), the bf16 operands of P(j)
      float bs[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) bs[g] = (acc[g][0] + acc[g][1]) + (acc[g][2] + acc[g][3]);
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int q = 8 * g + 4 * ks;
          pc[g][ks] = __builtin_shufflevector(__builtin_shufflevector(pr[q], pr[q + 1], 0, 1, 2, 3),
                                              __builtin_shufflevector(pr[q + 2], pr[q + 3], 0, 1, 2, 3),
                                              0, 1, 2, 3, 4, 5, 6, 7);
        }
      bool big = false;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        pin(pc[g], bs[g]);
        asm volatile("" : "+v"(lsum[g]));
        big = big || bs[g] > kPMax;
      }
      __builtin_amdgcn_sched_barrier(0);
      // (the rescale of O sits in a branch of its own: inside the rescue branch it made the
      // register allocator move output accumulators through AGPRs on every step)
      const bool over = wave_any(big);
      float alpha[NG];
      if (over) rescue(kb0 + j * kBC, pc, bs, alpha);
      // a diagonal or ragged block is masked only now
      if (j + 1 < wtiles && edge(kb0 + (j + 1) * kBC)) mask(n, kb0 + (j + 1) * kBC);
      if (over) {
#pragma unroll
        for (int g = 0; g < NG; ++g) rescale(g, alpha[g]);
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) l_part[g] += bs[g];
      end_step(phase);
    };
    // a step of a wave past its last key block: its share of the loads, and the barrier
    auto idle_step = [&](auto phase, int j) {
      issue_step(phase, j);
      end_step(phase);
    };
    // step j of a wave whose first block is j + 1 (window): that step's loads, then S(j+1),
    // formed as the prologue forms S(0); P(j) is zero
    auto pre_step = [&](auto phase, int j) {
      constexpr int PH = decltype(phase)::value;
      constexpr bool ODD = PH & 1;
      f32x16(&n)[NG] = ODD ? sA : sB;       // S(j+1), where step j+1 reads it
      bf16x8(&pz)[NG][KS] = ODD ? pB : pA;  // P(j), step j+1's previous block
      issue_step(phase, j);
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) pz[g][ks] = bf16x8{};
      qk(n, std::integral_constant<int, PH + 1>());
#pragma unroll
      for (int g = 0; g < NG; ++g) asm volatile("" : "+v"(n[g]));
      if (edge(kb0 + (j + 1) * kBC)) mask(n, kb0 + (j + 1) * kBC);
      float mt[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) mt[g] = rowmax(n[g]);
      repivot(mt, pz);
      sync_copies(VmOnly());
    };
    // Every wave runs ntiles steps (the same barriers); it computes blocks ws .. wtiles-1,
    // and the last P block of the wave is multiplied into O right after them. The main loop
    // runs a whole period of phases a pass (4 steps with four buffers, 2 with two); steps
    // whose phase is known only at run time (idle steps, the tail) dispatch on it. (A window
    // wave may start at any block: with more buffers its first steps would need such a
    // dispatch inside the loop, which made the compiler spill; windows keep two buffers and
    // the two-step loop.)
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    int j = 0;
    const bool computes = wtiles > ws;
    if constexpr (NBUF == 2) {
      if constexpr (WINDOW) {
        if (computes && ws > 0) {
          for (; j + 1 < ws; ++j) {
            if (j & 1)
              idle_step(P1(), j);
            else
              idle_step(P0(), j);
          }
          if (j & 1)
            pre_step(P1(), j);
          else
            pre_step(P0(), j);
          ++j;
          if (j & 1) {  // keep the pairs below starting on an even block
            step(P1(), j);
            ++j;
          }
        }
      }
      if (computes) {
        for (; j + 1 < wtiles; j += 2) {
          step(P0(), j);
          step(P1(), j + 1);
        }
        if (j < wtiles) {
          step(P0(), j);
          ++j;
          pv_tail(pA, P0());  // last block even: its P is in pA, its V in buffer 0
        } else {
          pv_tail(pB, P1());  // last block odd: its P is in pB, its V in buffer 1
        }
      }
      for (; j < ntiles; ++j) {
        if (j & 1)
          idle_step(P1(), j);
        else
          idle_step(P0(), j);
      }
    } else {
      using P2 = std::integral_constant<int, 2>;
      using P3 = std::integral_constant<int, 3>;
      if (computes) {
        for (; j + 3 < wtiles; j += 4) {
          step(P0(), j);
          step(P1(), j + 1);
          step(P2(), j + 2);
          step(P3(), j + 3);
        }
        if (j < wtiles) {
          step(P0(), j);
          if (++j < wtiles) {
            step(P1(), j);
            if (++j < wtiles) {
              step(P2(), j);
              ++j;
            }
          }
        }
        // the last block wtiles-1: its P is in pA (even) or pB (odd), its V in buffer
        // (wtiles-1) % 4
        switch ((wtiles - 1) % 4) {
          case 0: pv_tail(pA, P0()); break;
          case 1: pv_tail(pB, P1()); break;
          case 2: pv_tail(pA, P2()); break;
          default: pv_tail(pB, P3()); break;
        }
      }
      for (; j < ntiles; ++j) {
        switch (j % 4) {
          case 0: idle_step(P0(), j); break;
          case 1: idle_step(P1(), j); break;
          case 2: idle_step(P2(), j); break;
          default: idle_step(P3(), j); break;
        }
      }
    }
    }  // ntiles > 0

    __builtin_amdgcn_s_waitcnt(0);  // no copy into LDS outlives the block

    // ---- epilogue: one division, single bf16 rounding, natural-log LSE.
    // O is normalised by the sum of the weights it was accumulated with (bf16-rounded P), so
    // the output is an exact convex combination of the rounded weights; the LSE uses the
    // unrounded sum.
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int myq = qw + 32 * g + r;
      const float l_tot = pair_sum(l_part[g]);
      // lane r's query sum sits in lsum of lane r (r < 16) or lane r + 16 (r >= 16)
      const float lr_mf = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (r < 16 ? r : r + 16), __float_as_int(lsum[g][0])));
      const float lr_tot = pair_sum(lr_part[g]) + lr_mf;
      if (wave_active && myq < L) {
        const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
        uint16_t* og = p.o + base + (size_t)myq * rs;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            u32x2 wv;
            wv[0] = pack_bf16x2(oacc[g][db][4 * i + 0] * inv, oacc[g][db][4 * i + 1] * inv);
            wv[1] = pack_bf16x2(oacc[g][db][4 * i + 2] * inv, oacc[g][db][4 * i + 3] * inv);
            *(u32x2*)(og + db * 32 + 8 * i + 4 * hh) = wv;
          }
        if (hh == 0) {
          const float lse = l_tot > 0.f ? (m_ref[g] + log2_fast(l_tot)) * kLn2 : -INFINITY;
          if constexpr (VARLEN)
            p.lse[(size_t)h * p.total_rows + seq_start + myq] = lse;
          else
            p.lse[((size_t)bs * p.heads + h) * p.seqlen + myq] = lse;
        }
      }
    }
  };

  // Blocks of this workgroup: causal pairs (i, nb-1-i), heavy block first, or single blocks
  // i, for i = pi, pi + nqb, pi + 2 nqb, ...: the grid covers every block of a sequence of
  // up to the sized length in one round, and a longer packed sequence (max_seqlen
  // understated) is still computed in full. One inlined copy of the block body: later
  // blocks reuse its registers.
  int i = pi;
  bool second = false, first = true;
  for (;;) {
    const int hi = CAUSAL ? nb - 1 - i : i;
    if (CAUSAL ? i > hi : i >= nb) break;
    if (!first) __syncthreads();  // every wave is done with the LDS tiles of the last block
    first = false;
    run_block(second ? i : hi);
    if (CAUSAL && !second && i < hi) {
      second = true;
    } else {
      second = false;
      i += p.nqb;
    }
  }
}

template <int D, bool CAUSAL, bool VARLEN, bool WINDOW>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  FwdKernelArgs p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.o = (uint16_t*)a.o;
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
  const int nqb = (a.seqlen + FwdShape<D>::BR - 1) / FwdShape<D>::BR;
  p.nqb = CAUSAL ? (nqb + 1) / 2 : nqb;  // causal workgroups take a pair of query blocks
  p.scale_log2 = a.scale * kLog2e;
  const long long blocks = (long long)p.nqb * a.heads * a.batch;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  p.grid = (int)blocks;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, VARLEN, WINDOW>), dim3((unsigned)blocks), dim3(FwdShape<D>::NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  const bool varlen = a.cu_seqlens != nullptr;
  // a lower bound (sliding window) only for the dense layout: packed calls have none
  if (!varlen && a.lo_off != kNoLowerBound)
    return a.banded ? launch_t<D, true, false, true>(a, stream) : launch_t<D, false, false, true>(a, stream);
  if (a.banded) return varlen ? launch_t<D, true, true, false>(a, stream) : launch_t<D, true, false, false>(a, stream);
  return varlen ? launch_t<D, false, true, false>(a, stream) : launch_t<D, false, false, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  if (a.head_dim == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
