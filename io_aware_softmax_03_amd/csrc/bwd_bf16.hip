// Backward attention by recomputation, bf16 inputs, fp32 gradients, gfx950 MFMA.
//
// Method ("FlashAttention: IO-aware exact attention", "Tile decomposition": the backward
// recomputes tiles instead of storing P; "FlashAttention-2 and -3", "Fewer non-matmul
// FLOPs": a recomputed weight is exp(s - lse); "Parallelism over the sequence": the
// backward is parallel over key blocks, dK_j and dV_j belong to one block, dQ_i is
// accumulated with atomic additions in device memory).
//
// Kernel 1 (preprocess): D_i = sum_c dO_ic O_ic per row, LSE_i * log2(e) (and dK, dV <- 0
// when key-value heads are shared by groups of query heads). Launched only for shared
// key-value heads; otherwise kernel 3 runs first and forms D and the base-2 LSE of its own
// queries on the way (from the dO rows it loads anyway), storing them for kernel 2.
// Kernel 2 (dK, dV): one workgroup per (128-key block, batch*head); each of its 4 waves owns
// 32 keys and keeps K, V (as MFMA operands) and dK, dV (fp32 accumulators) in registers.
// It walks 32-query blocks (causal: only those that can see a key of the block); the Q and
// dO tiles go from HBM straight into LDS (buffer loads, one block ahead, double buffered):
//   S  = Q K^T            (queries x keys; one key per lane, 16 queries per lane)
//   P  = exp2(S*c - LSE2) , dP = dO V^T , dS = P * (dP - D)
//   dV += P^T dO ,  dK += dS^T Q   (P, dS straight from registers; dO, Q transposed by
//                                   the LDS transpose read)
// Kernel 3 (dQ): one workgroup per (128-query block, batch*head); each of its 4 waves owns
// 32 queries and keeps Q, dO (as MFMA operands), their base-2 LSE and D, and dQ (fp32
// accumulators) in registers. It walks 32-key blocks (causal: up to its last query), the K
// and V tiles copied into LDS one block ahead:
//   S^T = K Q^T , dP^T = V dO^T   (one query per lane, 16 keys per lane)
//   P = exp2(S*c - LSE2) , dS = P * (dP - D)
//   dQ += dS K                    (dS straight from registers, K^T by the transpose read)
// and writes each element of dQ once. The pages accumulate dQ across key blocks with atomic
// additions in device memory; on this chip those atomics took well over half of the
// backward's time, while recomputing S and dP per query block costs two more products.
// Grouped-query attention: a query head h reads K, V of key-value head h / (H / Hkv); the
// workgroup of query head h adds its dK, dV into the shared head's gradients with fp32
// atomics; with Hkv = H they are stored once.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kNW = 4;          // waves per workgroup
constexpr int kBK = 32 * kNW;   // keys per workgroup
constexpr int kBQ = 32;         // queries per step (kernel 2), keys per step (kernel 3)

struct PreArgs {
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  float* delta;  // D, then LSE * log2(e)
  float* dk;       // zeroed here when grouped (the main kernel then adds into it)
  float* dv;
  int heads, seqlen;
  long long rows;     // B * N * H
  long long rows_kv;  // B * N * Hkv rows of dK, dV to zero, or 0
};

template <int D>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(PreArgs p) {
  constexpr int CH = D / 8;
  const long long gid = (long long)group_id_x() * 256 + thread_id_x();
  const long long row = gid / CH;  // (b, n, h) row index in [B, N, H] order
  const int sub = (int)(gid % CH);
  float acc = 0.f;
  if (row < p.rows) {
    const size_t off = (size_t)row * D + sub * 8;
    const u32x4 a = *(const u32x4*)(p.o + off);
    const u32x4 g = *(const u32x4*)(p.dout + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = __builtin_fmaf(bf16_lo(a[e]), bf16_lo(g[e]), acc);
      acc = __builtin_fmaf(bf16_hi(a[e]), bf16_hi(g[e]), acc);
    }
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    if (row < p.rows_kv) {
      *(f32x4*)(p.dk + off) = z;
      *(f32x4*)(p.dk + off + 4) = z;
      *(f32x4*)(p.dv + off) = z;
      *(f32x4*)(p.dv + off + 4) = z;
    }
  }
  // sum over the CH lanes of the row (CH divides 64, rows are lane-aligned)
#pragma unroll
  for (int s = 1; s < CH; s <<= 1) acc += __shfl_xor(acc, s);
  if (row < p.rows && sub == 0) {
    const int h = (int)(row % p.heads);
    const long long bn = row / p.heads;
    const int n = (int)(bn % p.seqlen);
    const long long b = bn / p.seqlen;
    const size_t i = ((size_t)b * p.heads + h) * p.seqlen + n;
    p.delta[i] = acc;
    p.delta[(size_t)p.rows + i] = p.lse[i] * kLog2e;
  }
}

struct MainArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse;
  const float* delta;
  float* dk;
  float* dv;
  int heads, kv_heads, group, seqlen, nkb;  // query head h reads key-value head h / group
  int grid;         // workgroups launched
  long long rows;   // B * H * N: offset of the base-2 LSE in the workspace
  float scale, scale_log2;
};

// Q and dO tiles are read two ways: 16 consecutive rows at one 16-byte chunk
// (ds_read_b128, operands of S and dP) and 4 consecutive rows x 4 consecutive chunks (the
// transpose read, operands of dV and dK). XOR-ing the chunk index with this function of the
// row keeps both conflict-free: over 16 rows it takes 16 distinct values (8 for D = 64, per
// row parity), and over 4 aligned rows it differs in the chunk bits the 4 chunks do not use.
template <int D>
__device__ __forceinline__ int swz_row(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}
// c += a b on the matrix core with the accumulator in AGPRs. The file's MFMAs otherwise get
// VGPR accumulators (the scores and dP are read by the VALU); dK and dV would then take 128
// of the 256 VGPRs, and the kernel spilled to AGPRs and recomputed LDS addresses in its loop.
// The accumulator is written and read only by this chain (back-to-back accumulation into the
// same registers needs no wait states) until the guard before the epilogue; its A and B
// operands come from VGPRs written by the VALU or by LDS reads, which the compiler waits for
// as for any register input of inline assembly.
__device__ __forceinline__ void mfma32_agpr(f32x16& c, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kNW * 64, 1) void bwd_main_kernel(MainArgs p) {
  constexpr int CH = D / 8;
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  constexpr int QT = kBQ * D;                 // elements of a Q or dO tile
  constexpr int TILE_B = QT * 2;              // bytes of one Q or dO tile
  constexpr int ROWS_PER_KB = 1024 / (2 * D);
  constexpr int LOADS = TILE_B / 1024 / kNW;  // 1 KB wave-loads per tile per wave
  static_assert(TILE_B % (1024 * kNW) == 0, "tile split");

  // Q and dO tiles as separate LDS objects per buffer: each access names its buffer at
  // compile time, so a copy into one buffer does not make reads of the other wait.
  // (each Q buffer also holds its tile's base-2 LSE and D: 2 x 32 floats after the tile, so
  // that every copy target is a Q or dO buffer)
  __shared__ __attribute__((aligned(1024))) uint16_t s_q0[QT + 4 * kBQ];     // Q tiles
  __shared__ __attribute__((aligned(1024))) uint16_t s_q1[QT + 4 * kBQ];
  __shared__ __attribute__((aligned(1024))) uint16_t s_do0[QT];              // dO tiles
  __shared__ __attribute__((aligned(1024))) uint16_t s_do1[QT];

  // Work decode, XCD-aware (workgroup w runs on XCD w % 8): each XCD takes a contiguous
  // range of batch*head (so K, V, Q and dO of a head share its L2), and within it the key
  // blocks go in order of decreasing work (causal: low key blocks see the most queries),
  // all heads' first block before any head's second.
  const int total = p.grid;
  const int w = group_id_x();
  int kb, bh;
  const int nbh = total / p.nkb;
  if (total % 8 == 0 && nbh % 8 == 0) {
    const int per = nbh / 8;              // heads per XCD
    const int slot = w / 8;
    kb = slot / per;
    bh = (w % 8) * per + slot % per;
  } else {
    kb = w % p.nkb;
    bh = w / p.nkb;
  }
  const int h = bh % p.heads, b = bh / p.heads;
  const int N = p.seqlen;
  const size_t rs = (size_t)p.heads * D;        // Q, dO row stride
  const size_t base = ((size_t)b * N * p.heads + h) * D;
  const size_t rsk = (size_t)p.kv_heads * D;    // K, V, dK, dV row stride
  const size_t base_kv = ((size_t)b * N * p.kv_heads + h / p.group) * D;
  const float* dlt_g = p.delta + ((size_t)b * p.heads + h) * N;
  const float* lse_g = p.delta + (size_t)p.rows + ((size_t)b * p.heads + h) * N;  // base-2 LSE

  const int tid = thread_id_x(), wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r = lane & 31, hh = lane >> 5, nh = r >> 4, gi = lane & 15;
  const int kb0 = kb * kBK;
  const int kw = kb0 + 32 * wid;  // first key of this wave
  const int myk = kw + r;

  // K, V fragments of this wave's keys (B operands of S = Q K^T and dP = dO V^T)
  bf16x8 kf[KK], vf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
    if (myk < N) {
      xk = *(const u32x4*)(p.k + base_kv + (size_t)myk * rsk + 16 * kk + 8 * hh);
      xv = *(const u32x4*)(p.v + base_kv + (size_t)myk * rsk + 16 * kk + 8 * hh);
    }
    kf[kk] = __builtin_bit_cast(bf16x8, xk);
    vf[kk] = __builtin_bit_cast(bf16x8, xv);
  }
  f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dk_acc[db][i] = 0.f; dv_acc[db][i] = 0.f; }

  const int qstart = CAUSAL ? kb0 : 0;   // first query that can see a key of the block
  const int nsteps = (N - qstart + kBQ - 1) / kBQ;

  // ---- tile copies: wave-load `it` of this wave fills tile rows
  // (wid*LOADS + it)*ROWS_PER_KB + lane/CH at physical chunk lane%CH with the logical chunk
  // the row swizzle puts there; the buffer resource ends with the sequence, so rows past it
  // arrive as zeros (their LSE is +inf below, so their P and dS are 0).
  unsigned t_src[LOADS];
#pragma unroll
  for (int it = 0; it < LOADS; ++it) {
    const int lrow = (wid * LOADS + it) * ROWS_PER_KB + lane / CH;
    t_src[it] = (unsigned)(lrow * (int)rs + ((lane % CH) ^ swz_row<D>(lrow)) * 8) * 2u;
  }
  auto issue_tile = [&](auto bufc, int st) {
    const int q0 = qstart + st * kBQ;
    const unsigned bytes = (unsigned)(min(kBQ - 1, N - 1 - q0) * (int)rs + D) * 2u;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + base + (size_t)q0 * rs, bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.dout + base + (size_t)q0 * rs, bytes);
    uint16_t* q_dst = decltype(bufc)::value ? s_q1 : s_q0;
    uint16_t* do_dst = decltype(bufc)::value ? s_do1 : s_do0;
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int off = (wid * LOADS + it) * 1024;  // this wave-load's 1 KB slice of the tile
      copy16_to_lds(rq, t_src[it], (char*)q_dst + off);
      copy16_to_lds(rd, t_src[it], (char*)do_dst + off);
    }
    // the tile's base-2 LSE and D, 4 bytes per lane of wave 0 (rows past the end read 0: their
    // Q and dO rows are 0 too, so P = 1 there multiplies zero rows and dS = 0)
    if (wid == 0 && lane < kBQ) {
      const unsigned fb = (unsigned)min(kBQ, N - q0) * 4u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(lse_g + q0, fb), (lds_void*)(q_dst + QT), 4, 4u * lane, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(dlt_g + q0, fb), (lds_void*)(q_dst + QT + 2 * kBQ), 4, 4u * lane, 0, 0, 0);
    }
  };

  // End of a step: the tile copies of this step have landed and its LDS reads are done, then
  // the workgroup barrier.
  auto step_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("s_barrier" ::: "memory");
  };

  // Per-lane byte offsets of the LDS operand reads within a Q or dO tile, the same for every
  // tile and buffer: computed once (recomputed in the loop, they cost more VALU instructions
  // per step than the products' softmax work). Row reads (A operands of S = Q K^T and
  // dP = dO V^T): row r, chunk 2kk + hh. Transposing reads (B operands of dV += P^T dO and
  // dK += dS^T Q): k-step ks, 32-dim block db, rows 16ks + 4hh + gi/4 and 8 further.
  constexpr int NPT = 2 * DB;
  int rw_off[KK], tr_a[NPT], tr_b[NPT];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) rw_off[kk] = (r * D + (((2 * kk + hh) ^ swz_row<D>(r)) << 3)) * 2;
#pragma unroll
  for (int t = 0; t < NPT; ++t) {
    const int ks = t / DB, db = t % DB;
    const int row_a = 16 * ks + 4 * hh + (gi >> 2);
    const int row_b = row_a + 8;
    const int col = db * 32 + 16 * nh + 4 * (gi & 3);
    tr_a[t] = (row_a * D + (((col >> 3) ^ swz_row<D>(row_a)) << 3) + (col & 7)) * 2;
    tr_b[t] = (row_b * D + (((col >> 3) ^ swz_row<D>(row_b)) << 3) + (col & 7)) * 2;
  }

  // prologue: tile 0, its LSE and D
  if (nsteps > 0) issue_tile(std::integral_constant<int, 0>(), 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // step st (buffer parity B = st & 1): copies of tile st+1; S, dP, P, dS, dV, dK of tile st
  auto step = [&](auto bufc, int st) {
    constexpr int B = decltype(bufc)::value;
    using NB = std::integral_constant<int, B ^ 1>;
    const int q0 = qstart + st * kBQ;
    if (st + 1 < nsteps) issue_tile(NB(), st + 1);
    const uint16_t* sq = B ? s_q1 : s_q0;
    const uint16_t* sd = B ? s_do1 : s_do0;

    f32x16 sc, dp;  // S and dP: lane = key r, acc[4i+j] = query 8i + 4hh + j
    // the tile's base-2 LSE and D for this lane's queries, read now so they have landed by
    // the time P and dS are formed
    f32x4 l4[4], d4[4];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      l4[i4] = *(const f32x4*)((const float*)(sq + QT) + 8 * i4 + 4 * hh);
      d4[i4] = *(const f32x4*)((const float*)(sq + QT + 2 * kBQ) + 8 * i4 + 4 * hh);
    }
    {
      // Q and dO operands of k-step kk are read two k-steps ahead of their MFMAs
      bf16x8 aq[KK], ad[KK];
      auto rd = [&](int kk) {
        aq[kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)((const char*)sq + rw_off[kk]));
        ad[kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)((const char*)sd + rw_off[kk]));
      };
      rd(0);
      rd(1);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 2 < KK) rd(kk + 2);
        sc = mfma32(aq[kk], kf[kk], kk == 0 ? f32x16{} : sc);
        dp = mfma32(ad[kk], vf[kk], kk == 0 ? f32x16{} : dp);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 12, 2);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 2 < KK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 2);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    const bool edge = (CAUSAL && q0 < kw + 31) || (q0 + kBQ > N) || (kw + 32 > N);
    if (edge) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = q0 + 8 * (i >> 2) + 4 * hh + (i & 3);
        if ((CAUSAL && myk > qi) || myk >= N) sc[i] = -INFINITY;
      }
    }
    // P, dS, then dV += P^T dO, dK += dS^T Q (k-step ks: queries 16ks + 8(e/4) + 4hh + e%4),
    // laid out by hand in chunks fenced by scheduling barriers so that the VALU work of
    // k-step 1 runs beside the MFMAs of k-step 0: chunk 0 reads the operands of k-step 0 and
    // forms its P and dS; chunk db issues the two MFMAs of (k-step 0, block db), reads the
    // operands of (k-step 1, block db) and forms 8 / DB values of k-step 1; then the MFMAs
    // of k-step 1.
    f32x16 pr, ds;
    auto pds = [&](int i) {
      pr[i] = exp2_fast(__builtin_fmaf(sc[i], p.scale_log2, -l4[i >> 2][i & 3]));
      ds[i] = pr[i] * (dp[i] - d4[i >> 2][i & 3]);
    };
    auto pack_ks = [&](int ks, bf16x8& a_p, bf16x8& a_s) {
      const int o8 = 8 * ks;
      a_p = pack_bf16x8(pr[o8], pr[o8 + 1], pr[o8 + 2], pr[o8 + 3], pr[o8 + 4], pr[o8 + 5], pr[o8 + 6], pr[o8 + 7]);
      a_s = pack_bf16x8(ds[o8], ds[o8 + 1], ds[o8 + 2], ds[o8 + 3], ds[o8 + 4], ds[o8 + 5], ds[o8 + 6], ds[o8 + 7]);
    };
    {
      constexpr int NP = 2 * DB;
      bf16x8 bdo[NP], bq[NP];
      auto rd = [&](int t) {
        const char* cd = (const char*)sd;
        const char* cq = (const char*)sq;
        bdo[t] = join_tr(lds_read_tr((const uint16_t*)(cd + tr_a[t])), lds_read_tr((const uint16_t*)(cd + tr_b[t])));
        bq[t] = join_tr(lds_read_tr((const uint16_t*)(cq + tr_a[t])), lds_read_tr((const uint16_t*)(cq + tr_b[t])));
      };
      bf16x8 ap0, as0, ap1, as1;
#pragma unroll
      for (int db = 0; db < DB; ++db) rd(db);
#pragma unroll
      for (int i = 0; i < 8; ++i) pds(i);
      pack_ks(0, ap0, as0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        mfma32_agpr(dv_acc[db], ap0, bdo[db]);
        mfma32_agpr(dk_acc[db], as0, bq[db]);
        rd(DB + db);
#pragma unroll
        for (int i = 8 + db * (8 / DB); i < 8 + (db + 1) * (8 / DB); ++i) {
          pds(i);
          // pinned here: the IR optimisers would otherwise sink them to the pack below
          asm volatile("" : "+v"(pr[i]), "+v"(ds[i]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      pack_ks(1, ap1, as1);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        mfma32_agpr(dv_acc[db], ap1, bdo[DB + db]);
        mfma32_agpr(dk_acc[db], as1, bq[DB + db]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    step_sync();
  };
  int st = 0;
  for (; st + 1 < nsteps; st += 2) {
    step(std::integral_constant<int, 0>(), st);
    step(std::integral_constant<int, 1>(), st + 1);
  }
  if (st < nsteps) {
    step(std::integral_constant<int, 0>(), st);
    ++st;
  }

  // The last products' results are read only after enough wait states (the compiler cannot
  // count them for an MFMA issued from inline assembly): 24 NOP cycles, with the
  // accumulators as operands so that no read of them moves above.
#pragma unroll
  for (int db = 0; db < DB; ++db)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(dv_acc[db]), "+a"(dk_acc[db]));

  // dK = scale * dS^T Q, dV = P^T dO; lane holds [key 8i + 4hh + j][dim db*32 + r]. A key-value
  // head shared by a group of query heads sums the group's contributions (added into the
  // zeroed dK, dV); otherwise each element is written once.
  const bool grouped = p.group > 1;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kw + 8 * (i >> 2) + 4 * hh + (i & 3);
      if (key < N) {
        const size_t off = base_kv + (size_t)key * rsk + db * 32 + r;
        if (grouped) {
          atomicAdd(p.dk + off, dk_acc[db][i] * p.scale);
          atomicAdd(p.dv + off, dv_acc[db][i]);
        } else {
          p.dk[off] = dk_acc[db][i] * p.scale;
          p.dv[off] = dv_acc[db][i];
        }
      }
    }
}

struct DqArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const uint16_t* o;   // forward output (PRE only)
  const float* lse;    // natural-log LSE (PRE only)
  float* delta;        // D, then the base-2 LSE: read, or (PRE) written for kernel 2
  float* dq;
  int heads, kv_heads, group, seqlen, nqb;  // query head h reads key-value head h / group
  int grid;         // workgroups launched
  long long rows;   // B * H * N: offset of the base-2 LSE in the workspace
  float scale, scale_log2;
};

// Kernel 3: dQ of one 128-query block of one head (one workgroup, 4 waves of 32 queries).
// 216 registers per wave, so two workgroups share a CU and one wave's exponentials and
// LDS reads run beside the other's MFMAs. With PRE (key-value heads not shared) it also does
// kernel 1's work for its queries: it forms D and the base-2 LSE itself and stores them for
// kernel 2, which then runs after it, and kernel 1 is not launched.
template <int D, bool CAUSAL, bool PRE>
__global__ __launch_bounds__(kNW * 64, 2) void bwd_dq_kernel(DqArgs p) {
  constexpr int CH = D / 8;
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  constexpr int KT = kBQ * D;                 // elements of a K or V tile (32 keys)
  constexpr int TILE_B = KT * 2;
  constexpr int ROWS_PER_KB = 1024 / (2 * D);
  constexpr int LOADS = TILE_B / 1024 / kNW;  // 1 KB wave-loads per tile per wave
  static_assert(TILE_B % (1024 * kNW) == 0, "tile split");

  // K and V tiles, double buffered, each buffer its own LDS object (accesses name their
  // buffer at compile time, so a copy into one does not make reads of the other wait)
  __shared__ __attribute__((aligned(1024))) uint16_t s_k0[KT];
  __shared__ __attribute__((aligned(1024))) uint16_t s_k1[KT];
  __shared__ __attribute__((aligned(1024))) uint16_t s_v0[KT];
  __shared__ __attribute__((aligned(1024))) uint16_t s_v1[KT];

  // Work decode as in kernel 2: each XCD a contiguous range of batch*head, the query blocks
  // in order of decreasing work (causal: the last blocks see the most keys).
  const int total = p.grid;
  const int w = group_id_x();
  int qb, bh;
  const int nbh = total / p.nqb;
  if (total % 8 == 0 && nbh % 8 == 0) {
    const int per = nbh / 8;
    const int slot = w / 8;
    qb = slot / per;
    bh = (w % 8) * per + slot % per;
  } else {
    qb = w % p.nqb;
    bh = w / p.nqb;
  }
  if (CAUSAL) qb = p.nqb - 1 - qb;
  const int h = bh % p.heads, b = bh / p.heads;
  const int N = p.seqlen;
  const size_t rs = (size_t)p.heads * D;        // Q, dO, dQ row stride
  const size_t base = ((size_t)b * N * p.heads + h) * D;
  const size_t rsk = (size_t)p.kv_heads * D;    // K, V row stride
  const size_t base_kv = ((size_t)b * N * p.kv_heads + h / p.group) * D;

  const int tid = thread_id_x(), wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r = lane & 31, hh = lane >> 5, nh = r >> 4, gi = lane & 15;
  const int qw = qb * (32 * kNW) + 32 * wid;  // first query of this wave
  const int myq = qw + r;

  // Q, dO operands of this lane's query (B operands of S^T = K Q^T, dP^T = V dO^T: lane holds
  // head dims 16kk + 8hh .. +7 of query r), its base-2 LSE and D. Rows past the end are zero
  // with LSE 0 and D 0: their P is 1 against zero dP and D, so their dS is 0.
  bf16x8 qf[KK], dof[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    u32x4 xq = {0u, 0u, 0u, 0u}, xd = {0u, 0u, 0u, 0u};
    if (myq < N) {
      xq = *(const u32x4*)(p.q + base + (size_t)myq * rs + 16 * kk + 8 * hh);
      xd = *(const u32x4*)(p.dout + base + (size_t)myq * rs + 16 * kk + 8 * hh);
    }
    qf[kk] = __builtin_bit_cast(bf16x8, xq);
    dof[kk] = __builtin_bit_cast(bf16x8, xd);
  }
  float* dlt_g = p.delta + ((size_t)b * p.heads + h) * N;
  float* lse_g = p.delta + (size_t)p.rows + ((size_t)b * p.heads + h) * N;
  float lse2, dlt;
  if constexpr (PRE) {
    // D = sum_c dO_c O_c of this lane's query, added in kernel 1's order, so that both
    // launch paths give the same bits: a sum of each 8-dim chunk in order, then a binary tree
    // over the chunks (chunk index 2kk + hh: the lane holds chunks 2kk + hh, the other lane
    // half the rest, so the tree's first level pairs the two halves)
    float cs[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 xo = {0u, 0u, 0u, 0u};
      if (myq < N) xo = *(const u32x4*)(p.o + base + (size_t)myq * rs + 16 * kk + 8 * hh);
      const u32x4 xd = __builtin_bit_cast(u32x4, dof[kk]);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(bf16_lo(xo[e]), bf16_lo(xd[e]), acc);
        acc = __builtin_fmaf(bf16_hi(xo[e]), bf16_hi(xd[e]), acc);
      }
      cs[kk] = pair_sum(acc);
    }
#pragma unroll
    for (int st = 1; st < KK; st <<= 1)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        if ((kk & st) == 0 && (kk & (st - 1)) == 0) cs[kk] = cs[kk] + cs[kk + st];
    dlt = cs[0];
    lse2 = myq < N ? p.lse[((size_t)b * p.heads + h) * N + myq] * kLog2e : 0.f;
    if (hh == 0 && myq < N) {
      dlt_g[myq] = dlt;
      lse_g[myq] = lse2;
    }
  } else {
    lse2 = myq < N ? lse_g[myq] : 0.f;
    dlt = myq < N ? dlt_g[myq] : 0.f;
  }

  f32x16 dq_acc[DB];  // lane holds [query qw + 8i + 4hh + j][dim 32db + r] at [db][4i + j]
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq_acc[db][i] = 0.f;

  // key blocks of the workgroup, and of this wave (causal: up to its last query; a wave with
  // no queries computes nothing but still copies its share of every tile)
  const int kend = CAUSAL ? min(N, qb * (32 * kNW) + 32 * kNW) : N;
  const int ntiles = (kend + kBQ - 1) / kBQ;
  const int wtiles = qw >= N ? 0 : (CAUSAL ? min(ntiles, (qw + 31) / kBQ + 1) : ntiles);

  // tile copies: as kernel 2's Q and dO tiles (same 32 x D shape and row swizzle), from K and V
  unsigned t_src[LOADS];
#pragma unroll
  for (int it = 0; it < LOADS; ++it) {
    const int lrow = (wid * LOADS + it) * ROWS_PER_KB + lane / CH;
    t_src[it] = (unsigned)(lrow * (int)rsk + ((lane % CH) ^ swz_row<D>(lrow)) * 8) * 2u;
  }
  auto issue_tile = [&](auto bufc, int j) {
    const int k0 = j * kBQ;
    const unsigned bytes = (unsigned)(min(kBQ - 1, N - 1 - k0) * (int)rsk + D) * 2u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + base_kv + (size_t)k0 * rsk, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + base_kv + (size_t)k0 * rsk, bytes);
    uint16_t* dk_ = decltype(bufc)::value ? s_k1 : s_k0;
    uint16_t* dv_ = decltype(bufc)::value ? s_v1 : s_v0;
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int off = (wid * LOADS + it) * 1024;
      copy16_to_lds(rk, t_src[it], (char*)dk_ + off);
      copy16_to_lds(rv, t_src[it], (char*)dv_ + off);
    }
  };

  // Per-lane byte offsets of the LDS operand reads within a K or V tile, computed once (as in
  // kernel 2). Row reads (A operands of S^T = K Q^T, dP^T = V dO^T): row r, chunk 2kk + hh.
  // Transposing reads of K (B operand of dQ += dS K): k-step ks, 32-dim block db, rows
  // 16ks + 4hh + gi/4 and 8 further.
  constexpr int NPT = 2 * DB;
  int rw_off[KK], tr_a[NPT], tr_b[NPT];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) rw_off[kk] = (r * D + (((2 * kk + hh) ^ swz_row<D>(r)) << 3)) * 2;
#pragma unroll
  for (int t = 0; t < NPT; ++t) {
    const int ks = t / DB, db = t % DB;
    const int row_a = 16 * ks + 4 * hh + (gi >> 2);
    const int row_b = row_a + 8;
    const int col = db * 32 + 16 * nh + 4 * (gi & 3);
    tr_a[t] = (row_a * D + (((col >> 3) ^ swz_row<D>(row_a)) << 3) + (col & 7)) * 2;
    tr_b[t] = (row_b * D + (((col >> 3) ^ swz_row<D>(row_b)) << 3) + (col & 7)) * 2;
  }

  if (ntiles > 0) issue_tile(std::integral_constant<int, 0>(), 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  auto step = [&](auto bufc, int j) {
    constexpr int B = decltype(bufc)::value;
    using NB = std::integral_constant<int, B ^ 1>;
    if (j + 1 < ntiles) issue_tile(NB(), j + 1);
    if (j < wtiles) {
      const uint16_t* sk = B ? s_k1 : s_k0;
      const uint16_t* sv = B ? s_v1 : s_v0;
      f32x16 sc, dp;  // S^T, dP^T: lane = query r, acc[4i+j] = key k0 + 8i + 4hh + j
      {
        // K and V operands of k-step kk read two k-steps ahead of their MFMAs
        bf16x8 ak[KK], av[KK];
        auto rd = [&](int kk) {
          ak[kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)((const char*)sk + rw_off[kk]));
          av[kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)((const char*)sv + rw_off[kk]));
        };
        rd(0);
        rd(1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          if (kk + 2 < KK) rd(kk + 2);
          sc = mfma32(ak[kk], qf[kk], kk == 0 ? f32x16{} : sc);
          dp = mfma32(av[kk], dof[kk], kk == 0 ? f32x16{} : dp);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 3);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          if (kk + 2 < KK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 3);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 3);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      const int k0 = j * kBQ;
      if ((CAUSAL && k0 + 31 > qw) || k0 + kBQ > N) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if ((CAUSAL && key > myq) || key >= N) sc[i] = -INFINITY;
        }
      }
      // P, dS; the 8 values of k-step ks (keys 16ks + 4hh + 0..3, 16ks + 8 + 4hh + 0..3) are
      // the A operand of dQ += dS K for that k-step
      bf16x8 as[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float d8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * ks + e;
          d8[e] = exp2_fast(__builtin_fmaf(sc[i], p.scale_log2, -lse2)) * (dp[i] - dlt);
        }
        as[ks] = pack_bf16x8(d8[0], d8[1], d8[2], d8[3], d8[4], d8[5], d8[6], d8[7]);
      }
      // dQ += dS K: B operand K^T (keys in the same order as the A operand, 32 head dims of
      // block db) by the transpose read of the K tile, two operands ahead of their MFMAs
      constexpr int NP = 2 * DB;
      bf16x8 bk[NP];
      auto rdk = [&](int t) {
        const char* ck = (const char*)sk;
        bk[t] = join_tr(lds_read_tr((const uint16_t*)(ck + tr_a[t])), lds_read_tr((const uint16_t*)(ck + tr_b[t])));
      };
      rdk(0);
      rdk(1);
#pragma unroll
      for (int t = 0; t < NP; ++t) {
        if (t + 2 < NP) rdk(t + 2);
        dq_acc[t % DB] = mfma32(as[t / DB], bk[t], dq_acc[t % DB]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);  // this step's copies have landed, its LDS reads are done
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < ntiles; j += 2) {
    step(std::integral_constant<int, 0>(), j);
    step(std::integral_constant<int, 1>(), j + 1);
  }
  if (j < ntiles) step(std::integral_constant<int, 0>(), j);

  // dQ = scale * dS K, each element written once
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = qw + 8 * (i >> 2) + 4 * hh + (i & 3);
      if (q < N) p.dq[base + (size_t)q * rs + db * 32 + r] = dq_acc[db][i] * p.scale;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_main(const MainArgs& m, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL>), dim3(blocks), dim3(kNW * 64), 0, stream, m);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool PRE>
hipError_t launch_dq(const DqArgs& q, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, PRE>), dim3((unsigned)q.grid), dim3(kNW * 64), 0, stream, q);
  return hipGetLastError();
}

// Without shared key-value heads: kernel 3 (forming D and the base-2 LSE on the way), then
// kernel 2. With them: kernel 1 (which also clears dK, dV for kernel 2's atomic additions),
// kernel 2, kernel 3.
template <int D>
hipError_t launch_t(const BwdArgs& a, hipStream_t stream) {
  const bool fused = a.kv_heads == a.heads;
  const long long rows = (long long)a.batch * a.seqlen * a.heads;

  MainArgs m;
  m.q = (const uint16_t*)a.q;
  m.k = (const uint16_t*)a.k;
  m.v = (const uint16_t*)a.v;
  m.dout = (const uint16_t*)a.dout;
  m.lse = a.lse;
  m.delta = a.delta;
  m.dk = a.dk;
  m.dv = a.dv;
  m.heads = a.heads;
  m.kv_heads = a.kv_heads;
  m.group = a.heads / a.kv_heads;
  m.seqlen = a.seqlen;
  m.nkb = (a.seqlen + kBK - 1) / kBK;
  m.scale = a.scale;
  m.scale_log2 = a.scale * kLog2e;
  const long long blocks = (long long)m.nkb * a.batch * a.heads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  m.grid = (int)blocks;
  m.rows = rows;

  DqArgs q;
  q.q = m.q;
  q.k = m.k;
  q.v = m.v;
  q.dout = m.dout;
  q.o = (const uint16_t*)a.o;
  q.lse = a.lse;
  q.delta = a.delta;
  q.dq = a.dq;
  q.heads = m.heads;
  q.kv_heads = m.kv_heads;
  q.group = m.group;
  q.seqlen = m.seqlen;
  q.nqb = (a.seqlen + 32 * kNW - 1) / (32 * kNW);
  q.rows = rows;
  q.scale = m.scale;
  q.scale_log2 = m.scale_log2;
  const long long qblocks = (long long)q.nqb * a.batch * a.heads;
  if (qblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  q.grid = (int)qblocks;

  hipError_t e;
  if (fused) {
    e = a.causal ? launch_dq<D, true, true>(q, stream) : launch_dq<D, false, true>(q, stream);
    if (e != hipSuccess) return e;
    return a.causal ? launch_main<D, true>(m, (int)blocks, stream) : launch_main<D, false>(m, (int)blocks, stream);
  }

  PreArgs pre;
  pre.o = (const uint16_t*)a.o;
  pre.dout = (const uint16_t*)a.dout;
  pre.lse = a.lse;
  pre.delta = a.delta;
  pre.dk = a.dk;
  pre.dv = a.dv;
  pre.heads = a.heads;
  pre.seqlen = a.seqlen;
  pre.rows = rows;
  pre.rows_kv = (long long)a.batch * a.seqlen * a.kv_heads;
  const long long threads = pre.rows * (D / 8);
  const long long pblocks = (threads + 255) / 256;
  if (pblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_preprocess_kernel<D>), dim3((unsigned)pblocks), dim3(256), 0, stream, pre);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = a.causal ? launch_main<D, true>(m, (int)blocks, stream) : launch_main<D, false>(m, (int)blocks, stream);
  if (e != hipSuccess) return e;
  return a.causal ? launch_dq<D, true, false>(q, stream) : launch_dq<D, false, false>(q, stream);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_t<128>(a, stream);
  if (a.head_dim == 64) return launch_t<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
