// Backward attention by recomputation, bf16 inputs, fp32 gradients, gfx950 MFMA.
//
// Method ("FlashAttention: IO-aware exact attention", "Tile decomposition": the backward
// recomputes tiles instead of storing P; "FlashAttention-2 and -3", "Fewer non-matmul
// FLOPs": a recomputed weight is exp(s - lse); "Parallelism over the sequence": the
// backward is parallel over key blocks, dK_j and dV_j belong to one block, dQ_i is
// accumulated with atomic additions in device memory).
//
// Kernel 1 (preprocess): D_i = sum_c dO_ic O_ic per row, LSE_i * log2(e), dQ <- 0 (and
// dK, dV <- 0 when key-value heads are shared by groups of query heads).
// Kernel 2 (main): one workgroup per (128-key block, batch*head); each of its 4 waves owns
// 32 keys and keeps K, V (as MFMA operands) and dK, dV (fp32 accumulators) in registers.
// It walks 32-query blocks (causal: only those that can see a key of the block); the Q and
// dO tiles go from HBM straight into LDS (buffer loads, one block ahead, double buffered):
//   S  = Q K^T            (queries x keys; one key per lane, 16 queries per lane)
//   P  = exp2(S*c - LSE2) , dP = dO V^T , dS = P * (dP - D)
//   dV += P^T dO ,  dK += dS^T Q   (P, dS straight from registers; dO, Q transposed by
//                                   the LDS transpose read)
//   dS^T goes to LDS (double buffered); in the next step each wave forms 32 of the head dims
//   of dQ_i = dS K over all 128 keys of the block, with its MFMAs running beside the
//   exponentials of that step, and adds them into dQ with one fp32 atomic per element.
// One workgroup barrier per query block. Grouped-query attention: the workgroup of query
// head h reads K, V of key-value head h / (H / Hkv) and adds its dK, dV into the shared
// head's gradients with fp32 atomics; with Hkv = H they are stored once.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kNW = 4;          // waves per workgroup
constexpr int kBK = 32 * kNW;   // keys per workgroup
constexpr int kBQ = 32;         // queries per step
constexpr int kDsStride = 32;   // dS^T row stride in elements (64 bytes; 8-byte groups swizzled)

struct PreArgs {
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  float* delta;  // D, then LSE * log2(e)
  float* dq;
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
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *(f32x4*)(p.dq + off) = z;
    *(f32x4*)(p.dq + off + 4) = z;
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
  float* dq;
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
// dS^T element (row = key, col = query): 64-byte rows whose 8-byte groups are XOR-ed with
// (row / 4) % 8, so the row-wise writes (32 keys at one column group) and the transpose
// reads (4 consecutive keys x all 32 queries) are both conflict-free.
__device__ __forceinline__ int ds_off(int row, int col) {
  return row * kDsStride + ((((col >> 2) ^ (row >> 2)) & 7) << 2) + (col & 3);
}
template <int D>
__device__ __forceinline__ int swz_tr(int row) {   // rows read 8 at a time by the transpose read
  return D == 128 ? ((row & 7) << 1) : (((row >> 1) & 3) << 1);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kNW * 64, 1) void bwd_main_kernel(MainArgs p) {
  constexpr int NT = kNW * 64;
  constexpr int CH = D / 8;
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  constexpr int QT = kBQ * D;                 // elements of a Q or dO tile
  constexpr int TILE_B = QT * 2;              // bytes of one Q or dO tile
  constexpr int ROWS_PER_KB = 1024 / (2 * D);
  constexpr int LOADS = TILE_B / 1024 / kNW;  // 1 KB wave-loads per tile per wave
  static_assert(TILE_B % (1024 * kNW) == 0, "tile split");
  static_assert(D / 32 == kNW || D == 64, "dQ head-dim split assumes D = 32 * waves (or D = 64)");

  // Q and dO tiles as separate LDS objects per buffer: each access names its buffer at
  // compile time, so a copy into one buffer does not make reads of the other wait.
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kBK * D];            // K block (transpose reads)
  // (each Q buffer also holds its tile's base-2 LSE and D: 2 x 32 floats after the tile, so
  // that every copy target is a Q or dO buffer)
  __shared__ __attribute__((aligned(1024))) uint16_t s_q0[QT + 4 * kBQ];     // Q tiles
  __shared__ __attribute__((aligned(1024))) uint16_t s_q1[QT + 4 * kBQ];
  __shared__ __attribute__((aligned(1024))) uint16_t s_do0[QT];              // dO tiles
  __shared__ __attribute__((aligned(1024))) uint16_t s_do1[QT];
  __shared__ __attribute__((aligned(16))) uint16_t s_ds[2][kBK * kDsStride];  // dS^T [key][query]

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
  const size_t rs = (size_t)p.heads * D;        // Q, dO, dQ row stride
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
  // whole K block into LDS (row-major, read transposed for dQ = dS K)
  for (int ci = tid; ci < kBK * CH; ci += NT) {
    const int row = ci / CH, c = ci % CH;
    const int key = kb0 + row;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (key < N) x = *(const u32x4*)(p.k + base_kv + (size_t)key * rsk + c * 8);
    *(u32x4*)(s_k + row * D + ((c ^ swz_tr<D>(row)) << 3)) = x;
  }

  // The K operands of dQ = dS K for this wave's head dims are the same for every query
  // block: read them from LDS once (transpose reads), after the block is staged.
  constexpr int QCOLS = D / kNW;  // head dims of dQ per wave (32 for D = 128, 16 for D = 64)
  __syncthreads();
  bf16x8 kq[kBK / 16];
#pragma unroll
  for (int ks = 0; ks < kBK / 16; ++ks) {
    const int row_a = 16 * ks + 4 * hh + (gi >> 2);
    const int row_b = row_a + 8;
    int col = wid * QCOLS + 16 * nh + 4 * (gi & 3);
    if (QCOLS == 16) col = wid * QCOLS + 4 * (gi & 3);  // D = 64: lanes 16-31 repeat
    const int ca = (((col >> 3) ^ swz_tr<D>(row_a)) << 3) + (col & 7);
    const int cb = (((col >> 3) ^ swz_tr<D>(row_b)) << 3) + (col & 7);
    kq[ks] = join_tr(lds_read_tr(s_k + row_a * D + ca), lds_read_tr(s_k + row_b * D + cb));
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
    uint16_t* dq_ = decltype(bufc)::value ? s_q1 : s_q0;
    uint16_t* dd_ = decltype(bufc)::value ? s_do1 : s_do0;
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int off = (wid * LOADS + it) * 1024;  // this wave-load's 1 KB slice of the tile
      copy16_to_lds(rq, t_src[it], (char*)dq_ + off);
      copy16_to_lds(rd, t_src[it], (char*)dd_ + off);
    }
    // the tile's base-2 LSE and D, 4 bytes per lane of wave 0 (rows past the end read 0: their
    // Q and dO rows are 0 too, so P = 1 there multiplies zero rows and dS = 0)
    if (wid == 0 && lane < kBQ) {
      const unsigned fb = (unsigned)min(kBQ, N - q0) * 4u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(lse_g + q0, fb), (lds_void*)(dq_ + QT), 4, 4u * lane, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(dlt_g + q0, fb), (lds_void*)(dq_ + QT + 2 * kBQ), 4, 4u * lane, 0, 0, 0);
    }
  };

  f32x16 dq_acc;  // dQ of the previous query block: lane holds [query 8i + 4hh + j][dim wid*QCOLS + r]
  // dQ_{i} of this wave's head dims = dS_i K over the 128 keys of the block (dS^T from LDS)
  auto dq_mfma = [&](auto bufc) {
    const uint16_t* sds = s_ds[decltype(bufc)::value];
    // (all 128 keys, also on diagonal blocks: keys past the block's last query hold dS = 0,
    // and a branch per k-step would keep these products from interleaving with the step's
    // exponentials)
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int row_a = 16 * ks + 4 * hh + (gi >> 2);
      const int row_b = row_a + 8;
      const int qc = 16 * nh + 4 * (gi & 3);
      const bf16x8 ads = join_tr(lds_read_tr(sds + ds_off(row_a, qc)), lds_read_tr(sds + ds_off(row_b, qc)));
      dq_acc = mfma32(ads, kq[ks], ks == 0 ? f32x16{} : dq_acc);
    }
  };
  // Exactly kDqAtomics atomic instructions per call (rows past the end add 0 to the last
  // row), so the step's wait can leave them in flight: see step_sync.
  // A whole query block goes through buffer atomics: the block's wave-uniform base in the
  // buffer resource, the lane's offset in one VGPR, the row of accumulator element i in the
  // scalar offset, so no address arithmetic runs per atomic. Only the ragged last block (or a
  // block whose 32 rows span 4 GB or more) clamps rows one by one.
  const unsigned rs4 = (unsigned)rs * 4u;                                // dQ row stride, bytes
  const unsigned dq_lane = (unsigned)(4 * hh) * rs4 + 4u * (unsigned)r;   // lane's offset in a block
  const bool dq_buf = (size_t)rs * 4u * kBQ <= 0xffffffffu;
  auto dq_atomics = [&](int q0) {
    if (QCOLS == 32 || r < 16) {
      if (dq_buf && q0 + kBQ <= N) {
        const __amdgpu_buffer_rsrc_t rdq = make_rsrc(p.dq + base + (size_t)q0 * rs + wid * QCOLS, rs4 * kBQ);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(dq_acc[i] * p.scale, rdq, dq_lane,
                                                          (int)((8 * (i >> 2) + (i & 3)) * rs4), 0);
      } else {
        float* dqg = p.dq + base + wid * QCOLS + r;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = q0 + 8 * (i >> 2) + 4 * hh + (i & 3);
          const float x = qi < N ? dq_acc[i] * p.scale : 0.f;
          atomicAdd(dqg + (size_t)min(qi, N - 1) * rs, x);
        }
      }
    }
  };
  // End of a step: the tile copies of this step have landed and its LDS accesses are done,
  // then the workgroup barrier. Vector memory operations retire in issue order and the dQ
  // atomics of the step (if any) were issued after the copies, so waiting until at most
  // that many remain leaves the atomics in flight. The barrier is a bare s_barrier: the
  // fences of __syncthreads() (and the compiler's handling of the barrier builtin) would
  // wait for all of them.
  constexpr int kDqAtomics = 16;
  auto step_sync = [&](bool atomics_issued) {
    // s_waitcnt immediate: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
    constexpr int kWaitAtomics = (kDqAtomics & 15) | ((kDqAtomics >> 4) << 14) | (0x7 << 4) | (0x0 << 8);
    if (atomics_issued)
      __builtin_amdgcn_s_waitcnt(kWaitAtomics);  // vmcnt(16) lgkmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt(0);
    asm volatile("s_barrier" ::: "memory");
  };

  // prologue: tile 0, its LSE and D; dS^T buffer 1 cleared (the first step's dQ MFMAs read
  // it, and their zero result is not added anywhere)
  if (nsteps > 0) issue_tile(std::integral_constant<int, 0>(), 0);
  for (int e = tid; e < kBK * kDsStride / 2; e += NT) ((uint32_t*)s_ds[1])[e] = 0u;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // step st (buffer parity B = st & 1): copies of tile st+1; S, dP of tile st; P, dS beside
  // the dQ MFMAs of tile st-1; dS^T of tile st to LDS; dV, dK; atomics of dQ of tile st-1
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
        const int c = 2 * kk + hh;
        aq[kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)(sq + r * D + ((c ^ swz_row<D>(r)) << 3)));
        ad[kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)(sd + r * D + ((c ^ swz_row<D>(r)) << 3)));
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
    // P, dS of this tile beside the dQ MFMAs of the previous tile, laid out by hand in eight
    // chunks fenced by scheduling barriers: chunk t issues dQ MFMA t (its dS^T operand was
    // read two chunks earlier), the operand reads of k-step t + 2, and the VALU work of two
    // of the sixteen P, dS values, which runs while the MFMA does.
    f32x16 pr, ds;
    {
      const uint16_t* sds = s_ds[B ^ 1];
      bf16x8 ads[kBK / 16];
      auto rdq = [&](int ks) {
        const int row_a = 16 * ks + 4 * hh + (gi >> 2);
        const int row_b = row_a + 8;
        const int qc = 16 * nh + 4 * (gi & 3);
        ads[ks] = join_tr(lds_read_tr(sds + ds_off(row_a, qc)), lds_read_tr(sds + ds_off(row_b, qc)));
      };
      rdq(0);
      rdq(1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < kBK / 16; ++t) {
        if (t + 2 < kBK / 16) rdq(t + 2);
        dq_acc = mfma32(ads[t], kq[t], t == 0 ? f32x16{} : dq_acc);
#pragma unroll
        for (int i = 2 * t; i < 2 * t + 2; ++i) {
          pr[i] = exp2_fast(__builtin_fmaf(sc[i], p.scale_log2, -l4[i >> 2][i & 3]));
          ds[i] = pr[i] * (dp[i] - d4[i >> 2][i & 3]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    bf16x8 ap[2], as[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int o8 = 8 * ks;
      ap[ks] = pack_bf16x8(pr[o8], pr[o8 + 1], pr[o8 + 2], pr[o8 + 3], pr[o8 + 4], pr[o8 + 5], pr[o8 + 6], pr[o8 + 7]);
      as[ks] = pack_bf16x8(ds[o8], ds[o8 + 1], ds[o8 + 2], ds[o8 + 3], ds[o8 + 4], ds[o8 + 5], ds[o8 + 6], ds[o8 + 7]);
    }
    // dS^T -> LDS: row = key (32*wid + r), columns = queries 8i + 4hh + 0..3
    {
      // (written with inline ds_write_b64: for the C++ stores the compiler waits for the tile
      // copies in flight, not knowing they target other LDS buffers; the step's closing
      // lgkmcnt(0) orders these writes before the barrier)
      const unsigned dst = (unsigned)(uintptr_t)(const void*)s_ds[B];
      const int row = 32 * wid + r;
      const u32x4 w0 = __builtin_bit_cast(u32x4, as[0]), w1 = __builtin_bit_cast(u32x4, as[1]);
      const u32x2 v0 = {w0[0], w0[1]}, v1 = {w0[2], w0[3]}, v2 = {w1[0], w1[1]}, v3 = {w1[2], w1[3]};
      asm volatile("ds_write_b64 %0, %1" ::"v"(dst + 2u * ds_off(row, 0 + 4 * hh)), "v"(v0) : "memory");
      asm volatile("ds_write_b64 %0, %1" ::"v"(dst + 2u * ds_off(row, 8 + 4 * hh)), "v"(v1) : "memory");
      asm volatile("ds_write_b64 %0, %1" ::"v"(dst + 2u * ds_off(row, 16 + 4 * hh)), "v"(v2) : "memory");
      asm volatile("ds_write_b64 %0, %1" ::"v"(dst + 2u * ds_off(row, 24 + 4 * hh)), "v"(v3) : "memory");
    }
    __builtin_amdgcn_sched_barrier(0);
    if (st > 0) dq_atomics(q0 - kBQ);  // the dQ MFMAs have finished by now
    // dV += P^T dO, dK += dS^T Q  (k-step ks: queries 16ks + 8(e/4) + 4hh + e%4). Operand
    // pair t = (ks, db) is read from LDS two pairs ahead of its MFMAs, so each read has two
    // pairs of products to land behind.
    {
      constexpr int NP = 2 * DB;
      bf16x8 bdo[NP], bq[NP];
      auto rd = [&](int t) {
        const int ks = t / DB, db = t % DB;
        const int row_a = 16 * ks + 4 * hh + (gi >> 2);
        const int row_b = row_a + 8;
        const int col = db * 32 + 16 * nh + 4 * (gi & 3);
        const int ca = (((col >> 3) ^ swz_row<D>(row_a)) << 3) + (col & 7);
        const int cb = (((col >> 3) ^ swz_row<D>(row_b)) << 3) + (col & 7);
        bdo[t] = join_tr(lds_read_tr(sd + row_a * D + ca), lds_read_tr(sd + row_b * D + cb));
        bq[t] = join_tr(lds_read_tr(sq + row_a * D + ca), lds_read_tr(sq + row_b * D + cb));
      };
      rd(0);
      rd(1);
#pragma unroll
      for (int t = 0; t < NP; ++t) {
        if (t + 2 < NP) rd(t + 2);
        const int ks = t / DB, db = t % DB;
        dv_acc[db] = mfma32(ap[ks], bdo[t], dv_acc[db]);
        dk_acc[db] = mfma32(as[ks], bq[t], dk_acc[db]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
      for (int t = 0; t < NP; ++t) {
        if (t + 2 < NP) __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    step_sync(st > 0);
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
  // dQ of the last query block
  if (nsteps > 0) {
    if ((nsteps - 1) & 1) dq_mfma(std::integral_constant<int, 1>());
    else dq_mfma(std::integral_constant<int, 0>());
    dq_atomics(qstart + (nsteps - 1) * kBQ);
  }

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

template <int D, bool CAUSAL>
hipError_t launch_main(const MainArgs& m, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL>), dim3(blocks), dim3(kNW * 64), 0, stream, m);
  return hipGetLastError();
}

template <int D>
hipError_t launch_t(const BwdArgs& a, hipStream_t stream) {
  PreArgs pre;
  pre.o = (const uint16_t*)a.o;
  pre.dout = (const uint16_t*)a.dout;
  pre.lse = a.lse;
  pre.delta = a.delta;
  pre.dq = a.dq;
  pre.dk = a.dk;
  pre.dv = a.dv;
  pre.heads = a.heads;
  pre.seqlen = a.seqlen;
  pre.rows = (long long)a.batch * a.seqlen * a.heads;
  pre.rows_kv = a.kv_heads < a.heads ? (long long)a.batch * a.seqlen * a.kv_heads : 0;
  const long long threads = pre.rows * (D / 8);
  const long long pblocks = (threads + 255) / 256;
  if (pblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_preprocess_kernel<D>), dim3((unsigned)pblocks), dim3(256), 0, stream, pre);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  MainArgs m;
  m.q = (const uint16_t*)a.q;
  m.k = (const uint16_t*)a.k;
  m.v = (const uint16_t*)a.v;
  m.dout = (const uint16_t*)a.dout;
  m.lse = a.lse;
  m.delta = a.delta;
  m.dq = a.dq;
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
  m.rows = pre.rows;
  return a.causal ? launch_main<D, true>(m, (int)blocks, stream) : launch_main<D, false>(m, (int)blocks, stream);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_t<128>(a, stream);
  if (a.head_dim == 64) return launch_t<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
