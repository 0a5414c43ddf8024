// Backward attention by recomputation, bf16 inputs, fp32 gradients, gfx950 MFMA.
//
// Method ("FlashAttention: IO-aware exact attention", "Tile decomposition": the backward
// recomputes tiles instead of storing P; "FlashAttention-2 and -3", "Fewer non-matmul
// FLOPs": a recomputed weight is exp(s - lse); "Parallelism over the sequence": the
// backward is parallel over key blocks, dK_j and dV_j belong to one block, dQ_i is
// accumulated with atomic additions in device memory).
//
// Kernel 1 (preprocess): D_i = sum_c dO_ic O_ic per row, and dQ <- 0.
// Kernel 2 (main): one workgroup per (128-key block, batch*head); each of its 4 waves owns
// 32 keys and keeps K, V (as MFMA operands) and dK, dV (fp32 accumulators) in registers.
// It walks 32-query blocks (causal: only those that can see a key of the block), staged
// in LDS with the next block's loads in flight:
//   S  = Q K^T            (queries x keys; one key per lane, 16 queries per lane)
//   P  = exp2(S*c - LSE2) , dP = dO V^T , dS = P * (dP - D)
//   dV += P^T dO ,  dK += dS^T Q   (P, dS straight from registers; dO, Q transposed by
//                                   the LDS transpose read)
//   dS^T goes to LDS; then each wave forms 32 of the head dims of dQ_i = dS K over all
//   128 keys of the block and adds them into dQ with one fp32 atomic per element.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kNW = 4;          // waves per workgroup
constexpr int kBK = 32 * kNW;   // keys per workgroup
constexpr int kBQ = 32;         // queries per step
constexpr int kDsStride = 36;   // dS^T row stride in elements (72 bytes, conflict-free writes)

struct PreArgs {
  const uint16_t* o;
  const uint16_t* dout;
  float* delta;
  float* dq;
  int heads, seqlen;
  long long rows;  // B * N * H
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
  }
  // sum over the CH lanes of the row (CH divides 64, rows are lane-aligned)
#pragma unroll
  for (int s = 1; s < CH; s <<= 1) acc += __shfl_xor(acc, s);
  if (row < p.rows && sub == 0) {
    const int h = (int)(row % p.heads);
    const long long bn = row / p.heads;
    const int n = (int)(bn % p.seqlen);
    const long long b = bn / p.seqlen;
    p.delta[((size_t)b * p.heads + h) * p.seqlen + n] = acc;
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
  int heads, seqlen, nkb;
  int grid;  // workgroups launched
  float scale, scale_log2;
};

template <int D>
__device__ __forceinline__ int swz_row(int row) {  // rows read 32 at a time by ds_read_b128
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
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
  constexpr int LOADS = kBQ * CH / NT;        // 16-byte chunks per thread per tile
  static_assert(kBQ * CH % NT == 0, "tile split");
  static_assert(D / 32 == kNW || D == 64, "dQ head-dim split assumes D = 32 * waves (or D = 64)");

  __shared__ __attribute__((aligned(16))) uint16_t s_k[kBK * D];          // K block (transpose reads)
  __shared__ __attribute__((aligned(16))) uint16_t s_q[2][QT];             // Q tiles
  __shared__ __attribute__((aligned(16))) uint16_t s_do[2][QT];            // dO tiles
  __shared__ __attribute__((aligned(16))) uint16_t s_ds[kBK * kDsStride];  // dS^T [key][query]
  __shared__ __attribute__((aligned(16))) float s_lse[2][kBQ];
  __shared__ __attribute__((aligned(16))) float s_dlt[2][kBQ];

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
  const size_t rs = (size_t)p.heads * D;
  const size_t base = ((size_t)b * N * p.heads + h) * D;
  const float* lse_g = p.lse + ((size_t)b * p.heads + h) * N;
  const float* dlt_g = p.delta + ((size_t)b * p.heads + h) * N;

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
      xk = *(const u32x4*)(p.k + base + (size_t)myk * rs + 16 * kk + 8 * hh);
      xv = *(const u32x4*)(p.v + base + (size_t)myk * rs + 16 * kk + 8 * hh);
    }
    kf[kk] = __builtin_bit_cast(bf16x8, xk);
    vf[kk] = __builtin_bit_cast(bf16x8, xv);
  }
  // whole K block into LDS (row-major, read transposed for dQ = dS K)
  for (int ci = tid; ci < kBK * CH; ci += NT) {
    const int row = ci / CH, c = ci % CH;
    const int key = kb0 + row;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (key < N) x = *(const u32x4*)(p.k + base + (size_t)key * rs + c * 8);
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

  u32x4 qreg[LOADS], doreg[LOADS];
  float lreg = 0.f, dreg = 0.f;
  auto load_step = [&](int st) {
    const int q0 = qstart + st * kBQ;
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int ci = tid + it * NT;
      const int row = ci / CH, c = ci % CH;
      const int qi = q0 + row;
      u32x4 zq = {0u, 0u, 0u, 0u}, zd = {0u, 0u, 0u, 0u};
      if (qi < N) {
        zq = *(const u32x4*)(p.q + base + (size_t)qi * rs + c * 8);
        zd = *(const u32x4*)(p.dout + base + (size_t)qi * rs + c * 8);
      }
      qreg[it] = zq;
      doreg[it] = zd;
    }
    if (tid < kBQ) {
      const int qi = q0 + tid;
      lreg = qi < N ? lse_g[qi] * kLog2e : INFINITY;  // invalid rows get P = 0
      dreg = qi < N ? dlt_g[qi] : 0.f;
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int ci = tid + it * NT;
      const int row = ci / CH, c = ci % CH;
      *(u32x4*)(&s_q[buf][row * D + ((c ^ swz_row<D>(row)) << 3)]) = qreg[it];
      *(u32x4*)(&s_do[buf][row * D + ((c ^ swz_row<D>(row)) << 3)]) = doreg[it];
    }
    if (tid < kBQ) {
      s_lse[buf][tid] = lreg;
      s_dlt[buf][tid] = dreg;
    }
  };

  if (nsteps > 0) {
    load_step(0);
    store_step(0);
  }
  __syncthreads();

  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    const int q0 = qstart + st * kBQ;
    if (st + 1 < nsteps) load_step(st + 1);
    const uint16_t* sq = s_q[buf];
    const uint16_t* sd = s_do[buf];

    const bool active = myk - r < N && (!CAUSAL || q0 + kBQ - 1 >= kw);
    f32x16 pr, ds;  // P and dS, lane = key r, acc[4i+j] = query 8i + 4hh + j
    if (active) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) { s[i] = 0.f; dp[i] = 0.f; }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int c = 2 * kk + hh;
        const bf16x8 aq = __builtin_bit_cast(bf16x8, *(const u32x4*)(sq + r * D + ((c ^ swz_row<D>(r)) << 3)));
        const bf16x8 ad = __builtin_bit_cast(bf16x8, *(const u32x4*)(sd + r * D + ((c ^ swz_row<D>(r)) << 3)));
        s = mfma32(aq, kf[kk], s);
        dp = mfma32(ad, vf[kk], dp);
      }
      const bool edge = (CAUSAL && q0 < kw + 31) || (q0 + kBQ > N) || (kw + 32 > N);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 l4 = *(const f32x4*)(&s_lse[buf][8 * i4 + 4 * hh]);
        const f32x4 d4 = *(const f32x4*)(&s_dlt[buf][8 * i4 + 4 * hh]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * i4 + j;
          float pv = exp2_fast(__builtin_fmaf(s[i], p.scale_log2, -l4[j]));
          if (edge) {
            const int qi = q0 + 8 * i4 + 4 * hh + j;
            if ((CAUSAL && myk > qi) || myk >= N) pv = 0.f;
          }
          pr[i] = pv;
          ds[i] = pv * (dp[i] - d4[j]);
        }
      }
      // dV += P^T dO, dK += dS^T Q  (k-step ks: queries 16ks + 8(e/4) + 4hh + e%4)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int o8 = 8 * ks;
        const bf16x8 ap = pack_bf16x8(pr[o8], pr[o8 + 1], pr[o8 + 2], pr[o8 + 3],
                                      pr[o8 + 4], pr[o8 + 5], pr[o8 + 6], pr[o8 + 7]);
        const bf16x8 as = pack_bf16x8(ds[o8], ds[o8 + 1], ds[o8 + 2], ds[o8 + 3],
                                      ds[o8 + 4], ds[o8 + 5], ds[o8 + 6], ds[o8 + 7]);
        const int row_a = 16 * ks + 4 * hh + (gi >> 2);
        const int row_b = row_a + 8;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int col = db * 32 + 16 * nh + 4 * (gi & 3);
          const int ca = (((col >> 3) ^ swz_row<D>(row_a)) << 3) + (col & 7);
          const int cb = (((col >> 3) ^ swz_row<D>(row_b)) << 3) + (col & 7);
          const bf16x8 bdo = join_tr(lds_read_tr(sd + row_a * D + ca), lds_read_tr(sd + row_b * D + cb));
          const bf16x8 bq = join_tr(lds_read_tr(sq + row_a * D + ca), lds_read_tr(sq + row_b * D + cb));
          dv_acc[db] = mfma32(ap, bdo, dv_acc[db]);
          dk_acc[db] = mfma32(as, bq, dk_acc[db]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = 0.f;
    }
    // dS^T -> LDS: row = key (32*wid + r), columns = queries 8i + 4hh + 0..3
    {
      uint16_t* dst = s_ds + (32 * wid + r) * kDsStride + 4 * hh;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        u32x2 wv;
        wv[0] = pack_bf16x2(ds[4 * i4 + 0], ds[4 * i4 + 1]);
        wv[1] = pack_bf16x2(ds[4 * i4 + 2], ds[4 * i4 + 3]);
        *(u32x2*)(dst + 8 * i4) = wv;
      }
    }
    __syncthreads();

    // dQ_i[:, cols of this wave] = scale * dS K over the 128 keys of the block
    {
      f32x16 dq_acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) dq_acc[i] = 0.f;
      const int kmax = CAUSAL ? min(kBK, q0 + kBQ - kb0) : kBK;  // keys past the last query give dS = 0
#pragma unroll
      for (int ks = 0; ks < kBK / 16; ++ks) {
        if (16 * ks >= kmax) break;
        const int row_a = 16 * ks + 4 * hh + (gi >> 2);
        const int row_b = row_a + 8;
        // A = dS (queries x keys): transpose read of dS^T rows (keys), columns (queries)
        const int qc = 16 * nh + 4 * (gi & 3);
        const bf16x8 ads = join_tr(lds_read_tr(s_ds + row_a * kDsStride + qc),
                                   lds_read_tr(s_ds + row_b * kDsStride + qc));
        dq_acc = mfma32(ads, kq[ks], dq_acc);
      }
      // lane holds dQ[query 8i + 4hh + j][dim wid*QCOLS + r]
      if (QCOLS == 32 || r < 16) {
        float* dqg = p.dq + base + wid * QCOLS + r;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = q0 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (qi < N) atomicAdd(dqg + (size_t)qi * rs, dq_acc[i] * p.scale);
        }
      }
    }
    if (st + 1 < nsteps) store_step(buf ^ 1);
    __syncthreads();
  }

  // dK = scale * dS^T Q, dV = P^T dO; lane holds [key 8i + 4hh + j][dim db*32 + r]
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kw + 8 * (i >> 2) + 4 * hh + (i & 3);
      if (key < N) {
        const size_t off = base + (size_t)key * rs + db * 32 + r;
        p.dk[off] = dk_acc[db][i] * p.scale;
        p.dv[off] = dv_acc[db][i];
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
  pre.delta = a.delta;
  pre.dq = a.dq;
  pre.heads = a.heads;
  pre.seqlen = a.seqlen;
  pre.rows = (long long)a.batch * a.seqlen * a.heads;
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
  m.seqlen = a.seqlen;
  m.nkb = (a.seqlen + kBK - 1) / kBK;
  m.scale = a.scale;
  m.scale_log2 = a.scale * kLog2e;
  const long long blocks = (long long)m.nkb * a.batch * a.heads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  m.grid = (int)blocks;
  return a.causal ? launch_main<D, true>(m, (int)blocks, stream) : launch_main<D, false>(m, (int)blocks, stream);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_t<128>(a, stream);
  if (a.head_dim == 64) return launch_t<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
