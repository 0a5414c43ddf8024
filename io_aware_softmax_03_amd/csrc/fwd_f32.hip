// Forward attention in fp32 throughout (inputs, products, softmax, output).
//
// The exact-precision path: the tiled online softmax of the bf16 kernel ("Tile
// decomposition", "Online softmax"), with every product an fp32 FMA rather than a reduced
// precision matrix-core product, so results stay within fp32 rounding of the exact value.
//
// A workgroup of 256 threads owns RQ query rows of one head (RQ = 8, 4 or 1: the largest
// that still gives the grid two workgroups per compute unit) and streams the keys in blocks
// of 256, one key per thread:
//  - scores: thread t holds key t's row of K in registers and forms its RQ dot products
//    against the workgroup's Q rows (read from LDS as broadcasts), so no cross-lane sum is
//    needed; the block's row maxima are wave reductions merged through LDS;
//  - weights: each thread rescales its own partial row sums; they are added over the
//    workgroup once, at the end (all partials share the row's running maximum);
//  - P V: thread (g, c) accumulates output columns 4c..4c+3 of every row over key group g of
//    the block (V read straight from memory as 16-byte rows); the groups' partial outputs
//    are added through LDS at the end.
// K and V of a block are requested before its scores are formed (V, at d = 128, right after),
// so their latency overlaps the score and softmax work. It takes the same general mask as the bf16
// kernel (query i sees key j when i + lo_off <= j, and j <= i + hi_off when banded) and
// grouped key-value heads.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kKB = 256;      // keys per block, one per thread in the score phase
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return pair_max(x);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) x += __shfl_xor(x, off);
  return pair_sum(x);
}

template <int D, int RQ, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(F32Args p) {
  constexpr int NCQ = D / 4;             // 4-column groups of an output row
  constexpr int G = kThreads / NCQ;      // key groups of the P V phase
  constexpr int KPG = kKB / G;           // keys per group and block
  static_assert(kThreads % NCQ == 0 && KPG % 4 == 0, "P V layout");
  __shared__ __attribute__((aligned(16))) float qs[RQ * D];     // the workgroup's Q rows
  __shared__ __attribute__((aligned(16))) float ps[RQ * kKB];   // weights of the current block
  __shared__ __attribute__((aligned(16))) float os[G * RQ * D]; // partial outputs per key group
  __shared__ float red[RQ * kWaves];                            // per-wave maxima / sums

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
  const int tid = thread_id_x();
  const int lane = tid & 63, wave = tid >> 6;
  const int cq = tid % NCQ, grp = tid / NCQ;
  const size_t rs = (size_t)p.heads * D;      // Q / O row stride
  const size_t rsk = (size_t)p.kv_heads * D;  // K / V row stride
  const size_t base = ((size_t)seq_start * p.heads + h) * D;
  const float* kbase = p.k + ((size_t)seq_start_k * p.kv_heads + h / p.group) * D;
  const float* vbase = p.v + ((size_t)seq_start_k * p.kv_heads + h / p.group) * D + 4 * cq;

  // query blocks qb_first, qb_first + nqb, ...: a packed sequence longer than the grid was
  // sized for (max_seqlen understated) is still computed in full
  for (int qb = qb_first; qb * RQ < L; qb += p.nqb) {
    const int q0 = qb * RQ;
    const int nrow = min(RQ, L - q0);
    __syncthreads();  // the previous query block is done with the LDS buffers
    for (int e = tid; e < RQ * D; e += kThreads) {
      const int r = e / D, c = e % D;
      qs[e] = r < nrow ? p.q[base + (size_t)(q0 + r) * rs + c] : 0.f;
    }

    float m[RQ], lt[RQ], o[RQ][4];
#pragma unroll
    for (int r = 0; r < RQ; ++r) {
      m[r] = -INFINITY;
      lt[r] = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) o[r][c] = 0.f;
    }

    // keys any row of the block can see: from the first row's lowest to the last row's highest
    int kv_end = Lk;
    if constexpr (CAUSAL) kv_end = min(Lk, q0 + nrow + p.hi_off);
    const int kv_begin = max(0, q0 + p.lo_off);
    for (int k0 = kv_begin; k0 < kv_end; k0 += kKB) {
      // this thread's key row, and the V rows of its P V group (indices clamped into the
      // sequence; keys past its end get weight zero)
      float kr[D];
      {
        const float* src = kbase + (size_t)min(k0 + tid, Lk - 1) * rsk;
#pragma unroll
        for (int c = 0; c < D; c += 4) {
          const f32x4 x = *(const f32x4*)(src + c);
          kr[c] = x[0];
          kr[c + 1] = x[1];
          kr[c + 2] = x[2];
          kr[c + 3] = x[3];
        }
      }
      // at d = 64 the V rows are requested with the K row; at d = 128 (128 registers each) after
      // the scores, once the K row is dead, still ahead of the softmax's reductions
      f32x4 vr[KPG];
      auto load_v = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < KPG; ++j) vr[j] = *(const f32x4*)(vbase + (size_t)min(k0 + grp * KPG + j, Lk - 1) * rsk);
      };
      if constexpr (D == 64) load_v();
      if (k0 == kv_begin) __syncthreads();  // Q rows staged

      // scores of key k0 + tid against the RQ rows, four head dims at a time: the Q reads of
      // the next four dims are issued before the FMAs of the current ones, and scheduling
      // barriers keep the compiler from hoisting all RQ * D of them into registers (their
      // address also comes from an opaque zero, so they stay inside the key loop)
      int qoff = 0;
      asm volatile("" : "+v"(qoff));
      qoff &= ~3;  // a multiple of four floats: the reads stay 16-byte aligned
      // (with fewer than four rows each row's sum is split over four chains, one per
      // component of the 16-byte reads, so the FMAs do not wait on each other)
      constexpr int NA = RQ < 4 ? 4 : 1;
      float sa[RQ][NA];
#pragma unroll
      for (int r = 0; r < RQ; ++r)
#pragma unroll
        for (int a = 0; a < NA; ++a) sa[r][a] = 0.f;
      f32x4 qcur[RQ];
#pragma unroll
      for (int r = 0; r < RQ; ++r) qcur[r] = *(const f32x4*)(qs + qoff + r * D);
#pragma unroll
      for (int c = 0; c < D; c += 4) {
        f32x4 qnext[RQ];
        if (c + 4 < D) {
#pragma unroll
          for (int r = 0; r < RQ; ++r) qnext[r] = *(const f32x4*)(qs + qoff + r * D + c + 4);
        }
#pragma unroll
        for (int r = 0; r < RQ; ++r)
#pragma unroll
          for (int u = 0; u < 4; ++u) sa[r][u % NA] = __builtin_fmaf(qcur[r][u], kr[c + u], sa[r][u % NA]);
        __builtin_amdgcn_sched_barrier(0);
        if (c + 4 < D) {
#pragma unroll
          for (int r = 0; r < RQ; ++r) qcur[r] = qnext[r];
        }
      }
      if constexpr (D != 64) load_v();
      float s[RQ];
#pragma unroll
      for (int r = 0; r < RQ; ++r) {
        if constexpr (NA == 4)
          s[r] = (sa[r][0] + sa[r][1]) + (sa[r][2] + sa[r][3]);
        else
          s[r] = sa[r][0];
      }
      // the dot products are complete here (kept from being sunk into the masking code)
#pragma unroll
      for (int r = 0; r < RQ; ++r) asm volatile("" : "+v"(s[r]));
      const int key = k0 + tid;
#pragma unroll
      for (int r = 0; r < RQ; ++r) {
        const int i = q0 + r;
        const bool keep = r < nrow && key < Lk && key >= i + p.lo_off && (!CAUSAL || key <= i + p.hi_off);
        s[r] = keep ? s[r] * p.scale_log2 : -INFINITY;
        const float mw = wave_max(s[r]);
        if (lane == 0) red[r * kWaves + wave] = mw;
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < RQ; ++r) {
        float mb = red[r * kWaves];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) mb = fmaxf(mb, red[r * kWaves + w]);
        const float m_new = fmaxf(m[r], mb);
        const float piv = m_new == -INFINITY ? 0.f : m_new;  // no key of the row seen yet
        const float alpha = exp2_fast(m[r] - piv);
        const float pr = exp2_fast(s[r] - piv);
        lt[r] = lt[r] * alpha + pr;
        ps[r * kKB + tid] = pr;
        m[r] = m_new;
#pragma unroll
        for (int c = 0; c < 4; ++c) o[r][c] *= alpha;
      }
      __syncthreads();

      // O += P V over this thread's key group
#pragma unroll
      for (int j = 0; j < KPG; j += 4) {
#pragma unroll
        for (int r = 0; r < RQ; ++r) {
          const f32x4 pw = *(const f32x4*)(ps + r * kKB + grp * KPG + j);
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) o[r][c] = __builtin_fmaf(pw[u], vr[j + u][c], o[r][c]);
        }
      }
    }

    // row sums over the workgroup; partial outputs of the key groups added through LDS
#pragma unroll
    for (int r = 0; r < RQ; ++r) {
      const float sw = wave_sum(lt[r]);
      if (lane == 0) red[r * kWaves + wave] = sw;
#pragma unroll
      for (int c = 0; c < 4; ++c) os[(grp * RQ + r) * D + 4 * cq + c] = o[r][c];
    }
    __syncthreads();
    for (int e = tid; e < nrow * D; e += kThreads) {
      const int r = e / D, c = e % D;
      float l = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) l += red[r * kWaves + w];
      float acc = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) acc += os[(g * RQ + r) * D + c];
      p.o[base + (size_t)(q0 + r) * rs + c] = l > 0.f ? acc / l : 0.f;
    }
    if (tid < nrow) {
      float l = 0.f, mr = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) l += red[tid * kWaves + w];
#pragma unroll
      for (int r = 0; r < RQ; ++r)
        if (r == tid) mr = m[r];
      const float lse = l > 0.f ? (mr + log2_fast(l)) * kLn2 : -INFINITY;
      if constexpr (VARLEN)
        p.lse[(size_t)h * p.total_rows + seq_start + q0 + tid] = lse;
      else
        p.lse[((size_t)bs * p.heads + h) * p.seqlen + q0 + tid] = lse;
    }
  }  // query blocks
}

template <int D, int RQ, bool CAUSAL, bool VARLEN>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
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
  p.nqb = (a.seqlen + RQ - 1) / RQ;
  p.scale_log2 = a.scale * kLog2e;
  const long long blocks = (long long)p.nqb * a.heads * a.batch;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_f32_kernel<D, RQ, CAUSAL, VARLEN>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_rq(const FwdArgs& a, hipStream_t stream) {
  // the largest query block (8 or 4 rows) that still gives two workgroups per compute unit,
  // else one row per workgroup: small problems are bound by latency and the grid's width,
  // large ones by the K and V rows each workgroup streams (once per RQ rows)
  const long long bh = (long long)a.heads * a.batch;
  if ((a.seqlen + 7) / 8 * bh >= 512) return launch_t<D, 8, CAUSAL, VARLEN>(a, stream);
  if ((a.seqlen + 3) / 4 * bh >= 512) return launch_t<D, 4, CAUSAL, VARLEN>(a, stream);
  return launch_t<D, 1, CAUSAL, VARLEN>(a, stream);
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  const bool varlen = a.cu_seqlens != nullptr;
  if (a.banded) return varlen ? launch_rq<D, true, true>(a, stream) : launch_rq<D, true, false>(a, stream);
  return varlen ? launch_rq<D, false, true>(a, stream) : launch_rq<D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  if (a.head_dim == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
