// FP8 forward attention ("FlashAttention-2 and -3", section "FP8, and the outlier problem").
//
// Two kernels after one another on the caller's stream:
//
// 1. fp8_quant_qkv_kernel, one launch for Q, K and V (their workgroups interleaved): one
//    workgroup per block of 64 rows of one head. Q and K rows are optionally rotated by R = H_d D / sqrt(d) (incoherent
//    processing: Hadamard matrix times a random +-1 diagonal). The kernel forms x H_d D with
//    the fast Walsh-Hadamard transform in fp32 (butterflies at strides 1, 2, ..., d/2) and
//    leaves the 1/sqrt(d) to the score scale (1/d there). Each block gets one power-of-two
//    scale 2^e, the smallest with amax <= 448 * 2^e (block quantization), and every value
//    becomes the e4m3 code of x * 2^-e (exact scaling, round to nearest even). Q and K
//    codes are stored head-major, [B, H, rows, d]; V codes are stored per 64-key block
//    transposed, [B, H, block, d, 64], with the keys of a block in the order the attention
//    kernel's P registers hold them, so each lane's V^T operand is 32 contiguous bytes.
// 2. fwd_fp8_kernel: 4 waves of 32 query rows per workgroup, two workgroups per CU (about
//    220 registers a wave). Per 64-key block the K and V^T tiles (contiguous 8 KB blocks of
//    the workspace) are copied straight into LDS (K two blocks ahead, V^T one) and shared by
//    the four waves; S^T = K Q^T and O^T += V^T P^T run on
//    v_mfma_scale_f32_32x32x64_f8f6f4, the online softmax in fp32 (base 2), and P is
//    quantized to e4m3 as P * 2^8 (formed directly as 2^(s - m + 8)). Within a wave the
//    work is pipelined over three blocks: step j forms S(j+1) and multiplies P(j-1) into O on
//    the matrix core while the VALU forms the codes of P(j) (exact running maximum, so
//    P <= 1). The block scales enter exactly: 2^(eq + ek) on the score scale, 2^ev and 2^-8
//    through the MFMA's E8M0 operand scales. The row sum and the LSE use the unquantized P.
//
// Operand layouts of v_mfma_scale_f32_32x32x64_f8f6f4 with e4m3 operands (lane l, r = l%32,
// hh = l/32): A row r, B column r; the 32 bytes of a lane are 32 of the 64 k indices, and A
// and B are paired by (hh, byte), so any k order used for both operands is the same product.
// C: lane holds C[8i + 4hh + j][r] at acc[4i + j] (as for the bf16 32x32 products).
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kRows = 64;  // quantization block and key block
constexpr int kPScaleLog2 = 8;

// x * 2^-e rounded to e4m3 (pairs; lo byte first)
__device__ __forceinline__ uint32_t cvt4_fp8(float a, float b, float c, float d, int e) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(a, -e), __builtin_amdgcn_ldexpf(b, -e), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(c, -e), __builtin_amdgcn_ldexpf(d, -e), w, true);
  return (uint32_t)w;
}

struct QuantArgs {
  const uint16_t* x;   // bf16 [B, N, Hx, d]
  const float* signs;  // [d] of +-1 (rotation) or unused
  uint8_t* out;        // rows: [B, Hx, nblk * 64, d]; transposed V: [B, Hx, nblk, d, 64]
  int* exps;           // [B, Hx, nblk]
  int heads, seqlen, nblk;
};

// key slot (0..63) of the transposed V block -> key within the block. The attention kernel
// packs the 32 probabilities a lane holds for keys 32t + 8i + 4hh + j as bytes 16t + 4i + j
// of its B operand in lane half hh; V^T must hold the same key at slot 32hh + 16t + 4i + j.
__device__ __forceinline__ int slot_key(int s) {
  const int hh = s >> 5, t = (s >> 4) & 1, i = (s >> 2) & 3, j = s & 3;
  return 32 * t + 8 * i + 4 * hh + j;
}

// value of lane l ^ M within each group of four lanes (DPP quad permutation)
template <int M>
__device__ __forceinline__ float quad_xor(float x) {
  constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xf, 0xf, false));
}

template <int D, bool ROTATE, bool VT>
__device__ __forceinline__ void fp8_quant_block(const QuantArgs& p, int w) {
  constexpr int EPT = D / 4;  // elements per thread: each row is spread over 4 threads
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[VT ? kRows * D : 16];
  // heads fastest: consecutive blocks w take the same 64 rows of every head, which are
  // contiguous in the [B, N, H, d] input, so the running workgroups read whole rows
  const int h = w % p.heads;
  const int blk = (w / p.heads) % p.nblk;
  const int b = w / (p.heads * p.nblk);
  const int bh = b * p.heads + h;
  const int t = thread_id_x();
  const int r = t >> 2, part = t & 3;
  const int row = blk * kRows + r;

  float y[EPT];
  if (row < p.seqlen) {
    const uint16_t* src = p.x + (((size_t)b * p.seqlen + row) * p.heads + h) * D + part * EPT;
#pragma unroll
    for (int c = 0; c < EPT / 8; ++c) {
      const u32x4 v = *(const u32x4*)(src + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[8 * c + 2 * e] = bf16_lo(v[e]);
        y[8 * c + 2 * e + 1] = bf16_hi(v[e]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPT; ++i) y[i] = 0.f;
  }

  float sg[ROTATE ? EPT : 1];
  if constexpr (ROTATE) {
#pragma unroll
    for (int c = 0; c < EPT / 4; ++c) {
      const f32x4 v = *(const f32x4*)(p.signs + part * EPT + 4 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) sg[4 * c + e] = v[e];
    }
  }

  if constexpr (ROTATE) {
    // x H_d: butterflies (a, b) -> (a + b, a - b), strides 1 .. EPT/2 inside the thread,
    // then EPT and 2 EPT between the row's four threads (adjacent lanes of a quad)
#pragma unroll
    for (int hs = 1; hs < EPT; hs <<= 1)
#pragma unroll
      for (int i = 0; i < EPT; ++i)
        if ((i & hs) == 0) {
          const float a = y[i], c = y[i + hs];
          y[i] = a + c;
          y[i + hs] = a - c;
        }
    // (the upper lane of a pair forms o - y, the lower y + o: one FMA with a lane sign of
    // -1 or +1, exact in the product, so the same single rounding as the difference or sum)
    {
      const float sgn = (part & 1) != 0 ? -1.f : 1.f;
#pragma unroll
      for (int i = 0; i < EPT; ++i) y[i] = __builtin_fmaf(y[i], sgn, quad_xor<1>(y[i]));
    }
    {
      const float sgn = (part & 2) != 0 ? -1.f : 1.f;
#pragma unroll
      for (int i = 0; i < EPT; ++i) y[i] = __builtin_fmaf(y[i], sgn, quad_xor<2>(y[i]));
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) y[i] *= sg[i];
  }

  // block maximum magnitude -> exponent: smallest e with amax <= 448 * 2^e
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) am = fmaxf(am, fabsf(y[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  if ((t & 63) == 0) red[t >> 6] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int e = 0;
  if (am > 0.f) {
    const int E = __builtin_amdgcn_frexp_expf(am);    // am = f * 2^E, f in [0.5, 1)
    const float f = __builtin_amdgcn_frexp_mantf(am);
    e = f <= 0.875f ? E - 9 : E - 8;                 // 448 = 0.875 * 2^9
  }
  if (t == 0) p.exps[bh * p.nblk + blk] = e;

  uint32_t code[EPT / 4];
#pragma unroll
  for (int i = 0; i < EPT / 4; ++i) code[i] = cvt4_fp8(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3], e);

  if constexpr (!VT) {
    uint8_t* dst = p.out + ((size_t)bh * p.nblk * kRows + row) * D + part * EPT;
#pragma unroll
    for (int c = 0; c < EPT / 16; ++c) {
      u32x4 v = {code[4 * c], code[4 * c + 1], code[4 * c + 2], code[4 * c + 3]};
      *(u32x4*)(dst + 16 * c) = v;
    }
  } else {
    // stage the block's codes [key][dim] in LDS, then write it transposed: thread t covers
    // 16 * (D / 64) consecutive bytes of the [d][64] block
#pragma unroll
    for (int c = 0; c < EPT / 16; ++c) {
      u32x4 v = {code[4 * c], code[4 * c + 1], code[4 * c + 2], code[4 * c + 3]};
      *(u32x4*)(tile + r * D + part * EPT + 16 * c) = v;
    }
    __syncthreads();
    // 4 x 4 byte blocks: slots 4sg .. 4sg+3 (four consecutive keys from slot_key(4sg)) of
    // dims 4dg .. 4dg+3; one 4-byte LDS read per key, a byte transpose, one 4-byte store per
    // dim (16 consecutive threads fill a dim's 64 bytes)
    uint8_t* dst = p.out + ((size_t)bh * p.nblk + blk) * D * kRows;
    constexpr int GROUPS = (D / 4) * (kRows / 4);
#pragma unroll
    for (int g = t; g < GROUPS; g += 256) {
      const int dg = g / (kRows / 4), sg = g % (kRows / 4);
      const int k0 = slot_key(4 * sg);
      uint32_t wk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) wk[j] = *(const uint32_t*)(tile + (k0 + j) * D + 4 * dg);
      // v_perm_b32(a, b, sel): selector bytes 0-3 pick bytes of b, 4-7 bytes of a
      const uint32_t t0 = __builtin_amdgcn_perm(wk[1], wk[0], 0x05010400u);
      const uint32_t t1 = __builtin_amdgcn_perm(wk[1], wk[0], 0x07030602u);
      const uint32_t t2 = __builtin_amdgcn_perm(wk[3], wk[2], 0x05010400u);
      const uint32_t t3 = __builtin_amdgcn_perm(wk[3], wk[2], 0x07030602u);
      const uint32_t od[4] = {__builtin_amdgcn_perm(t2, t0, 0x05040100u), __builtin_amdgcn_perm(t2, t0, 0x07060302u),
                              __builtin_amdgcn_perm(t3, t1, 0x05040100u), __builtin_amdgcn_perm(t3, t1, 0x07060302u)};
#pragma unroll
      for (int e = 0; e < 4; ++e) *(uint32_t*)(dst + (4 * dg + e) * kRows + 4 * sg) = od[e];
    }
  }
}

// Q, K (rotated when ROTATE) and V (transposed) quantized by one launch: workgroups
// 3i, 3i+1, 3i+2 take block i of Q, K and V (i < nkv), the rest the remaining blocks of Q
// (more query than key-value heads), so the three passes' loads, arithmetic and stores overlap
// and there is one tail instead of three.
template <int D, bool ROTATE>
__global__ __launch_bounds__(256) void fp8_quant_qkv_kernel(QuantArgs q, QuantArgs k, QuantArgs v, int nkv) {
  const int w = group_id_x();
  if (w < 3 * nkv) {
    const int t = w % 3, i = w / 3;
    if (t == 0)
      fp8_quant_block<D, ROTATE, false>(q, i);
    else if (t == 1)
      fp8_quant_block<D, ROTATE, false>(k, i);
    else
      fp8_quant_block<D, false, true>(v, i);
  } else {
    fp8_quant_block<D, ROTATE, false>(q, w - 2 * nkv);
  }
}

struct AttnArgs {
  const uint8_t* q8;   // [B, H, Np, d]
  const uint8_t* k8;   // [B, Hkv, Np, d]
  const uint8_t* v8t;  // [B, Hkv, nblk, d, 64]
  const int* eq;       // [B, H, nblk]
  const int* ek;       // [B, Hkv, nblk]
  const int* ev;       // [B, Hkv, nblk]
  uint16_t* o;         // bf16 [B, N, H, d]
  float* lse;          // [B, H, N]
  int heads, kv_heads, group, seqlen, nblk, nqb;
  float c2;            // scale * log2(e), divided by d when Q and K were rotated
};

// v_max3_f32 as one instruction (plain fmaxf chains are not always fused)
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// LDS tiles of one 64-key block, filled by buffer loads straight into LDS. 16-byte chunks are
// XOR-swizzled by row so that the 16 lanes of each quarter-wave read hit 16 distinct bank
// groups: K rows (128 bytes, 8 chunks) by (row / 2) % 8; V^T rows (64 bytes, 4 chunks, one
// row per head dim) by (row / 4) % 4.
template <int D>
__device__ __forceinline__ int swz_kt(int row) { return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3); }
__device__ __forceinline__ int swz_vt8(int row) { return (row >> 2) & 3; }

constexpr int kQRows = 128;  // query rows per workgroup: 4 waves x 32

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(AttnArgs p) {
  constexpr int KS = D / 64;          // k-steps of S^T over the head dim
  constexpr int DB = D / 32;          // 32-dim blocks of O^T
  constexpr int TILE = kRows * D;     // bytes of one K block or one V^T block
  constexpr int LOADS = TILE / 1024 / 4;  // 1 KB wave-loads per wave per tile
  static_assert(TILE % 4096 == 0, "tile must split over four waves");
  __shared__ __attribute__((aligned(1024))) char k_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILE];
  auto kbuf = [&](auto bc) -> char* { return (decltype(bc)::value & 1) ? k_lds1 : k_lds0; };
  auto vbuf = [&](auto bc) -> char* { return (decltype(bc)::value & 1) ? v_lds1 : v_lds0; };

  const int w = group_id_x();
  const int pi = w % p.nqb;
  const int bh = w / p.nqb;
  const int h = bh % p.heads, bs = bh / p.heads;
  const int hk = h / p.group;
  const int N = p.seqlen;
  const int nb = (N + kQRows - 1) / kQRows;
  const size_t Np = (size_t)p.nblk * kRows;
  const uint8_t* qhead = p.q8 + ((size_t)bs * p.heads + h) * Np * D;
  const uint8_t* khead = p.k8 + ((size_t)bs * p.kv_heads + hk) * Np * D;
  const uint8_t* vhead = p.v8t + ((size_t)bs * p.kv_heads + hk) * Np * D;
  // block exponents of K and V, read through the constant address space so that the
  // per-step reads are scalar loads (written by the quantization launches before this one)
  typedef const __attribute__((address_space(4))) int cint;
  cint* ekp = (cint*)(p.ek + ((size_t)bs * p.kv_heads + hk) * p.nblk);
  cint* evp = (cint*)(p.ev + ((size_t)bs * p.kv_heads + hk) * p.nblk);

  const int tid = thread_id_x();
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r = lane & 31, hh = lane >> 5;

  // per-lane source offsets of this wave's wave-loads (the lane fetches the logical chunk
  // the swizzle puts at its physical place) and LDS read offsets of the operands
  unsigned k_src[LOADS], v_src[LOADS];
#pragma unroll
  for (int it = 0; it < LOADS; ++it) {
    const int byte = (wid * LOADS + it) * 1024 + 16 * lane;  // physical byte in the tile
    const int kr = byte / (D), kp = (byte % D) / 16;
    k_src[it] = (unsigned)(kr * D + ((kp ^ swz_kt<D>(kr)) * 16));
    const int vr = byte / kRows, vp = (byte % kRows) / 16;
    v_src[it] = (unsigned)(vr * kRows + ((vp ^ swz_vt8(vr)) * 16));
  }
  int k_off[2][KS][2], v_off[DB][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row = 32 * t + r, chunk = 4 * ks + 2 * hh + c;
        k_off[t][ks][c] = row * D + ((chunk ^ swz_kt<D>(row)) * 16);
      }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = 32 * db + r, chunk = 2 * hh + c;
      v_off[db][c] = row * kRows + ((chunk ^ swz_vt8(row)) * 16);
    }

  auto run_block = [&](int qb) {
    const int q0 = qb * kQRows;
    const int qw = q0 + 32 * wid;  // this wave's 32 rows
    const bool active = qw < N;
    // key blocks of the workgroup (all waves load and wait on them) and of this wave
    const int nkb = CAUSAL ? min(p.nblk, (min(q0 + kQRows, N) - 1) / kRows + 1) : p.nblk;
    const int nkw = !active ? 0 : CAUSAL ? (qw + 31) / kRows + 1 : p.nblk;
    const int eq = active ? p.eq[((size_t)bs * p.heads + h) * p.nblk + qw / kRows] : 0;
    i32x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = active ? *(const i32x8*)(qhead + (size_t)(qw + r) * D + 64 * ks + 32 * hh) : i32x8{};
    // pinned here, before the key loop, so the loads are not sunk into it
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[ks]));

    // copies of key block kb into buffer BUF: K (row-major) and V^T tiles, each wave its share
    auto issue_k = [&](auto bufc, int kb) {
      const __amdgpu_buffer_rsrc_t src = make_rsrc(khead + (size_t)kb * TILE, TILE);
      char* dst = kbuf(bufc) + wid * LOADS * 1024;
#pragma unroll
      for (int it = 0; it < LOADS; ++it) copy16_to_lds(src, k_src[it], dst + it * 1024);
    };
    auto issue_v = [&](auto bufc, int kb) {
      const __amdgpu_buffer_rsrc_t src = make_rsrc(vhead + (size_t)kb * TILE, TILE);
      char* dst = vbuf(bufc) + wid * LOADS * 1024;
#pragma unroll
      for (int it = 0; it < LOADS; ++it) copy16_to_lds(src, v_src[it], dst + it * 1024);
    };
    auto read8 = [](const char* base, int o0, int o1) {
      const u32x4 a = *(const u32x4*)(base + o0);
      const u32x4 b = *(const u32x4*)(base + o1);
      return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    };

    // running maximum (log2 units of the scaled score; P in (0, 1]), this lane's half of the
    // running row sum of P, and O^T
    float m = -1e30f, l = 0.f;
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

    // value 16t + i of a score block: S^T[key kb*64 + 32t + 8(i/4) + 4hh + i%4][query qw + r]
    auto edge = [&](int kb) { return (CAUSAL && kb * kRows + kRows - 1 > qw) || kb * kRows + kRows > N; };
    auto mask = [&](f32x16 (&s)[2], int kb) {
      const int q = qw + r;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * kRows + 32 * t + 8 * (i >> 2) + 4 * hh + (i & 3);
          if ((CAUSAL && key > q) || key >= N) s[t][i] = -INFINITY;
        }
    };
    // S^T = K Q^T of one block from K buffer BUF (the first block, before the loop)
    auto qk = [&](f32x16 (&s)[2], auto bufc) {
      const char* kb_ = kbuf(bufc);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        s[t] = mfma_f8(read8(kb_, k_off[t][0][0], k_off[t][0][1]), qf[0], f32x16{}, 127, 127);
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) s[t] = mfma_f8(read8(kb_, k_off[t][ks][0], k_off[t][ks][1]), qf[ks], s[t], 127, 127);
      }
    };
    // O^T += V^T P^T of the wave's last block, on its own
    auto pv_tail = [&](const i32x8& pb, auto bufc, int kb) {
      const char* vb_ = vbuf(bufc);
      const int sv = evp[kb] + 127;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        oacc[db] = mfma_f8(read8(vb_, v_off[db][0], v_off[db][1]), pb, oacc[db], sv, 127 - kPScaleLog2);
    };

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;

    // ---- step j (parity PH = j & 1) of a wave, for j < nkw: copies K(j+2) -> K buffer j&1
    // and V(j) -> V buffer j&1; forms S(j+1) = K(j+1) Q^T from K buffer !(j&1) on the matrix
    // core beside the softmax of block j (maximum, exponentials, sums, e4m3 codes of P(j)), then
    // O^T += V(j-1)^T P(j-1)^T from V buffer !(j&1). O is rescaled by the step's factor once
    // the P(j-1) product (formed against the previous maximum) is in. Past the last block the
    // K copies repeat it (that buffer is free and never read), so a step has no branches.
    //
    // The step is laid out as NSLOT slots of one MFMA each (the score MFMAs first), fenced by
    // scheduling barriers; each slot carries VPS probabilities' worth of VALU work (scale FMA,
    // exponential, sum, conversion) and the LDS operand reads of the MFMA two slots on.
    constexpr int NQK = 2 * KS;            // score MFMAs: two 32-key halves x head-dim k-steps
    constexpr int NSLOT = NQK + DB;        // + P V MFMAs
    constexpr int VPS = 32 / NSLOT;        // probabilities per slot (4 at d = 128, 8 at d = 64)
    constexpr int AH = 1;                  // operand reads, slots ahead of their MFMA
    static_assert(32 % NSLOT == 0, "slot plan");
    auto fma_slot = [](int v) { return v / VPS - 1 < -1 ? -1 : v / VPS - 1; };
    auto exp_slot = [](int v) { return v / VPS; };
    auto add_slot = [](int v) { return v / VPS + 1 < NSLOT ? v / VPS + 1 : NSLOT; };
    auto cvt_slot = [](int qd) { return (4 * qd + 3) / VPS + 1 < NSLOT ? (4 * qd + 3) / VPS + 1 : NSLOT; };
    auto read_slot = [](int u) { return u - AH < -1 ? -1 : u - AH; };

    f32x16 sA[2], sB[2];
    i32x8 pA = i32x8{}, pB = i32x8{};
    float cs_cur = 0.f;  // score factor of block j: scale log2(e) 2^(eq + ek[j])

    auto step = [&](auto phase, int j) {
      constexpr int PH = decltype(phase)::value;
      constexpr bool ODD = PH & 1;
      f32x16(&c)[2] = ODD ? sB : sA;  // S(j)
      f32x16(&n)[2] = ODD ? sA : sB;  // S(j+1)
      i32x8& pc = ODD ? pB : pA;      // P(j)
      i32x8& pp = ODD ? pA : pB;      // P(j-1)
      const char* kb_ = kbuf(std::integral_constant<int, PH + 1>());  // K(j+1)
      const char* vb_ = vbuf(std::integral_constant<int, PH + 1>());  // V(j-1)
      const int sv = j > 0 ? evp[j - 1] + 127 : 127;
      const int ek_next = ekp[min(j + 1, p.nblk - 1)];

      // preamble: mask, block maximum, new running maximum and factor
      if (edge(j)) mask(c, j);
      float mx;
      {
        float a0 = vmax3(c[0][0], c[0][1], c[0][2]), a1 = vmax3(c[1][0], c[1][1], c[1][2]);
#pragma unroll
        for (int i = 3; i < 15; i += 2) {
          a0 = vmax3(a0, c[0][i], c[0][i + 1]);
          a1 = vmax3(a1, c[1][i], c[1][i + 1]);
        }
        a0 = vmax3(a0, c[0][15], c[1][15]);
        mx = pair_max(fmaxf(a0, a1)) * cs_cur;
      }
      const float m_new = fmaxf(m, mx);
      const bool grow = wave_any(m_new > m);
      const float alpha = exp2_fast(m - m_new);
      l *= alpha;
      m = m_new;
      const float mm = m - (float)kPScaleLog2;  // codes are P * 2^8 = 2^(s cs - m + 8)
      const float cs = cs_cur;

      i32x8 op[NSLOT];
      float acc[4];
      uint32_t code[8];
      auto slot = [&](auto tc) {
        constexpr int t = decltype(tc)::value;
        // LDS operand reads
#pragma unroll
        for (int u = 0; u < NSLOT; ++u) {
          if (read_slot(u) == t) {
            if (u < NQK)
              op[u] = read8(kb_, k_off[u / KS][u % KS][0], k_off[u / KS][u % KS][1]);
            else
              op[u] = read8(vb_, v_off[u - NQK][0], v_off[u - NQK][1]);
          }
        }
        // the slot's MFMA
        if constexpr (t >= 0 && t < NQK) {
          constexpr int tt = t / KS, ks = t % KS;
          n[tt] = mfma_f8(op[t], qf[ks], ks == 0 ? f32x16{} : n[tt], 127, 127);
        } else if constexpr (t >= NQK && t < NSLOT) {
          constexpr int db = t - NQK;
          oacc[db] = mfma_f8(op[t], pp, oacc[db], sv, 127 - kPScaleLog2);
        }
        // VALU work on P(j)
#pragma unroll
        for (int v = 0; v < 32; ++v) {
          const int tt = v / 16, i = v % 16;
          if (fma_slot(v) == t) c[tt][i] = __builtin_fmaf(c[tt][i], cs, -mm);
          if (exp_slot(v) == t) c[tt][i] = exp2_fast(c[tt][i]);
          if (add_slot(v) == t) acc[v % 4] = v < 4 ? c[tt][i] : acc[v % 4] + c[tt][i];
        }
#pragma unroll
        for (int qd = 0; qd < 8; ++qd) {
          if (cvt_slot(qd) == t) {
            const int tt = qd / 4, i = 4 * (qd % 4);
            // (both halves of the register are written: its old contents, P(j-2)'s codes,
            // need no clearing)
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[tt][i], c[tt][i + 1], pc[qd], false);
            code[qd] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[tt][i + 2], c[tt][i + 3], w, true);
            asm volatile("" : "+v"(code[qd]));  // keeps the conversion in its slot
          }
        }
        // the sums stay in their slots too (sunk, they all landed in the next step's tail)
        if constexpr (t >= 1) asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
        __builtin_amdgcn_sched_barrier(0);
      };

      slot(std::integral_constant<int, -1>());
      issue_k(std::integral_constant<int, PH>(), min(j + 2, nkb - 1));
      issue_v(std::integral_constant<int, PH>(), j);
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, NSLOT + 1>(slot);

      // tail: the codes of P(j), the row sum, O rescaled past the P(j-1) product. S(j+1) is
      // pinned here: the IR optimisers would otherwise sink its MFMAs past the barrier, next
      // to their first use in the following step, out of the slots that overlap them with the
      // softmax.
      asm volatile("" : "+v"(n[0]), "+v"(n[1]));
#pragma unroll
      for (int qd = 0; qd < 8; ++qd) pc[qd] = (int)code[qd];
      l = __builtin_fmaf((acc[0] + acc[1]) + (acc[2] + acc[3]), 1.0f / (1 << kPScaleLog2), l);
      if (grow) {
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      }
      cs_cur = __builtin_amdgcn_ldexpf(p.c2, eq + ek_next);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of K(j+2), V(j) have landed
      __syncthreads();                // ... and everyone's; K(j), V(j-2) buffers are free
    };
    // a step of a wave past its last key block: its share of the copies, and the barrier
    auto idle_step = [&](auto phase, int j) {
      constexpr int PH = decltype(phase)::value;
      issue_k(std::integral_constant<int, PH>(), min(j + 2, nkb - 1));
      issue_v(std::integral_constant<int, PH>(), j);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    using F0 = std::integral_constant<int, 0>;
    using F1 = std::integral_constant<int, 1>;

    // ---- prologue: K(0) -> K buffer 0, K(1) -> K buffer 1; V buffer 1 is cleared, so the
    // first step's P V (zero codes of P(-1) times that buffer) adds exact zeros
    if (nkb > 0) {
      issue_k(B0(), 0);
      issue_k(B1(), min(1, nkb - 1));
      {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int o = tid * 16; o < TILE; o += 256 * 16) *(u32x4*)(v_lds1 + o) = z;
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (nkw > 0) {
        qk(sA, B0());
        cs_cur = __builtin_amdgcn_ldexpf(p.c2, eq + ekp[0]);
      }
      __syncthreads();  // every wave is done with K(0)

      int j = 0;
      if (nkw > 0) {
        for (; j + 1 < nkw; j += 2) {
          step(F0(), j);
          step(F1(), j + 1);
        }
        if (j < nkw) {
          step(F0(), j);
          ++j;
          pv_tail(pA, B0(), j - 1);  // last block even: its P in pA, its V^T in buffer 0
        } else {
          pv_tail(pB, B1(), j - 1);  // last block odd: its P in pB, its V^T in buffer 1
        }
      }
      for (; j < nkb; ++j) {
        if (j & 1)
          idle_step(F1(), j);
        else
          idle_step(F0(), j);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // no copy into LDS outlives the block

    // epilogue: O = O~ / l (bf16), LSE = (m + log2 l) ln 2
    const int q = qw + r;
    const float lt = pair_sum(l);
    if (active && q < N) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      uint16_t* og = p.o + (((size_t)bs * N + q) * p.heads + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x2 wv;
          wv[0] = pack_bf16x2(oacc[db][4 * i + 0] * inv, oacc[db][4 * i + 1] * inv);
          wv[1] = pack_bf16x2(oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv);
          *(u32x2*)(og + 32 * db + 8 * i + 4 * hh) = wv;
        }
      if (hh == 0) p.lse[((size_t)bs * p.heads + h) * N + q] = lt > 0.f ? (m + log2_fast(lt)) * kLn2 : -INFINITY;
    }
  };

  // causal: workgroup p takes query blocks nb-1-p and p, so all do the same work
  const int heavy = CAUSAL ? nb - 1 - pi : pi;
  const int passes = CAUSAL ? (pi < heavy ? 2 : pi == heavy ? 1 : 0) : (pi < nb ? 1 : 0);
  for (int pass = 0; pass < passes; ++pass) {
    if (pass) __syncthreads();  // every wave is done with the first block's tiles
    run_block(pass ? pi : heavy);
  }
}

template <int D>
hipError_t launch_d(const Fp8Args& a, hipStream_t stream) {
  const int nblk = (a.seqlen + kRows - 1) / kRows;
  const size_t Np = (size_t)nblk * kRows;
  uint8_t* ws = (uint8_t*)a.workspace;
  const Fp8Layout L = fp8_layout(a.batch, a.heads, a.kv_heads, a.seqlen, D);
  uint8_t* q8 = ws + L.q8;
  uint8_t* k8 = ws + L.k8;
  uint8_t* v8t = ws + L.v8t;
  int* eq = (int*)(ws + L.eq);
  int* ek = (int*)(ws + L.ek);
  int* ev = (int*)(ws + L.ev);
  (void)Np;
  const bool rot = a.signs != nullptr;
  {
    const QuantArgs qa{(const uint16_t*)a.q, a.signs, q8, eq, a.heads, a.seqlen, nblk};
    const QuantArgs ka{(const uint16_t*)a.k, a.signs, k8, ek, a.kv_heads, a.seqlen, nblk};
    const QuantArgs va{(const uint16_t*)a.v, a.signs, v8t, ev, a.kv_heads, a.seqlen, nblk};
    const size_t nq = (size_t)a.batch * a.heads * nblk, nkv = (size_t)a.batch * a.kv_heads * nblk;
    if (nq + 2 * nkv > 0x7fffffffu) return hipErrorInvalidConfiguration;
    if (nq + 2 * nkv > 0) {
      if (rot)
        hipLaunchKernelGGL((fp8_quant_qkv_kernel<D, true>), dim3((unsigned)(nq + 2 * nkv)), dim3(256), 0, stream, qa, ka, va, (int)nkv);
      else
        hipLaunchKernelGGL((fp8_quant_qkv_kernel<D, false>), dim3((unsigned)(nq + 2 * nkv)), dim3(256), 0, stream, qa, ka, va, (int)nkv);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }

  AttnArgs p;
  p.q8 = q8;
  p.k8 = k8;
  p.v8t = v8t;
  p.eq = eq;
  p.ek = ek;
  p.ev = ev;
  p.o = (uint16_t*)a.o;
  p.lse = a.lse;
  p.heads = a.heads;
  p.kv_heads = a.kv_heads;
  p.group = a.heads / a.kv_heads;
  p.seqlen = a.seqlen;
  p.nblk = nblk;
  const int nb = (a.seqlen + kQRows - 1) / kQRows;
  p.nqb = a.causal ? (nb + 1) / 2 : nb;
  p.c2 = a.scale * kLog2e / (rot ? (float)D : 1.f);
  const long long blocks = (long long)p.nqb * a.heads * a.batch;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.causal)
    hipLaunchKernelGGL((fwd_fp8_kernel<D, true>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<D, false>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

Fp8Layout fp8_layout(int B, int H, int Hkv, int N, int d) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t nblk = ((size_t)N + kRows - 1) / kRows;
  const size_t rows_q = (size_t)B * H * nblk * kRows, rows_kv = (size_t)B * Hkv * nblk * kRows;
  Fp8Layout L;
  L.q8 = 0;
  L.k8 = up(L.q8 + rows_q * d);
  L.v8t = up(L.k8 + rows_kv * d);
  L.eq = up(L.v8t + rows_kv * d);
  L.ek = up(L.eq + (size_t)B * H * nblk * sizeof(int));
  L.ev = up(L.ek + (size_t)B * Hkv * nblk * sizeof(int));
  L.total = up(L.ev + (size_t)B * Hkv * nblk * sizeof(int));
  return L;
}

hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  if (a.head_dim == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
