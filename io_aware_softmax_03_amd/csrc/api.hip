// C ABI of the attention library: argument validation on the host, then kernel launches
// on the caller's stream. Every check happens before the first HIP call, so invalid calls
// return an error code without touching the device; there is no fallback path.
#include <math.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "fa_launch.hpp"

namespace {

constexpr long long kMaxElems = 1LL << 62;
constexpr int kMaxSplits = 1024;
constexpr int kMaxPageSize = 1024;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
// grouped-query attention: Hkv key-value heads shared by groups of H / Hkv query heads
bool heads_ok(int H, int Hkv) { return H > 0 && Hkv > 0 && Hkv <= H && H % Hkv == 0; }
bool head_dim_ok(int d) { return d == 64 || d == 128; }
// Checked on the bit pattern: this file is built with NaNs assumed absent, which lets the
// compiler drop floating-point NaN tests.
bool scale_ok(float s) {
  const uint32_t b = __builtin_bit_cast(uint32_t, s);
  const uint32_t exp_bits = (b >> 23) & 0xffu;
  return (b >> 31) == 0u && exp_bits != 0xffu && (b & 0x7fffffffu) != 0u;  // positive, finite, non-zero
}

int fits(long long a, long long b, long long c, long long d) {
  // a*b*c*d <= kMaxElems for non-negative factors
  long long x = a;
  for (long long f : {b, c, d}) {
    if (f != 0 && x > kMaxElems / f) return 0;
    x *= f;
  }
  return 1;
}

int from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// longest query or key sequence the forward accepts: keeps every key position plus a mask
// offset inside int32
constexpr long long kMaxSeq = 1LL << 30;

long long clamp_off(long long x) { return x < -kMaxSeq ? -kMaxSeq : (x > kMaxSeq ? kMaxSeq : x); }

// Forward launch arguments. Masking is bottom-right aligned: query i sits at key position
// i + nk - nq; a window keeps `left` keys before it and `right` after (-1: unlimited), and
// causal means right = 0.
fa::FwdArgs fwd_args(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu,
                     int batch, int H, int Hkv, int nq, int total_rows, int nk, int d, float scale,
                     bool causal, int left, int right) {
  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.cu_seqlens = cu;
  a.batch = batch;
  a.heads = H;
  a.kv_heads = Hkv;
  a.seqlen = nq;
  a.total_rows = total_rows;
  a.head_dim = d;
  a.scale = scale;
  a.seqlen_k = nk;
  const long long off = (long long)nk - nq;
  const int r = causal ? 0 : right;
  a.banded = r >= 0;
  a.hi_off = a.banded ? (int)clamp_off(off + r) : 0;
  a.lo_off = left >= 0 ? (int)clamp_off(off - left) : fa::kNoLowerBound;
  return a;
}

}  // namespace

extern "C" {

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid or inconsistent sizes";
    case FA_ERR_HEADDIM: return "unsupported head dimension (supported: 64, 128)";
    case FA_ERR_DTYPE: return "unsupported dtype for this entry point";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_ARG: return "invalid argument (scale, flag, split count or pointer alignment)";
    case FA_ERR_HIP: return "HIP runtime error while launching a kernel";
    case FA_ERR_SCRATCH:
      return "problem too large for the fixed scratch of the allocation-free entry point (64 MiB)";
    default: return "unknown status";
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
           int d, float scale, int causal, int dtype, void* stream) {
  if (B < 0 || N < 0 || N > kMaxSeq || !heads_ok(H, Hkv)) return FA_ERR_SHAPE;
  if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F32) return FA_ERR_DTYPE;
  if (!scale_ok(scale) || (causal != 0 && causal != 1)) return FA_ERR_ARG;
  if (!fits(B, N, H, d)) return FA_ERR_SHAPE;
  if (B == 0 || N == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ARG;
  const fa::FwdArgs a = fwd_args(q, k, v, o, lse, nullptr, B, H, Hkv, N, N, N, d, scale, causal != 0, -1, -1);
  hipStream_t s = (hipStream_t)stream;
  return from_hip(dtype == FA_DTYPE_BF16 ? fa::launch_fwd_bf16(a, s) : fa::launch_fwd_f32(a, s));
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens,
                  int num_seqs, int total_tokens, int max_seqlen, int H, int Hkv, int d, float scale,
                  int causal, int dtype, void* stream) {
  if (num_seqs < 0 || total_tokens < 0 || max_seqlen < 0 || !heads_ok(H, Hkv)) return FA_ERR_SHAPE;
  if (total_tokens > kMaxSeq) return FA_ERR_SHAPE;
  if (max_seqlen > total_tokens) return FA_ERR_SHAPE;
  if (total_tokens > 0 && (max_seqlen == 0 || num_seqs == 0)) return FA_ERR_SHAPE;
  if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F32) return FA_ERR_DTYPE;
  if (!scale_ok(scale) || (causal != 0 && causal != 1)) return FA_ERR_ARG;
  if (!fits(total_tokens, H, d, 1)) return FA_ERR_SHAPE;
  if (total_tokens == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse || !cu_seqlens) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ARG;
  // queries and keys of a packed sequence coincide, so bottom-right and top-left agree
  const fa::FwdArgs a = fwd_args(q, k, v, o, lse, cu_seqlens, num_seqs, H, Hkv, max_seqlen, total_tokens,
                                 max_seqlen, d, scale, causal != 0, -1, -1);
  hipStream_t s = (hipStream_t)stream;
  return from_hip(dtype == FA_DTYPE_BF16 ? fa::launch_fwd_bf16(a, s) : fa::launch_fwd_f32(a, s));
}

int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                  int Nq, int Nk, int d, float scale, int causal, int window_left, int window_right,
                  int dtype, void* stream) {
  if (B < 0 || Nq < 0 || Nk < 0 || Nq > kMaxSeq || Nk > kMaxSeq || !heads_ok(H, Hkv)) return FA_ERR_SHAPE;
  if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F32) return FA_ERR_DTYPE;
  if (!scale_ok(scale) || (causal != 0 && causal != 1)) return FA_ERR_ARG;
  if (window_left < -1 || window_right < -1 || (causal && window_right > 0)) return FA_ERR_ARG;
  if (!fits(B, Nq, H, d) || !fits(B, Nk, Hkv, d)) return FA_ERR_SHAPE;
  if (B == 0 || Nq == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ARG;
  const fa::FwdArgs a =
      fwd_args(q, k, v, o, lse, nullptr, B, H, Hkv, Nq, Nq, Nk, d, scale, causal != 0, window_left, window_right);
  hipStream_t s = (hipStream_t)stream;
  return from_hip(dtype == FA_DTYPE_BF16 ? fa::launch_fwd_bf16(a, s) : fa::launch_fwd_f32(a, s));
}

size_t fa_fwd_fp8_workspace_bytes(int B, int H, int Hkv, int N, int d) {
  if (B < 0 || N < 0 || !heads_ok(H, Hkv) || !head_dim_ok(d) || N > kMaxSeq) return 0;
  return fa::fp8_layout(B, H, Hkv, N, d).total;
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, const float* signs, void* o, float* lse, int B,
               int H, int Hkv, int N, int d, float scale, int causal, void* workspace, size_t workspace_bytes,
               void* stream) {
  if (B < 0 || N < 0 || N > kMaxSeq || !heads_ok(H, Hkv)) return FA_ERR_SHAPE;
  if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
  if (!scale_ok(scale) || (causal != 0 && causal != 1)) return FA_ERR_ARG;
  if (!fits(B, N, H, d)) return FA_ERR_SHAPE;
  if (B == 0 || N == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!workspace || workspace_bytes < fa_fwd_fp8_workspace_bytes(B, H, Hkv, N, d)) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      ((uintptr_t)workspace & 255u) != 0 || ((uintptr_t)signs & 15u) != 0)
    return FA_ERR_ARG;
  fa::Fp8Args a{q, k, v, signs, o, lse, workspace, B, H, Hkv, N, d, scale, causal != 0};
  return from_hip(fa::launch_fwd_fp8(a, (hipStream_t)stream));
}

size_t fa_bwd_workspace_bytes(int B, int H, int N) {
  if (B < 0 || H < 0 || N < 0) return 0;
  return 2 * (size_t)B * H * N * sizeof(float);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           float* dq, float* dk, float* dv, int B, int H, int Hkv, int N, int d, float scale, int causal,
           int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || N < 0 || N > kMaxSeq || !heads_ok(H, Hkv)) return FA_ERR_SHAPE;
  if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (!scale_ok(scale) || (causal != 0 && causal != 1)) return FA_ERR_ARG;
  if (!fits(B, N, H, d)) return FA_ERR_SHAPE;
  if (B == 0 || N == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(B, H, N)) return FA_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ARG;
  fa::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, (float*)workspace, B, H, Hkv, N, d, scale, causal != 0};
  return from_hip(fa::launch_bwd_bf16(a, (hipStream_t)stream));
}

size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits) {
  if (B < 0 || H < 0 || d < 0 || num_splits < 0) return 0;
  return (size_t)B * H * num_splits * (d + 2) * sizeof(float);
}

int fa_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B, int H,
              int Hkv, int L, int d, float scale, int num_splits, int dtype, void* workspace,
              size_t workspace_bytes, void* stream) {
  if (B < 0 || L <= 0 || !heads_ok(H, Hkv)) return FA_ERR_SHAPE;
  if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (!scale_ok(scale) || num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_ARG;
  if (!fits(B, L, H, d)) return FA_ERR_SHAPE;
  if (B == 0) return FA_OK;
  if (!q || !k_cache || !v_cache || !o) return FA_ERR_NULL;
  if (!workspace || workspace_bytes < fa_decode_workspace_bytes(B, H, d, num_splits)) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace)) return FA_ERR_ARG;
  fa::DecodeArgs a{q, k_cache, v_cache, o, lse, (float*)workspace, B, H, Hkv, L, d, num_splits, scale,
                   nullptr, nullptr, 0, 0, 0};
  return from_hip(fa::launch_decode_bf16(a, (hipStream_t)stream));
}

int fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B,
                      int H, int Hkv, int L, int d, float scale, int num_splits, int dtype, void* stream) {
  if (B < 0 || L <= 0 || !heads_ok(H, Hkv)) return FA_ERR_SHAPE;
  if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (!scale_ok(scale) || num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_ARG;
  if (!fits(B, L, H, d)) return FA_ERR_SHAPE;
  // the partials (fa_decode_workspace_bytes) must fit the fixed scratch; fits() bounds the
  // product first so the comparison cannot overflow
  if (!fits(B, H, num_splits, d + 2) ||
      (long long)B * H * num_splits * (d + 2) * (long long)sizeof(float) > (long long)fa::kDecodeScratchBytes)
    return FA_ERR_SCRATCH;
  if (B == 0) return FA_OK;
  if (!q || !k_cache || !v_cache || !o) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return FA_ERR_ARG;
  void* scratch = nullptr;
  const hipError_t e = fa::decode_scratch(&scratch);
  if (e != hipSuccess) return FA_ERR_HIP;
  fa::DecodeArgs a{q, k_cache, v_cache, o, lse, (float*)scratch, B, H, Hkv, L, d, num_splits, scale,
                   nullptr, nullptr, 0, 0, 0};
  return from_hip(fa::launch_decode_bf16(a, (hipStream_t)stream));
}

int fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int* block_table,
                    const int* seqlens, void* o, float* lse, int B, int H, int Hkv, int d, int page_size,
                    int num_pages, int max_pages, float scale, int num_splits, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (B < 0 || num_pages <= 0 || max_pages <= 0 || !heads_ok(H, Hkv)) return FA_ERR_SHAPE;
  if (page_size < 1 || page_size > kMaxPageSize || (page_size & (page_size - 1)) != 0) return FA_ERR_SHAPE;
  if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (!scale_ok(scale) || num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_ARG;
  // key positions (up to max_pages * page_size) stay below 2^30, so 32-bit key arithmetic
  // cannot overflow; pool rows and table offsets are formed in 64 bits
  if ((long long)max_pages * page_size > (1LL << 30) || (long long)num_pages * page_size > 0x7fffffffLL)
    return FA_ERR_SHAPE;
  if (!fits(1, (long long)num_pages * page_size, Hkv, d) || !fits(B, H, d, 1)) return FA_ERR_SHAPE;
  if (B == 0) return FA_OK;
  if (!q || !k_pages || !v_pages || !block_table || !seqlens || !o) return FA_ERR_NULL;
  if (!workspace || workspace_bytes < fa_decode_workspace_bytes(B, H, d, num_splits)) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(workspace) ||
      ((uintptr_t)block_table & 3u) != 0 || ((uintptr_t)seqlens & 3u) != 0)
    return FA_ERR_ARG;
  fa::DecodeArgs a{q, k_pages, v_pages, o, lse, (float*)workspace, B, H, Hkv, 0, d, num_splits, scale,
                   block_table, seqlens, page_size, num_pages, max_pages};
  return from_hip(fa::launch_decode_bf16(a, (hipStream_t)stream));
}

}  // extern "C"
