// Host-side launch functions implemented in the kernel sources and called by the C ABI
// after argument validation. Each returns hipSuccess or the launch error.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int* cu_seqlens;  // NULL for the dense [B, N, H, d] layout
  int batch;              // dense: B; packed: number of sequences
  int heads;
  int kv_heads;           // K and V heads; divides heads (query head h reads h / (heads / kv_heads))
  int seqlen;             // dense: N; packed: max_seqlen (sizes the grid)
  int total_rows;         // dense: N; packed: total_tokens (LSE row stride)
  int head_dim;
  float scale;
  // Masking, bottom-right aligned: query i sees key j when i + lo_off <= j and, if banded,
  // j <= i + hi_off. Causal square attention: banded, hi_off = 0, lo_off = kNoLowerBound.
  int seqlen_k;  // dense: Nk (keys per sequence); packed: unused
  bool banded;
  int lo_off, hi_off;
};

// no lower bound: below -(every key position) for any length the entry points accept
constexpr int kNoLowerBound = -(1 << 30);

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  float* dq;
  float* dk;
  float* dv;
  float* delta;  // workspace: D [B, H, N], then LSE * log2(e) [B, H, N]
  int batch, heads, kv_heads, seqlen, head_dim;  // K, V, dK, dV have kv_heads heads
  float scale;
  bool causal;
};

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  void* o;
  float* lse;       // may be NULL
  float* partials;  // workspace: [B, H, S] max, [B, H, S] sum, [B, H, S, d] output
  int batch, heads, kv_heads, cache_len, head_dim, num_splits;
  float scale;
  // paged cache (block_table != NULL): caches are page pools [num_pages, page_size, Hkv, d],
  // block_table [B, max_pages] int32, seqlens [B] int32 (cache_len unused)
  const int* block_table;
  const int* seqlens;
  int page_size, num_pages, max_pages;
};

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);

// Fixed device scratch of the allocation-free decode (fa_decode_noalloc): bytes, and its
// address on the current device (looked up once per device, then cached).
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
hipError_t decode_scratch(void** ptr);

// FP8 forward: bf16 Q, K, V are quantized into the workspace, then attended in e4m3.
struct Fp8Args {
  const void* q;       // bf16 [B, N, H, d]
  const void* k;       // bf16 [B, N, Hkv, d]
  const void* v;
  const float* signs;  // [d] of +-1: rotate Q and K; NULL: no rotation
  void* o;             // bf16 [B, N, H, d]
  float* lse;          // [B, H, N]
  void* workspace;     // fp8_layout(...).total bytes, 256-byte aligned
  int batch, heads, kv_heads, seqlen, head_dim;
  float scale;
  bool causal;
};

// byte offsets inside the FP8 workspace: codes of Q [B, H, Np, d], K [B, Hkv, Np, d],
// transposed V blocks [B, Hkv, Np / 64, d, 64], then int32 exponents per 64-row block
struct Fp8Layout {
  size_t q8, k8, v8t, eq, ek, ev, total;
};
Fp8Layout fp8_layout(int B, int H, int Hkv, int N, int d);

hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream);

}  // namespace fa
