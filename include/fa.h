/*
 * fa.h — exact scaled-dot-product attention on MI355X (gfx950), FlashAttention style.
 *
 * What every call computes, per (batch, head):
 *     S = scale * Q K^T,  P = softmax_rows(S)  (masked entries excluded),  O = P V,
 *     LSE_i = ln sum_j exp(S_ij)               (natural log of the scaled scores)
 * without ever writing an N x N matrix to device memory: query row-blocks are
 * held on chip while key/value column-blocks stream past, and the softmax is
 * carried online (running maximum, running sum, unnormalised output rescaled
 * when the maximum moves, one division at the end).
 *   Definitions: "FlashAttention: IO-aware exact attention", sections
 *   "Tile decomposition" and "Online softmax"; "FlashAttention-2 and -3"
 *   (efficient-attention/flash-2-3), section "Fewer non-matmul FLOPs"
 *   (unnormalised accumulator, log-sum-exp kept for the backward pass).
 *
 * Conventions shared by every entry point
 *   Layout   Q, K, V, O, dO, dQ, dK, dV are contiguous [B, N, H, d] (the
 *            (batch, T, heads, d) layout of the flash-attn package, "Flash
 *            Attention and the Online-Softmax Trick" §7). Packed variable-length
 *            tensors are [total_tokens, H, d]. LSE is fp32 [B, H, N]
 *            ([H, total_tokens] for varlen, [B, H] for decode).
 *   Heads    the forward and decode calls take Hkv key-value heads for H query
 *            heads, Hkv dividing H (grouped-query attention: "FlashAttention-2
 *            and -3", section "Using it, the real way", fewer key-value heads
 *            shared in groups without copying K and V). Query heads form Hkv
 *            consecutive groups of H / Hkv; group j reads key-value head j. K
 *            and V then have Hkv in place of H in their shapes. Hkv = H is
 *            ordinary multi-head attention.
 *   Causal   query i sees key j when j <= i, both counted from the start of
 *            the sequence. For the square shapes accepted here this is both the
 *            top-left and the bottom-right alignment described in
 *            "FlashAttention-2 and -3", section "Using it, the real way".
 *   Scale    multiplies Q K^T before the softmax; callers normally pass
 *            1/sqrt(d). Must be finite and > 0.
 *   dtype    FA_DTYPE_BF16: bf16 inputs, fp32 accumulation, O rounded once to
 *            bf16 (round to nearest even). FA_DTYPE_F32: fp32 throughout.
 *   Head dim d must be 64 or 128.
 *   Memory   every pointer is device memory owned by the caller; the library
 *            allocates nothing and keeps no state between calls. Workspaces
 *            are passed in after a size query. The one exception is
 *            fa_decode_noalloc, whose partials live in a fixed scratch array
 *            of the library (one per GPU, for the life of the process).
 *   Streams  `stream` is a hipStream_t (NULL = the default stream). Calls only
 *            enqueue kernels on that stream: no host synchronisation and no
 *            device-to-host copy. Results are ready when the stream is.
 *   Errors   arguments are checked on the host before any HIP call, so a bad
 *            call returns an error code without touching the device; there is
 *            never a fallback to another algorithm ("Using it, the real way":
 *            ask for the fused kernel and get an error rather than a slower
 *            path). A failed kernel launch returns FA_ERR_HIP.
 *   Sizes    element counts of every tensor must fit in int64; sequence
 *            lengths (and packed token counts) are at most 2^30.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,      /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,     /* a size is <= 0, too large, or inconsistent */
  FA_ERR_HEADDIM = -3,   /* d is not supported (supported: 64, 128) */
  FA_ERR_DTYPE = -4,     /* dtype not supported by this entry point */
  FA_ERR_WORKSPACE = -5, /* workspace missing or smaller than the size query returned */
  FA_ERR_ARG = -6,       /* other invalid argument (scale, num_splits, flags) */
  FA_ERR_HIP = -7,       /* the HIP runtime reported an error launching a kernel */
  FA_ERR_SCRATCH = -8    /* too large for the fixed scratch of fa_decode_noalloc */
} fa_status;

typedef enum { FA_DTYPE_F32 = 0, FA_DTYPE_BF16 = 1 } fa_dtype;

/* Human-readable text for a status code (static storage; never NULL). */
const char* fa_strerror(int status);

/*
 * fa_fwd — dense forward.
 *   q        [B, N, H, d] of `dtype` (read only)
 *   k, v     [B, N, Hkv, d] of `dtype` (read only)
 *   o        [B, N, H, d] of `dtype` (written)
 *   lse      fp32 [B, H, N] (written): LSE_i = m_i + ln l_i, kept for fa_bwd
 *            ("Fewer non-matmul FLOPs"). May not be NULL.
 *   causal   0 or 1.
 * Key/value blocks that lie entirely above the causal diagonal are never
 * visited ("Fewer non-matmul FLOPs": skipping the masked causal tiles). The
 * launch grid is (query blocks) x (batch * heads) ("Parallelism over the
 * sequence").
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Hkv, int N, int d, float scale, int causal, int dtype, void* stream);

/*
 * fa_fwd_window — forward with Nq queries against Nk keys and an optional
 * sliding window ("FlashAttention-2 and -3", section "Using it, the real way":
 * causal aligned bottom-right, as chunked prefill and decoding with a cache
 * need; kernels support sliding windows natively; a block mask skips the tiles
 * with no visible entry).
 *   q, o          [B, Nq, H, d];  k, v  [B, Nk, Hkv, d];  lse  fp32 [B, H, Nq]
 *   Query i stands at key position p_i = i + Nk - Nq. Key j is visible when
 *     p_i - window_left <= j    (window_left >= 0; -1: no lower bound)
 *     j <= p_i + window_right   (window_right >= 0; -1: no upper bound)
 *   causal = 1 sets the upper bound to p_i (window_right must be -1 or 0). With
 *   Nq = Nk, causal and no window this is fa_fwd's causal mask; a 64-key causal
 *   window shows each query itself and the 64 keys before it.
 *   A query with no visible key (e.g. i < Nq - Nk under causal) gets O = 0 and
 *   LSE = -inf. Per 256-query block only the 32-key blocks between the first
 *   row's lowest and the last row's highest visible key are read.
 *   Nq, Nk <= 2^30; Nk may be 0 (every row then has no visible key).
 */
int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
                  int causal, int window_left, int window_right, int dtype, void* stream);

/*
 * fa_fwd_varlen — forward over sequences packed end to end without padding
 * ("FlashAttention-2 and -3", section "Variable-length batches without padding").
 *   q, o         [total_tokens, H, d]
 *   k, v         [total_tokens, Hkv, d]
 *   lse          fp32 [H, total_tokens]
 *   cu_seqlens   device int32 [num_seqs + 1]: cu_seqlens[0] = 0, nondecreasing,
 *                cu_seqlens[num_seqs] = total_tokens. Sequence s occupies rows
 *                cu_seqlens[s] .. cu_seqlens[s+1]-1. The offsets live on the
 *                device and the host does not read them (the Python binding
 *                checks a host copy before the call). Offsets that break the
 *                contract cannot make the kernels access memory outside the
 *                tensors: sequence s is taken as rows max(0, min(c_s, T)) ..
 *                min(max(c_{s+1}, that start), T) - 1 (T = total_tokens);
 *                rows in no such range are not written.
 *   max_seqlen   the longest sequence length; sizes the launch grid. A sequence
 *                longer than max_seqlen is still computed in full (its extra
 *                query blocks are taken by the same workgroups, more slowly).
 * Attention never crosses a sequence boundary (block-diagonal mask); causal is
 * counted within each sequence. Empty sequences are allowed.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens, int num_seqs, int total_tokens, int max_seqlen,
                  int H, int Hkv, int d, float scale, int causal, int dtype, void* stream);

/* Bytes of workspace fa_bwd needs: the row statistic D = rowsum(dO * O) and the LSE in base 2
 * (LSE * log2(e)), each fp32 [B, H, N]. */
size_t fa_bwd_workspace_bytes(int B, int H, int N);

/*
 * fa_bwd — backward by recomputation ("FlashAttention: IO-aware exact
 * attention", "Tile decomposition", last paragraph; "FlashAttention-2 and -3",
 * "Parallelism over the sequence", last paragraph).
 *   q, dout         [B, N, H, d] bf16, the forward's query and the upstream gradient
 *   k, v            [B, N, Hkv, d] bf16, the forward's keys and values
 *   o, lse          the forward's outputs for the same inputs (fa_fwd)
 *   dq              fp32 [B, N, H, d] (written): each element written once, by a pass over
 *                   query blocks that recomputes S and dP (the page accumulates dQ across
 *                   key blocks with atomics instead; the result is the same sum).
 *   dk, dv          fp32 [B, N, Hkv, d] (written). With Hkv = H each element is written
 *                   once per key block; with Hkv < H a shared head receives the sum of
 *                   its group's gradients (cleared by the call, then added with device
 *                   atomics).
 *   workspace       >= fa_bwd_workspace_bytes(B, H, N) bytes of device memory.
 * Probabilities are recomputed from Q, K and the saved LSE as exp(s - LSE); the
 * gradient is dV = P^T dO, dS = P * (dO V^T - D), dQ = scale dS K, dK = scale dS^T Q.
 * Only FA_DTYPE_BF16 is accepted. With Hkv = H the outputs are the same bits run to
 * run; with Hkv < H the order of the atomic additions into dk, dv varies, so those
 * are reproducible to rounding, not bit for bit.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, float* dq, float* dk, float* dv,
           int B, int H, int Hkv, int N, int d, float scale, int causal, int dtype,
           void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace fa_fwd_fp8 needs: the e4m3 codes of Q, K and V (one byte per
 * element, rows padded to a multiple of 64) and one int32 exponent per 64-row block of
 * each. 0 for invalid sizes. */
size_t fa_fwd_fp8_workspace_bytes(int B, int H, int Hkv, int N, int d);

/*
 * fa_fwd_fp8 — forward attention computed in FP8 e4m3 ("FlashAttention-2 and -3",
 * section "FP8, and the outlier problem"), same inputs and outputs as fa_fwd with
 * dtype FA_DTYPE_BF16:
 *   q [B, N, H, d], k, v [B, N, Hkv, d] bf16; o [B, N, H, d] bf16; lse fp32 [B, H, N]
 *   signs     device fp32 [d] of +1/-1 (16-byte aligned), or NULL. Given, Q and K are rotated by
 *             R = H_d diag(signs) / sqrt(d) (incoherent processing: the scores are
 *             unchanged in exact arithmetic, outliers are spread over all coordinates).
 *   Each block of 64 rows of one head of Q, K and V gets its own power-of-two scale
 *   (block quantization); P is quantized to e4m3 before the second product; both
 *   products run on the FP8 matrix cores with fp32 accumulation; the softmax runs in
 *   fp32. O approximates exact attention to FP8 accuracy, not to bf16 accuracy.
 *   workspace  at least fa_fwd_fp8_workspace_bytes(B, H, Hkv, N, d) bytes, 256-byte
 *              aligned; overwritten. After the call it holds the quantized operands,
 *              with Np = N rounded up to a multiple of 64, nb = Np / 64 and each part
 *              starting at the next multiple of 256 bytes: Q codes [B, H, Np, d],
 *              K codes [B, Hkv, Np, d] (rotated when signs are given), V codes per
 *              64-key block transposed [B, Hkv, nb, d, 64] with slot s holding key
 *              32*((s>>4)&1) + 8*((s>>2)&3) + 4*(s>>5) + (s&3) of the block, then int32
 *              exponents [B, H, nb], [B, Hkv, nb], [B, Hkv, nb]: a block's values are
 *              its e4m3 codes (OCP, bias 7) times 2^exponent.
 * Causal is top-left (square). The call enqueues one quantization launch (Q, K and V) and
 * the attention launch.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, const float* signs, void* o, float* lse,
               int B, int H, int Hkv, int N, int d, float scale, int causal,
               void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace fa_decode needs for `num_splits` partials per (batch, head):
 * fp32 running max, running sum and a d-wide partial output for each. */
size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits);

/*
 * fa_decode — one query token per (batch, head) against a contiguous KV cache,
 * split over the keys (Flash-Decoding; "FlashAttention-2 and -3", section
 * "Decoding needs a different split").
 *   q          [B, H, d]
 *   k_cache,
 *   v_cache    [B, L, Hkv, d]
 *   o          [B, H, d] (written)
 *   lse        fp32 [B, H] (written) or NULL
 *   num_splits 1 .. 1024 chunks of ceil(L / num_splits) keys. Each chunk yields
 *              its running max, sum and partial output; a second small kernel
 *              merges them with log-sum-exp weights (each chunk weighted by its
 *              softmax mass). The merged result does not depend on num_splits
 *              beyond rounding.
 * The new token sees every cached key (no mask). Only FA_DTYPE_BF16.
 * With Hkv < H one workgroup serves all query heads of a key-value head, so
 * each cached key and value is read from memory once for the whole group.
 */
int fa_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
              int B, int H, int Hkv, int L, int d, float scale, int num_splits, int dtype,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_noalloc — fa_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments, layouts and results as fa_decode,
 * without the workspace arguments. The chunk partials go to a fixed 64 MiB
 * scratch array inside the library instead: one per GPU, held from the first
 * call on that GPU until the process ends. The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); its first call on a device
 * looks the array's address up once (hipGetSymbolAddress) and caches it.
 *   Limit   B * H * num_splits * (d + 2) * 4 bytes (fa_decode_workspace_bytes)
 *           must be at most 64 MiB, else FA_ERR_SCRATCH: e.g. B = 64, H = 32,
 *           d = 128 takes up to 63 splits.
 *   Sharing every call on one GPU uses the same array and leaves the last call's
 *           partials in it (no call needs it cleared: every partial is written
 *           before it is read). Calls that overlap on one GPU (other streams,
 *           other host threads) race on it: serialise them.
 */
int fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                      int B, int H, int Hkv, int L, int d, float scale, int num_splits, int dtype,
                      void* stream);

/*
 * fa_decode_paged — fa_decode over a paged KV cache ("FlashAttention-2 and -3",
 * section "Paged KV caches, a preview of serving"): keys and values live in a
 * pool of fixed-size pages, and a per-sequence block table maps logical block
 * j (tokens j*page_size .. (j+1)*page_size - 1) to a physical page. The kernel
 * gathers whole pages; the split over keys and the merge are those of
 * fa_decode, with each sequence cut into num_splits chunks of
 * ceil(seqlens[b] / num_splits) keys.
 *   q           [B, H, d]
 *   k_pages,
 *   v_pages     [num_pages, page_size, Hkv, d]
 *   block_table int32 [B, max_pages], row-major; entry j of row b is the page
 *               holding tokens j*page_size .. of sequence b. Entries past the
 *               sequence's last page are never read.
 *   seqlens     int32 [B]: tokens cached for each sequence, 0 .. max_pages *
 *               page_size. Slots past seqlens[b] in its last page are ignored.
 *   o           [B, H, d] (written); a sequence with no tokens gets zeros
 *   lse         fp32 [B, H] (written) or NULL; -inf for a sequence with no tokens
 *   page_size   a power of two, 1 .. 1024; max_pages * page_size <= 2^30
 *   workspace   at least fa_decode_workspace_bytes(B, H, d, num_splits) bytes
 * All pointers are device pointers; block_table and seqlens are read on the
 * device (4-byte aligned), the rest need 16-byte alignment. The kernel clamps
 * seqlens to [0, max_pages * page_size] and page ids to [0, num_pages - 1], so
 * bad table contents give wrong values, never reads outside the buffers; they
 * are not reported as errors. Only FA_DTYPE_BF16.
 */
int fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                    const int* block_table, const int* seqlens, void* o, float* lse,
                    int B, int H, int Hkv, int d, int page_size, int num_pages, int max_pages,
                    float scale, int num_splits, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
