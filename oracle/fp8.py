"""FP8 forward attention emulated in float64, step by step (test infrastructure only).

Follows "FlashAttention-2 and -3", section "FP8, and the outlier problem": FP8 e4m3 has 4
exponent bits and 3 mantissa bits, largest value 448. Two tricks keep the error down:

1. Incoherent processing: Q and K are both multiplied by the same random orthogonal
   R = (Hadamard matrix) x (random +-1 diagonal), normalised; R R^T = I leaves the scores
   unchanged in exact arithmetic while spreading each outlier over all d coordinates.
2. Block quantization: one scale per block of Q, K and V (the blocks the kernel loads), so an
   outlier only inflates its own block's scale.

Then the tiled online softmax runs on the quantized operands; P is quantized to e4m3 too
before the second product (the page: the kernel reshuffles the registers holding P before
the second FP8 product).

Readings where the page is silent (each listed in the design notes):
* e4m3 is the OCP "fn" format: no infinities, subnormals down to 2^-9, largest 448;
  conversion rounds to nearest, ties to even, and saturates at +-448.
* R = H_d D / sqrt(d) (Sylvester Hadamard H_d, D = diag(signs)); a row x becomes x R. The
  rotated row that gets quantized is y = (x H_d) D, without the 1/sqrt(d): (qR)(kR)^T =
  y_q y_k^T / d, so 1/d joins the score scale (a power of two for d = 64, 128). x H_d is
  formed by the fast Walsh-Hadamard transform in float32, butterflies (a, b) -> (a + b,
  a - b) at strides 1, 2, 4, ..., d/2 in that order: a quantized code is an integer the
  float arithmetic decides, so the emulation takes that decision in the kernel's precision
  and order (IEEE float32 additions give the same result on both sides).
* A block's scale is the power of two 2^e with e the smallest integer such that
  amax <= 448 * 2^e (amax = 0: e = 0), so dividing by it is exact and the block's largest
  magnitude lands in (224, 448]. Blocks are 64 consecutive rows (tokens) of one head, for
  Q, K and V alike.
* P is quantized per key block as the online algorithm forms it: P~ = exp(S - m_new) in
  (0, 1] against the running maximum, times 2^8, rounded to e4m3, divided by 2^8. The row
  sum l and the LSE use the unquantized P~; O~ accumulates the quantized P times V. The
  scores, maxima and exponentials are float64 here; a kernel forming them in float32 can
  take the neighbouring code for a P~ * 2^8 within float32 rounding of a rounding midpoint.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_SUBNORMAL = 2.0 ** -9
P_SCALE_LOG2 = 8


def round_e4m3(x) -> np.ndarray:
    """Nearest OCP e4m3 value (ties to even significand), saturating at +-448, in float64.

    Normal values are 2^e (1 + m/8) for e in -6..8 (m <= 6 at e = 8); subnormals are
    2^-6 (m/8) = m 2^-9. In the binade [2^e, 2^(e+1)) the spacing is 2^(e-3); below 2^-6 it
    is 2^-9. Rounding x to that grid with ties to even is rounding x / spacing to the nearest
    even integer on ties."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    spacing = np.exp2(e - 3)
    r = np.round(a / spacing) * spacing    # np.round: ties to even, exact for these values
    r = np.minimum(r, E4M3_MAX)
    return np.sign(x) * r


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two): H_1 = [1],
    H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht_f32(x) -> np.ndarray:
    """x H_d for the rows of x (last axis, a power of two), in float32 butterflies at
    strides 1, 2, ..., d/2 (the fast Walsh-Hadamard transform)."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = 1
    while h < d:
        z = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = z[..., 0, :].copy(), z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(y.shape)
        h *= 2
    return y


def rotate_unnormalised(x, signs) -> np.ndarray:
    """(x H_d) D in float32: the rotated rows before quantization (x R times sqrt(d))."""
    return fwht_f32(x) * np.asarray(signs, dtype=np.float32)


def rotation(signs) -> np.ndarray:
    """R = H_d diag(signs) / sqrt(d), orthogonal for any +-1 signs."""
    s = np.asarray(signs, dtype=np.float64)
    d = s.shape[0]
    return hadamard(d) * s[None, :] / math.sqrt(d)


def scale_exponent(amax: float) -> int:
    """Smallest e with amax <= 448 * 2^e (0 for amax = 0). With amax = f 2^E, f in [0.5, 1)
    and 448 = 0.875 * 2^9: e = E - 9 when f <= 0.875, else E - 8."""
    if amax <= 0:
        return 0
    f, E = math.frexp(float(amax))
    return E - 9 if f <= 0.875 else E - 8


def block_exponents(x, block_rows: int) -> np.ndarray:
    """Power-of-two scale exponent per block of rows of a [rows, d] slice."""
    x = np.asarray(x, dtype=np.float64)
    nb = -(-x.shape[0] // block_rows)
    e = np.zeros(nb, dtype=np.int64)
    for b in range(nb):
        e[b] = scale_exponent(np.abs(x[b * block_rows:(b + 1) * block_rows]).max(initial=0.0))
    return e


def quantize_rows(x, block_rows: int):
    """Block quantization of a [rows, d] slice: returns (dequantized values, exponents).
    Each block's values are x / 2^e rounded to e4m3, times 2^e."""
    x = np.asarray(x, dtype=np.float64)
    e = block_exponents(x, block_rows)
    scale = np.repeat(np.exp2(e.astype(np.float64)), block_rows)[:x.shape[0]]
    return round_e4m3(x / scale[:, None]) * scale[:, None], e


def fp8_p_operand(P) -> np.ndarray:
    """The P operand of the second product: e4m3(P * 2^8) / 2^8 (module notes)."""
    return round_e4m3(np.asarray(P, dtype=np.float64) * 2.0 ** P_SCALE_LOG2) * 2.0 ** -P_SCALE_LOG2


def fp8_online_attention(q, k, v, scale, causal=False, block_cols=64, quantize_p=True, row_offset=0):
    """The tiled online softmax on (already quantized) operands, q [Nq, d], k, v [Nk, d],
    in float64: per key block of `block_cols` (counted from key 0), P~ = exp(S - m_new)
    against the running maximum, quantized as e4m3(P~ * 2^8) / 2^8 for the second product;
    the row sum and the LSE use P~ itself. Query row i sits at position row_offset + i
    (causal: it sees keys up to that position). Returns (O, LSE)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    nq, nk = q.shape[0], k.shape[0]
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    acc = np.zeros((nq, v.shape[1]))
    rows = row_offset + np.arange(nq)[:, None]
    for j0 in range(0, nk, block_cols):
        j1 = min(j0 + block_cols, nk)
        S = float(scale) * (q @ k[j0:j1].T)
        if causal:
            S = np.where(np.arange(j0, j1)[None, :] <= rows, S, -np.inf)
        m_new = np.maximum(m, S.max(axis=1))
        m_ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - m_ref), 0.0)
        P = np.exp(S - m_ref[:, None])
        Pq = fp8_p_operand(P) if quantize_p else P
        l = alpha * l + P.sum(axis=1)
        acc = alpha[:, None] * acc + Pq @ v[j0:j1]
        m = m_new
    O = acc / np.where(l > 0, l, 1.0)[:, None]
    lse = np.where(l > 0, np.where(np.isfinite(m), m, 0.0) + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return O, lse


def fp8_operands(q, k, v, scale, signs=None, block_rows=64, quantize=True):
    """Rotation (when `signs` is given) and block quantization of one head's q, k, v:
    returns the dequantized operands and the score scale (scale / d after a rotation)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    if signs is not None:
        # x R = (x H D) / sqrt(d): rotate without the normalisation, put 1/d on the scores
        d = q.shape[1]
        q = rotate_unnormalised(q, signs).astype(np.float64)
        k = rotate_unnormalised(k, signs).astype(np.float64)
        scale = float(scale) / d
    if quantize:
        q, _ = quantize_rows(q, block_rows)
        k, _ = quantize_rows(k, block_rows)
        v, _ = quantize_rows(v, block_rows)
    return q, k, v, scale


def fp8_attention_head(q, k, v, scale, causal=False, signs=None, block_rows=64, block_cols=64,
                       quantize=True):
    """FP8 forward for one (batch, head) slice, q [Nq, d], k, v [Nk, d]; returns (O, LSE).

    Steps: rotate q and k by R (when `signs` is given), block-quantize q, k and v, then the
    tiled online softmax over key blocks of `block_cols` with P quantized per block.
    ``quantize=False`` skips both quantizations (the same algorithm in float64), and
    block_rows >= the length gives one scale per tensor slice."""
    qh, kh, vh, sc = fp8_operands(q, k, v, scale, signs, block_rows, quantize)
    return fp8_online_attention(qh, kh, vh, sc, causal, block_cols, quantize)


def attn_fwd_fp8(q, k, v, scale, causal=False, signs=None, block_rows=64, block_cols=64, quantize=True):
    """Dense FP8 forward. q: [B, N, H, d]; k, v: [B, N, Hkv, d] (grouped as in attn_fwd).
    Returns O [B, N, H, d], LSE [B, H, N]."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, N, H, _ = q.shape
    Hkv = k.shape[2]
    O = np.empty(q.shape)
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            j = h // (H // Hkv)
            O[b, :, h], lse[b, h] = fp8_attention_head(q[b, :, h], k[b, :, j], v[b, :, j], scale, causal, signs,
                                                       block_rows, block_cols, quantize)
    return O, lse
