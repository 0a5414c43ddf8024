"""Work and traffic accounting for the attention entry points (host-side arithmetic only).

These are the conventions the bench reports against and the figures the pages
derive on paper; tests pin each against the numbers the pages print.
"""
from __future__ import annotations

import math


def fwd_flops(B, H, N, d, causal):
    """Forward FLOPs by convention: two products of 2*N*N*d each per head, halved when causal.

    Per tile the two products cost 4*Br*Bc*d ("FlashAttention-2 and -3",
    "Fewer non-matmul FLOPs" and "FlashAttention-3, built for asynchrony").
    """
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def varlen_fwd_flops(lengths, H, d, causal):
    """Packed forward: useful work is the sum of per-sequence squares ("Variable-length batches")."""
    f = sum(4.0 * H * L * L * d for L in lengths)
    return f / 2 if causal else f


def bwd_flops(B, H, N, d, causal):
    """Backward FLOPs by the stated convention: five products, 2.5x the forward."""
    return 2.5 * fwd_flops(B, H, N, d, causal)


def decode_flops(B, H, L, d):
    return 4.0 * B * H * L * d


def decode_bytes(B, H, L, d, elem_bytes=2):
    """Compulsory HBM bytes of one decode step: K and V caches read once, plus q and o."""
    return 2.0 * B * L * H * d * elem_bytes + 2.0 * B * H * d * elem_bytes


def decode_paged_bytes(seqlens, H, d, elem_bytes=2, table_bytes=0):
    """Compulsory HBM bytes of one paged decode step: each sequence's valid K and V tokens
    read once, plus q and o, plus the block-table entries read ("Paged KV caches, a
    preview of serving": the gather touches only the pages a sequence owns)."""
    seqlens = list(seqlens)
    tokens = sum(seqlens)
    B = len(seqlens)
    return 2.0 * tokens * H * d * elem_bytes + 2.0 * B * H * d * elem_bytes + table_bytes


def fwd_compulsory_bytes(B, H, N, d, elem_bytes=2):
    """Q, K, V read once, O written once, fp32 LSE written once."""
    return 4.0 * B * N * H * d * elem_bytes + 4.0 * B * H * N


def fwd_grid_blocks(B, H, N, block_rows):
    """FlashAttention-2 launch grid: (query blocks) x (batch * heads)
    ("Parallelism over the sequence")."""
    return math.ceil(N / block_rows) * B * H


def fa1_grid_blocks(B, H):
    """FlashAttention-1 launch grid: one block per (sequence, head) ("three leaks")."""
    return B * H


def idle_fraction(blocks, n_units):
    """Fraction of compute units left idle when blocks < units, one block per unit."""
    return max(0.0, 1.0 - blocks / n_units)


def non_matmul_time_ratio(d, ops_per_score=5, penalty=16):
    """Non-matmul time relative to matmul time per tile:
    penalty * ops * Br*Bc / (4*Br*Bc*d) = penalty*ops/(4d)  ("Fewer non-matmul FLOPs")."""
    return penalty * ops_per_score / (4.0 * d)


def exp_to_matmul_time(d, matmul_rate, exp_rate):
    """Time of the Br*Bc exponentials relative to the 4*Br*Bc*d matmul FLOPs of one tile,
    each at its own unit's rate ("FlashAttention-3, built for asynchrony")."""
    return (1.0 / exp_rate) / (4.0 * d / matmul_rate)


def padded_and_useful_scores(lengths):
    """Scores per head with padding to the longest sequence, and the useful ones."""
    lengths = list(lengths)
    return len(lengths) * max(lengths) ** 2, sum(L * L for L in lengths)


def naive_score_matrix(n, elem_bytes=2):
    """Entries and bytes of one n x n score matrix (naive attention materialises it)."""
    return n * n, n * n * elem_bytes


def causal_tiles_visited(n_rows, n_cols, block_rows, block_cols):
    """Number of (query block, key block) tiles with at least one visible entry
    under the top-left causal mask; tiles above the diagonal are skipped."""
    count = 0
    for i in range(math.ceil(n_rows / block_rows)):
        last_row = min((i + 1) * block_rows, n_rows) - 1
        count += min(math.ceil(n_cols / block_cols), last_row // block_cols + 1)
    return count


def band_key_range(i, nq, nk, causal, window_left=-1, window_right=-1):
    """Visible keys [lo, hi] (inclusive; empty when lo > hi) of query i under the
    bottom-right alignment: query i stands at key position i + nk - nq; a sliding window
    keeps `window_left` keys before and `window_right` after it (negative: unlimited;
    causal: right = 0) ("Using it, the real way")."""
    pos = i + nk - nq
    right = 0 if causal else window_right
    hi = nk - 1 if right < 0 else min(nk - 1, pos + right)
    lo = 0 if window_left < 0 else max(0, pos - window_left)
    return lo, hi


def band_visible_pairs(nq, nk, causal, window_left=-1, window_right=-1):
    """Number of visible (query, key) pairs: the useful score entries of one head."""
    total = 0
    for i in range(nq):
        lo, hi = band_key_range(i, nq, nk, causal, window_left, window_right)
        total += max(0, hi - lo + 1)
    return total


def band_fwd_flops(B, H, nq, nk, d, causal, window_left=-1, window_right=-1):
    """Useful forward FLOPs of a banded forward: 4*d per visible pair (two products)."""
    return 4.0 * B * H * d * band_visible_pairs(nq, nk, causal, window_left, window_right)


def band_tiles_visited(nq, nk, block_q, block_k, causal, window_left=-1, window_right=-1):
    """(query block, key block) tiles holding at least one visible entry: per query block,
    the key blocks between its first row's lowest visible key and its last row's highest.
    Tiles outside are skipped ("a block mask of the tiles that are entirely masked")."""
    tiles = []
    for qb in range(math.ceil(nq / block_q)):
        first, last = qb * block_q, min((qb + 1) * block_q, nq) - 1
        ranges = [band_key_range(i, nq, nk, causal, window_left, window_right) for i in range(first, last + 1)]
        ranges = [(a, b) for a, b in ranges if a <= b]
        if not ranges:
            continue
        # the rows' key ranges move right with the row, overlapping: their union is one range
        lo, hi = min(a for a, _ in ranges), max(b for _, b in ranges)
        tiles.extend((qb, kb) for kb in range(lo // block_k, hi // block_k + 1))
    return tiles


def fwd_computed_scores(lengths, H, causal, rows_per_wave=32, keys_per_block=32):
    """(query, key) scores the bf16 forward kernel forms, masked ones included: per sequence
    and head, each wave of rows_per_wave query rows forms whole blocks of keys_per_block
    keys, up to the block holding its last row's last visible key (all blocks when not
    causal). Useful work is fewer: the diagonal blocks are partly masked."""
    total = 0
    for L in lengths:
        per_head = 0
        for qw in range(0, L, rows_per_wave):
            last = min(qw + rows_per_wave, L) - 1 if causal else L - 1
            per_head += (last // keys_per_block + 1) * keys_per_block * rows_per_wave
        total += per_head * H
    return total


# Per-SIMD issue rates of gfx950 from its unit counts (256 CUs x 4 SIMDs at 2.4 GHz): the
# fp32 vector peak of 157.3 TFLOP/s is 32 FMA lanes per clock per SIMD, so a wave64 VALU
# instruction takes 2 cycles; transcendental instructions (v_exp_f32) run at a quarter of
# that rate, 8 cycles; a 32x32x16 bf16 MFMA takes 32 cycles (1024 FLOP per clock).
VALU_CYCLES, TRANS_CYCLES, MFMA_32X32X16_CYCLES = 2.0, 8.0, 32.0
N_SIMD, CLOCK_HZ = 1024, 2.4e9


def valu_bound_seconds(scores, exp_per_score, other_valu_per_score):
    """Lower bound on a launch's time from its VALU work: per score, exp_per_score
    transcendental and other_valu_per_score other lane-operations, at the full-rate and
    quarter-rate VALU throughput of every SIMD at 2.4 GHz."""
    cycles = scores / 64.0 * (exp_per_score * TRANS_CYCLES + other_valu_per_score * VALU_CYCLES)
    return cycles / N_SIMD / CLOCK_HZ


def mfma_bound_seconds(scores, d, extra_mfma_fraction=0.0):
    """Lower bound on a launch's time from its matrix-core work: 4*d FLOP per formed score
    (S = Q K^T and O += P V), plus a fraction of extra MFMA time (e.g. row sums), at the
    dense bf16 peak."""
    return scores * 4.0 * d * (1.0 + extra_mfma_fraction) / (N_SIMD * 1024.0 * CLOCK_HZ)
