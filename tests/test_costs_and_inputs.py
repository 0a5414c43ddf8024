"""Host-side accounting pinned to the figures the pages print, and the seeded inputs."""
import json
import math
import os

import numpy as np

from io_aware_softmax_03_amd import costs
import synth

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_naive_matrix_size():
    g = G["naive_score_matrix"]
    entries, nbytes = costs.naive_score_matrix(g["n"], g["elem_bytes"])
    assert entries == g["entries_approx"] and nbytes == g["bytes_approx"]
    g = G["score_floats_32k"]
    assert abs(costs.naive_score_matrix(g["n"])[0] / g["floats_approx"] - 1) < 0.08


def test_fa1_idle_fraction():
    g = G["fa1_idle"]
    blocks = costs.fa1_grid_blocks(g["batch"], g["heads"])
    assert blocks == g["blocks"]
    assert round(costs.idle_fraction(blocks, g["n_sm"]), 2) == g["idle_fraction_approx"]


def test_fa2_grid():
    g = G["fa2_grid"]
    blocks = costs.fwd_grid_blocks(g["batch"], g["heads"], g["seq"], g["block_rows"])
    assert blocks == g["blocks"] == g["query_blocks"] * g["batch_heads"]
    assert round(blocks / g["n_sm"]) == g["fills_approx"]


def test_non_matmul_share():
    g = G["non_matmul_share"]
    r64 = costs.non_matmul_time_ratio(64, g["ops_per_score"], g["penalty"])
    r128 = costs.non_matmul_time_ratio(128, g["ops_per_score"], g["penalty"])
    assert round(r64, 2) == g["ratio_d64_approx"] and round(r128, 2) == g["ratio_d128_approx"]


def test_exp_vs_matmul():
    g = G["exp_vs_matmul_h100"]
    assert 4 * g["d"] == g["matmul_flops_per_score"]
    assert abs(g["matmul_tflops"] / g["sfu_tflops"] / g["rate_ratio_approx"] - 1) < 0.02
    r = costs.exp_to_matmul_time(g["d"], g["matmul_tflops"], g["sfu_tflops"])
    assert abs(r - g["exp_time_over_matmul_time_approx"]) < 0.01


def test_varlen_padding_cost():
    g = G["varlen_padding"]
    padded, useful = costs.padded_and_useful_scores(g["lengths"])
    assert padded == g["padded_scores_approx"]
    assert useful == 10_009_216 and round(useful / 1e6) * 1e6 == g["useful_scores_approx"]


def test_flop_conventions():
    # causal forward at B=2, H=16, N=8192, d=128 is 4*B*H*N^2*d/2
    assert costs.fwd_flops(2, 16, 8192, 128, True) == 4 * 2 * 16 * 8192 ** 2 * 128 / 2
    assert costs.bwd_flops(4, 16, 4096, 128, True) == 2.5 * costs.fwd_flops(4, 16, 4096, 128, True)
    assert costs.varlen_fwd_flops([10, 20], 2, 64, False) == 4 * 2 * 64 * (100 + 400)
    # 128x128 tiles of a causal 8192 square: 64*65/2 visible tiles
    assert costs.causal_tiles_visited(8192, 8192, 128, 128) == 64 * 65 // 2


def test_bf16_rounding_and_widening():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.1415926], dtype=np.float32)
    bits = synth.bf16_bits_from_f32(x)
    back = synth.f32_from_bf16_bits(bits)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1; 1 + 3*2^-8 -> 1 + 2^-6
    assert back.tolist()[:4] == [1.0, 1.0, 1.0 + 2 ** -6, -2.5]
    assert abs(back[4] - 3.140625) == 0.0
    # widening is exact: re-rounding the widened values changes nothing
    assert np.array_equal(synth.bf16_bits_from_f32(back), bits)


def test_per_slice_seeding():
    a = synth.bnhd_tensor(5, synth.TENSOR_K, 2, 6, 3, 4, dtype="f32")
    s = synth.normal_slice(5, synth.TENSOR_K, 1, 2, (6, 4))
    assert np.array_equal(a[1, :, 2, :], s)
    lengths = synth.varlen_lengths(3, 16, 128, 4096)
    assert lengths.min() >= 128 and lengths.max() <= 4096 and len(lengths) == 16
