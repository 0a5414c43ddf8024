#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X; prints ONE JSON line on stdout.

Headline workload: causal bf16 forward, B=2, H=16, N=8192, d=128 (one step = one fa_fwd
call over that batch, inputs resident in device memory). Reported as TFLOP/s by the
convention 4*B*H*N^2*d/2 and as a fraction of the dense bf16 MFMA peak.

Also measured in the same run (field "extra"): the backward (B=4, H=16, N=4096, d=128,
causal), split-KV decode (B=64, H=32, L=32768, d=128, 64 splits), the same decode over a
paged cache (16-token pages, lengths 16384..32768), grouped-query decode (32 query heads
over 8 key-value heads), a chunked prefill (2048 queries on 16384 keys) and a 1024-key
sliding window (N=8192) through the banded forward, the FP8 forward on the headline shape,
the packed varlen
forward (16 sequences, H=32, d=64) and the fp32 forward (N=256, d=64); and the float64
CPU oracle timed on a bounded sample of the headline workload (field "cpu_baseline").

Every workload, the headline included, first runs its call untimed for about SETTLE_S seconds
(field "settle_s"; --settle-s), then its W warm-up calls, then the K timed ones: after a
switch between workloads the clock takes a fraction of a second to settle (the headline
measured right after the paged decode with W=5, K=20 ran 7% slower than after 1500 warm-up
calls; with the settle, within 1.5%).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (bf16 causal N=8192 d=128) and % of MFMA peak"
# 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP per clock per CU (the published 2.5 PFLOP/s)
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS  # dense e4m3 matrix-core peak (5.0 PFLOP/s)
SETTLE_S = 0.25  # seconds of untimed calls before each workload's warm-up
# other (non-transcendental) VALU lane-operations per formed score of the d=64 packed forward,
# from its SQ counters (SQ_INSTS_VALU - SQ_INSTS_VALU_TRANS_F32 per formed score x 64 lanes;
# profiles/fwd_bwd_counters.md)
VALU_OPS_PER_SCORE_D64 = 3.8
FWD_ROWS_PER_WAVE_D64 = 64  # the d=64 forward's waves own 64 query rows (two 32-row groups)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_causal_b2_h16_n8192_d128_traffic.json")
# the sources the forward kernel is compiled from (its file and the shared device header)
FWD_SOURCES = [os.path.join(ROOT, "io_aware_softmax_03_amd", "csrc", f) for f in ("fwd_bf16.hip", "fa_device.hpp")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def time_launches(fn, steps, warmup, settle_s=0.0):
    """Warm up, then time `steps` calls: wall clock between synchronisations, and per-call
    HIP event pairs recorded on the stream the kernels are launched on. With settle_s > 0,
    calls run untimed for about that many seconds before the `warmup` calls (the secondary
    workloads use it: the GPU clock rises over tens of milliseconds of sustained load)."""
    import torch
    if settle_s > 0:
        t_end = time.perf_counter() + settle_s
        while time.perf_counter() < t_end:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ev = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    time_launches.last_median = sorted(ev)[len(ev) // 2]
    return wall_ms, sum(ev) / len(ev), min(ev)


def traffic_from_profile():
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current forward kernel source; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != source_digest(FWD_SOURCES):
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(target_s):
    """The float64 oracle on whole heads of the headline workload (same shapes and value
    distribution), head by head until about target_s seconds of CPU work."""
    import numpy as np
    import oracle
    import synth
    from io_aware_softmax_03_amd import costs
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover - informational only
        threads = None
    N, d = 8192, 128
    scale = 1 / math.sqrt(d)
    heads, elapsed = 0, 0.0
    while elapsed < target_s and heads < 32:
        b, h = divmod(heads, 16)
        qkv = [synth.f32_from_bf16_bits(synth.bf16_bits_from_f32(synth.normal_slice(2, t, b, h, (N, d))))
               .astype(np.float64) for t in (synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V)]
        t0 = time.perf_counter()
        oracle.attention_head(*qkv, scale, causal=True)
        elapsed += time.perf_counter() - t0
        heads += 1
    flops = costs.fwd_flops(1, heads, N, d, True)
    cores = threads or len(os.sched_getaffinity(0))
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} of 32 (b,h) heads of the causal B=2 H=16 N=8192 d=128 forward, float64 numpy "
                      f"oracle materialising S and P, {elapsed:.1f} s; host affinity "
                      f"{len(os.sched_getaffinity(0))} cpus"}


def extra_measurements(steps, only=None):
    """The secondary workloads; `only`, a set of names, restricts them (for profiler runs)."""
    import torch
    import io_aware_softmax_03_amd as fa
    from io_aware_softmax_03_amd import costs
    import synth
    out = {}
    gen = torch.Generator(device="cuda")

    def _bwd():
        # backward, B=4 H=16 N=4096 d=128 causal (preprocess, dK/dV and dQ kernels per call)
        B, H, N, d = 4, 16, 4096, 128
        gen.manual_seed(4)
        q, k, v, g = (torch.randn((B, N, H, d), generator=gen, device="cuda", dtype=torch.bfloat16) for _ in range(4))
        o, lse = fa.fwd(q, k, v, causal=True)
        grads = tuple(torch.empty((B, N, H, d), dtype=torch.float32, device="cuda") for _ in range(3))
        ws = torch.empty(fa.lib().fa_bwd_workspace_bytes(B, H, N), dtype=torch.uint8, device="cuda")
        wall, ev, best = time_launches(lambda: fa.bwd(q, k, v, o, lse, g, causal=True, out=grads, workspace=ws),
                                       steps, 3, SETTLE_S)
        fl = costs.bwd_flops(B, H, N, d, True)
        out["bwd_causal_b4_h16_n4096_d128"] = {
            "ms": round(ev, 4), "tflops": round(fl / ev / 1e9, 2), "frac_mfma_peak": round(fl / ev / 1e9 / PEAK_BF16_TFLOPS, 4),
            "flops_convention": "10*B*H*N^2*d/2 (five products)"}
        del q, k, v, g, o, lse, grads, ws


    def _varlen():
        # varlen forward: 16 sequences, lengths uniform in [128, 4096], H=32, d=64, causal, Q x4 on heads 16-31
        lengths = synth.varlen_lengths(3, 16, 128, 4096).tolist()
        cu = torch.tensor(synth.cu_seqlens_from_lengths(lengths), dtype=torch.int32, device="cuda")
        T, H, d = sum(lengths), 32, 64
        gen.manual_seed(3)
        q, k, v = (torch.randn((T, H, d), generator=gen, device="cuda", dtype=torch.float32) for _ in range(3))
        q[:, 16:] *= 4
        q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
        fa.check_cu_seqlens(synth.cu_seqlens_from_lengths(lengths), T, max(lengths))  # once, on the host
        wall, ev, best = time_launches(
            lambda: fa.fwd_varlen(q, k, v, cu, max(lengths), causal=True, validate=False), steps, 3, SETTLE_S)
        fl = costs.varlen_fwd_flops(lengths, H, d, True)
        # both rooflines of this d=64 launch over the scores the kernel forms (masked ones
        # in diagonal blocks included): matrix core (4*d FLOP per score, plus the row-sum
        # MFMAs, 1/8 of the 32x32x16 time at d=64) and VALU (per score one v_exp_f32 and
        # VALU_OPS_PER_SCORE other lane-operations, counted on this kernel by the SQ
        # counters), each at its unit's nominal rate at 2.4 GHz
        scores = costs.fwd_computed_scores(lengths, H, True, rows_per_wave=FWD_ROWS_PER_WAVE_D64)
        t_mfma = costs.mfma_bound_seconds(scores, d, 1 / 8) * 1e3
        t_valu = costs.valu_bound_seconds(scores, 1.0, VALU_OPS_PER_SCORE_D64) * 1e3
        out["varlen_causal_16seq_h32_d64"] = {
            "ms": round(ev, 4), "tflops": round(fl / ev / 1e9, 2),
            "frac_mfma_peak": round(fl / ev / 1e9 / PEAK_BF16_TFLOPS, 4), "total_tokens": T,
            "formed_scores": scores, "mfma_bound_ms": round(t_mfma, 4), "valu_bound_ms": round(t_valu, 4),
            "frac_of_mfma_bound": round(t_mfma / ev, 4), "frac_of_valu_bound": round(t_valu / ev, 4),
            "valu_per_score": f"1 exp (quarter rate) + {VALU_OPS_PER_SCORE_D64} other VALU ops (full rate)"}
        del q, k, v


    def _window():
        # banded forwards (bf16, d=128, causal, bottom-right): chunked prefill of 2048 new
        # queries against a 16384-key cache, and a 1024-key sliding window over 8192 tokens.
        # Work counted as 4*d per visible (query, key) pair.
        for name, B, H, Nq, Nk, left in (("fwd_chunked_prefill_b4_h16_q2048_k16384_d128", 4, 16, 2048, 16384, -1),
                                         ("fwd_sliding_window1024_b2_h16_n8192_d128", 2, 16, 8192, 8192, 1024)):
            d = 128
            gen.manual_seed(10)
            q = torch.randn((B, Nq, H, d), generator=gen, device="cuda", dtype=torch.bfloat16)
            k, v = (torch.randn((B, Nk, H, d), generator=gen, device="cuda", dtype=torch.bfloat16) for _ in range(2))
            o = torch.empty_like(q)
            lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
            wall, ev, best = time_launches(lambda: fa.fwd_window(q, k, v, causal=True, window=(left, -1), out=(o, lse)),
                                           steps, 3, SETTLE_S)
            fl = costs.band_fwd_flops(B, H, Nq, Nk, d, True, left)
            out[name] = {"ms": round(ev, 4), "tflops": round(fl / ev / 1e9, 2),
                         "frac_mfma_peak": round(fl / ev / 1e9 / PEAK_BF16_TFLOPS, 4),
                         "flops_convention": "4*d per visible (query, key) pair"}
            del q, k, v, o, lse


    def _fp8():
        # FP8 forward on the headline shape (causal B=2 H=16 N=8192 d=128), Q and K rotated:
        # one quantization launch (Q, K, V) plus the attention launch per call
        B, H, N, d = 2, 16, 8192, 128
        gen.manual_seed(11)
        q, k, v = (torch.randn((B, N, H, d), generator=gen, device="cuda", dtype=torch.bfloat16) for _ in range(3))
        signs = torch.from_numpy(synth.rademacher_signs(11, d)).to("cuda")
        ws = torch.empty(fa.lib().fa_fwd_fp8_workspace_bytes(B, H, H, N, d), dtype=torch.uint8, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        wall, ev, best = time_launches(lambda: fa.fwd_fp8(q, k, v, signs=signs, causal=True, out=(o, lse), workspace=ws),
                                       steps, 3, SETTLE_S)
        fl = costs.fwd_flops(B, H, N, d, True)
        out["fwd_fp8_causal_b2_h16_n8192_d128_rotated"] = {
            "ms": round(ev, 4), "tflops": round(fl / ev / 1e9, 2),
            "frac_fp8_mfma_peak": round(fl / ev / 1e9 / PEAK_FP8_TFLOPS, 4),
            "flops_convention": "4*B*H*N^2*d/2, per call (quantization of Q, K, V included)"}
        del q, k, v, o, lse, ws


    def _f32():
        # fp32 forward, B=1 H=1 N=256 d=64 (latency bound: one 256-key block per workgroup).
        # "us": HIP events around each call (host launch cost included: the kernel is shorter
        # than a call's host work); "us_graph": per call inside a replayed HIP graph of 64
        # calls, the kernel's own duration plus the gap between graph nodes
        gen.manual_seed(1)
        q, k, v = (torch.randn((1, 256, 1, 64), generator=gen, device="cuda") for _ in range(3))
        o = torch.empty_like(q)
        lse = torch.empty((1, 1, 256), dtype=torch.float32, device="cuda")
        wall, ev, best = time_launches(lambda: fa.fwd(q, k, v, out=(o, lse)), steps, 3, SETTLE_S)
        o_eager = o.clone()
        calls = 64
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fa.fwd(q, k, v, out=(o, lse))
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(calls):
                fa.fwd(q, k, v, out=(o, lse))
        o.zero_()
        torch.cuda.synchronize()
        gwall, gev, gbest = time_launches(graph.replay, max(10, steps // 10), 3)
        if not torch.equal(o, o_eager):
            raise RuntimeError("fp32 forward: graph replay differs from the eager call")
        out["fwd_f32_n256_d64"] = {"us": round(ev * 1e3, 2), "us_graph": round(gev * 1e3 / calls, 2)}
        del q, k, v, o, lse, graph


    def _decode():
        # decode: B=64 H=32 L=32768 d=128, 64 splits (34 GB of bf16 cache)
        B, H, L, d = 64, 32, 32768, 128
        gen.manual_seed(5)
        q = torch.randn((B, H, d), generator=gen, device="cuda", dtype=torch.bfloat16)
        kc = torch.randn((B, L, H, d), generator=gen, device="cuda", dtype=torch.bfloat16)
        vc = torch.randn((B, L, H, d), generator=gen, device="cuda", dtype=torch.bfloat16)
        ws = torch.empty(fa.lib().fa_decode_workspace_bytes(B, H, d, 64), dtype=torch.uint8, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
        wall, ev, best = time_launches(lambda: fa.decode(q, kc, vc, num_splits=64, workspace=ws, out=(o, lse)),
                                       max(3, steps // 2), 2, SETTLE_S)
        nb = costs.decode_bytes(B, H, L, d)
        out["decode_b64_h32_l32768_d128_s64"] = {"ms": round(ev, 4), "gbs": round(nb / ev / 1e6, 1),
                                                 "frac_hbm_peak": round(nb / ev / 1e6 / PEAK_HBM_GBS, 4),
                                                 "bytes_convention": "K and V caches read once + q + o"}
        del q, kc, vc, ws
        torch.cuda.empty_cache()


    def _decode_gqa():
        # grouped-query decode: 32 query heads over 8 key-value heads, L=32768, d=128; 32 splits
        # (a sweep over 16..256 puts the grouped kernel's best at 32: with 8 key-value heads a
        # 64-way split leaves each wave only 512 keys)
        B, H, Hkv, L, d = 64, 32, 8, 32768, 128
        gen.manual_seed(9)
        q = torch.randn((B, H, d), generator=gen, device="cuda", dtype=torch.bfloat16)
        kc = torch.randn((B, L, Hkv, d), generator=gen, device="cuda", dtype=torch.bfloat16)
        vc = torch.randn((B, L, Hkv, d), generator=gen, device="cuda", dtype=torch.bfloat16)
        ws = torch.empty(fa.lib().fa_decode_workspace_bytes(B, H, d, 32), dtype=torch.uint8, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
        wall, ev, best = time_launches(lambda: fa.decode(q, kc, vc, num_splits=32, workspace=ws, out=(o, lse)),
                                       max(3, steps // 2), 2, SETTLE_S)
        nb = costs.decode_bytes(B, Hkv, L, d) + 2.0 * B * (H - Hkv) * d * 2
        out["decode_gqa_b64_h32_kv8_l32768_d128_s32"] = {
            "ms": round(ev, 4), "gbs": round(nb / ev / 1e6, 1), "frac_hbm_peak": round(nb / ev / 1e6 / PEAK_HBM_GBS, 4),
            "bytes_convention": "K and V caches (8 heads) read once + q + o (32 heads)"}
        del q, kc, vc, ws
        torch.cuda.empty_cache()


    def _decode_paged():
        # paged decode: B=64 H=32 d=128, 16-token pages scattered over the pool, lengths uniform
        # in [16384, 32768], 32 splits (the sweep's best; sequences are up to half as long as
        # the contiguous decode's)
        B, H, d, P = 64, 32, 128, 16
        seqlens = synth.varlen_lengths(8, B, 16384, 32768).tolist()
        table, num_pages = synth.paged_layout(8, seqlens, P, 0)
        gen.manual_seed(8)
        q = torch.randn((B, H, d), generator=gen, device="cuda", dtype=torch.bfloat16)
        kp = torch.randn((num_pages, P, H, d), generator=gen, device="cuda", dtype=torch.bfloat16)
        vp = torch.randn((num_pages, P, H, d), generator=gen, device="cuda", dtype=torch.bfloat16)
        tab = torch.from_numpy(table).to("cuda")
        sl = torch.tensor(seqlens, dtype=torch.int32, device="cuda")
        ws = torch.empty(fa.lib().fa_decode_workspace_bytes(B, H, d, 32), dtype=torch.uint8, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
        wall, ev, best = time_launches(
            lambda: fa.decode_paged(q, kp, vp, tab, sl, num_splits=32, workspace=ws, out=(o, lse)),
            max(3, steps // 2), 2, SETTLE_S)
        nb = costs.decode_paged_bytes(seqlens, H, d)
        out["decode_paged_b64_h32_p16_l16k_32k_d128_s32"] = {
            "ms": round(ev, 4), "gbs": round(nb / ev / 1e6, 1), "frac_hbm_peak": round(nb / ev / 1e6 / PEAK_HBM_GBS, 4),
            "tokens": int(sum(seqlens)), "bytes_convention": "valid K and V tokens read once + q + o"}
        del q, kp, vp, ws
        torch.cuda.empty_cache()

    for name, fn in [("bwd", _bwd), ("varlen", _varlen), ("window", _window), ("fp8", _fp8), ("f32", _f32), ("decode", _decode), ("decode_gqa", _decode_gqa), ("decode_paged", _decode_paged)]:
        if only is None or name in only:
            fn()
    return out


def main():
    global SETTLE_S
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=1500)
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--extra-only", default=None,
                    help="comma-separated secondary workloads to run (bwd, varlen, window, fp8, f32, decode, "
                         "decode_gqa, decode_paged); for profiler runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="untimed seconds of calls before each workload's warm-up, the headline's too "
                         "(0 for profiler runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (untimed), so that a counter "
                         "profile of this command holds a kernel of known traffic to scale HBM counters by")
    args = ap.parse_args()
    SETTLE_S = args.settle_s
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import io_aware_softmax_03_amd as fa
    from io_aware_softmax_03_amd import costs

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {n} bytes read, {n} bytes written")
        del src, dst

    # The secondary workloads run first, so the headline follows sustained GPU load rather than
    # an idle GPU whose clock is still rising; like each of them it then runs untimed for
    # SETTLE_S seconds before its W warm-up steps and K timed steps.
    extra = None
    if not args.no_extra:
        log("[bench] secondary workloads")
        only = set(args.extra_only.split(",")) if args.extra_only else None
        extra = extra_measurements(args.steps, only)
        log(f"[bench] extra: {json.dumps(extra)}")
        torch.cuda.empty_cache()

    B, H, N, d = 2, 16, 8192, 128
    log(f"[bench] headline: causal bf16 forward B={B} H={H} N={N} d={d}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2)
    q, k, v = (torch.randn((B, N, H, d), generator=gen, device="cuda", dtype=torch.bfloat16) for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    step = lambda: fa.fwd(q, k, v, causal=True, out=(o, lse))  # noqa: E731
    wall_ms, kern_ms, kern_min = time_launches(step, args.steps, args.warmup, SETTLE_S)
    kern_median = time_launches.last_median
    flops = costs.fwd_flops(B, H, N, d, True)
    value = flops / (wall_ms * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    log(f"[bench] fwd: {wall_ms:.4f} ms/step wall, {kern_ms:.4f} ms/launch (min {kern_min:.4f}) "
        f"-> {achieved:.1f} TFLOP/s")

    prop = torch.cuda.get_device_properties(0)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: N(0,1) bf16 Q/K/V drawn on the device from a seeded generator",
        "config": {"workload": "causal attention forward B=2 H=16 N=8192 d=128 bf16 (fp32 accumulate)",
                   "batch": B, "heads": H, "seq_len": N, "head_dim": d, "causal": True,
                   "flops_per_step": flops, "flops_convention": "4*B*H*N^2*d/2"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile(),
                     "kernel": "fwd_bf16_kernel<128, causal, dense>", "launch_ms": round(kern_ms, 4),
                     "launch_ms_median": round(kern_median, 4), "launch_ms_min": round(kern_min, 4)},
        "device": {"name": prop.name, "gcn_arch": getattr(prop, "gcnArchName", ""),
                   "cus": prop.multi_processor_count},
    }
    if extra is not None:
        result["extra"] = extra
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (float64 oracle)")
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
