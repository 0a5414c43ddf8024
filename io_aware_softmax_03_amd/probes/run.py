"""Run the gfx950 hardware probes (probes.hip) on cuda:0 and print a markdown table.

Usage: ``python -m io_aware_softmax_03_amd.probes.run`` (after ``build()``). The probes measure
what the attention kernels are designed against: dense bf16 matrix-core throughput at one
and at several waves per SIMD, the same with the forward kernel's per-score VALU work issued
between MFMAs, streaming HBM read and copy bandwidth, and which XCD each workgroup runs on.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_probes.so")
MFMA_FLOP = 2 * 32 * 32 * 16  # one v_mfma_f32_32x32x16_bf16


def _lib():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m io_aware_softmax_03_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.probe_mfma.argtypes = [P, I, I, I, P]
    lib.probe_mfma_exp.argtypes = [P, I, I, I, P]
    lib.probe_read.argtypes = [P, Z, P, I, P]
    lib.probe_copy.argtypes = [P, P, Z, I, P]
    lib.probe_xcc.argtypes = [P, I, P]
    for f in (lib.probe_mfma, lib.probe_mfma_exp, lib.probe_read, lib.probe_copy, lib.probe_xcc):
        f.restype = I
    return lib


def _time(fn, reps=5, warmup=2):
    """Median milliseconds of fn() (HIP events on the current stream)."""
    for _ in range(warmup):
        fn()
    ts = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        e.synchronize()
        ts.append(s.elapsed_time(e))
    ts.sort()
    return ts[len(ts) // 2]


def _check(st, name):
    if st != 0:
        raise RuntimeError(f"{name}: hipError {st}")


def main():
    assert torch.cuda.is_available(), "the probes need a GPU"
    lib = _lib()
    stream = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = []

    iters = 4000
    for label, fn_name, waves, grid in (("MFMA bf16 32x32x16, 1 wave/SIMD", "mfma", 1, 4 * cus),
                                        ("MFMA bf16 32x32x16, 3 waves/SIMD", "mfma", 2, 12 * cus),
                                        ("MFMA + 1 exp + 4 FMA per MFMA, 1 wave/SIMD", "mfma_exp", 1, 4 * cus),
                                        ("MFMA + 1 exp + 4 FMA per MFMA, several waves/SIMD", "mfma_exp", 2, 12 * cus)):
        out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
        if fn_name == "mfma":
            f = lambda: _check(lib.probe_mfma(out.data_ptr(), grid, iters, waves, stream), "probe_mfma")  # noqa: E731
        else:
            f = lambda: _check(lib.probe_mfma_exp(out.data_ptr(), grid, iters, waves, stream), "probe_mfma_exp")  # noqa: E731
        # warm the clock with a longer run before timing
        _time(f, reps=3, warmup=20)
        ms = _time(f)
        nacc = 4 if (fn_name == "mfma_exp" and waves != 1) else 8
        flops = grid * 4 * iters * nacc * MFMA_FLOP
        rows.append((label, f"{flops / ms / 1e9:.0f} TFLOP/s",
                     f"{grid} workgroups x 4 waves, {iters} rounds of {nacc} MFMAs"))

    nbytes = 8 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    grid = 64 * cus
    out = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
    ms = _time(lambda: _check(lib.probe_read(src.data_ptr(), nbytes // 16, out.data_ptr(), grid, stream), "probe_read"))
    rows.append(("HBM streaming read (nontemporal, 16 B per lane)", f"{nbytes / ms / 1e6:.0f} GB/s", "8 GiB"))
    half = nbytes // 2
    dst = torch.empty(half, dtype=torch.uint8, device="cuda")
    ms = _time(lambda: _check(lib.probe_copy(src.data_ptr(), dst.data_ptr(), half // 16, grid, stream), "probe_copy"))
    rows.append(("HBM copy (read + write counted)", f"{2 * half / ms / 1e6:.0f} GB/s", "4 GiB to 4 GiB"))
    del src, dst, out

    grid = 4096
    xo = torch.empty(grid, dtype=torch.int32, device="cuda")
    _check(lib.probe_xcc(xo.data_ptr(), grid, stream), "probe_xcc")
    torch.cuda.synchronize()
    x = xo.cpu()
    same = int((x == (torch.arange(grid) % 8)).sum())
    rows.append(("workgroup w on XCD w % 8", f"{same}/{grid}", "XCC id register read by each workgroup"))

    print("| probe | result | setup |")
    print("|---|---|---|")
    for r in rows:
        print(f"| {r[0]} | {r[1]} | {r[2]} |")


if __name__ == "__main__":
    main()
