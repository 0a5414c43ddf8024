"""The C ABI loads, exports every symbol include/fa.h declares, and rejects bad arguments
on the host (these calls return before any HIP call, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

from io_aware_softmax_03_amd import _clib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_clib.LIB_PATH),
                                reason="libfa.so not built (run python -m io_aware_softmax_03_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(_clib.SIGNATURES)


def test_every_declared_symbol_is_exported():
    raw = ctypes.CDLL(_clib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name, value in re.findall(r"(FA_(?:OK|ERR_[A-Z]+))\s*=\s*(-?\d+)", text):
        assert getattr(_clib, name) == int(value)
    for name, value in re.findall(r"(FA_DTYPE_[A-Z0-9]+)\s*=\s*(\d+)", text):
        assert getattr(_clib, name) == int(value)


def test_strerror():
    lib = _clib.lib()
    for code in range(-8, 1):
        assert lib.fa_strerror(code)
    assert b"unknown" in lib.fa_strerror(42)


def test_workspace_sizes():
    lib = _clib.lib()
    assert lib.fa_bwd_workspace_bytes(4, 16, 4096) == 2 * 4 * 16 * 4096 * 4
    assert lib.fa_decode_workspace_bytes(64, 32, 128, 64) == 64 * 32 * 64 * 130 * 4
    assert lib.fa_bwd_workspace_bytes(-1, 1, 1) == 0


FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced by failing calls


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, Hkv=1, N=16, d=64, scale=0.125,
             causal=0, dtype=_clib.FA_DTYPE_BF16, stream=None)
    a.update(kw)
    return _clib.lib().fa_fwd(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), _clib.FA_ERR_SHAPE), (dict(H=0), _clib.FA_ERR_SHAPE), (dict(N=-5), _clib.FA_ERR_SHAPE),
    (dict(Hkv=0), _clib.FA_ERR_SHAPE), (dict(Hkv=2), _clib.FA_ERR_SHAPE), (dict(H=6, Hkv=4), _clib.FA_ERR_SHAPE),
    (dict(H=6, Hkv=-3), _clib.FA_ERR_SHAPE),
    (dict(d=96), _clib.FA_ERR_HEADDIM), (dict(d=256), _clib.FA_ERR_HEADDIM),
    (dict(dtype=7), _clib.FA_ERR_DTYPE), (dict(scale=0.0), _clib.FA_ERR_ARG),
    (dict(scale=float("nan")), _clib.FA_ERR_ARG), (dict(scale=-1.0), _clib.FA_ERR_ARG),
    (dict(causal=2), _clib.FA_ERR_ARG), (dict(q=None), _clib.FA_ERR_NULL), (dict(lse=None), _clib.FA_ERR_NULL),
    (dict(o=FAKE + 2), _clib.FA_ERR_ARG), (dict(B=1 << 30, N=1 << 30, H=1 << 10), _clib.FA_ERR_SHAPE),
])
def test_fwd_rejects(kw, code):
    assert fwd(**kw) == code


def test_fwd_empty_is_noop():
    # nothing to compute: succeeds without touching memory, even with NULL pointers
    assert fwd(B=0, q=None, k=None, v=None, o=None, lse=None) == _clib.FA_OK
    assert fwd(N=0, q=None, k=None, v=None, o=None, lse=None) == _clib.FA_OK


def fwd_window(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=4, Hkv=2, Nq=16, Nk=64, d=128, scale=0.1,
             causal=1, left=-1, right=-1, dtype=_clib.FA_DTYPE_BF16, stream=None)
    a.update(kw)
    return _clib.lib().fa_fwd_window(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(Nq=-1), _clib.FA_ERR_SHAPE), (dict(Nk=-1), _clib.FA_ERR_SHAPE), (dict(Nq=(1 << 30) + 1), _clib.FA_ERR_SHAPE),
    (dict(Nk=(1 << 30) + 1), _clib.FA_ERR_SHAPE), (dict(Hkv=3), _clib.FA_ERR_SHAPE), (dict(left=-2), _clib.FA_ERR_ARG),
    (dict(right=-5), _clib.FA_ERR_ARG), (dict(right=3), _clib.FA_ERR_ARG), (dict(causal=2), _clib.FA_ERR_ARG),
    (dict(d=80), _clib.FA_ERR_HEADDIM), (dict(dtype=9), _clib.FA_ERR_DTYPE), (dict(k=None), _clib.FA_ERR_NULL),
    (dict(lse=FAKE + 4), _clib.FA_ERR_ARG), (dict(scale=float("inf")), _clib.FA_ERR_ARG),
])
def test_fwd_window_rejects(kw, code):
    assert fwd_window(**kw) == code


def test_fwd_window_accepts_upper_window_without_causal_and_empty_queries():
    assert fwd_window(Nq=0, q=None, k=None, v=None, o=None, lse=None) == _clib.FA_OK
    assert fwd_window(B=0, causal=0, right=3, q=None, k=None, v=None, o=None, lse=None) == _clib.FA_OK


def varlen(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, cu=FAKE, num_seqs=2, total=10, max_seqlen=6, H=2,
             Hkv=2, d=128, scale=0.1, causal=1, dtype=_clib.FA_DTYPE_BF16, stream=None)
    a.update(kw)
    return _clib.lib().fa_fwd_varlen(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), _clib.FA_ERR_NULL), (dict(max_seqlen=11), _clib.FA_ERR_SHAPE),
    (dict(max_seqlen=0), _clib.FA_ERR_SHAPE), (dict(num_seqs=0), _clib.FA_ERR_SHAPE),
    (dict(num_seqs=-1), _clib.FA_ERR_SHAPE), (dict(d=32), _clib.FA_ERR_HEADDIM),
    (dict(dtype=3), _clib.FA_ERR_DTYPE), (dict(causal=-1), _clib.FA_ERR_ARG),
    (dict(Hkv=3), _clib.FA_ERR_SHAPE), (dict(Hkv=0), _clib.FA_ERR_SHAPE),
])
def test_varlen_rejects(kw, code):
    assert varlen(**kw) == code


def test_varlen_empty_is_noop():
    assert varlen(total=0, max_seqlen=0, q=None, k=None, v=None, o=None, lse=None, cu=None) == _clib.FA_OK


def bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, H=2, Hkv=2, N=64,
             d=128, scale=0.1, causal=1, dtype=_clib.FA_DTYPE_BF16, ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return _clib.lib().fa_bwd(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=_clib.FA_DTYPE_F32), _clib.FA_ERR_DTYPE), (dict(ws=None), _clib.FA_ERR_WORKSPACE),
    (dict(ws_bytes=2 * 64 * 2 * 4 - 1), _clib.FA_ERR_WORKSPACE), (dict(dq=None), _clib.FA_ERR_NULL),
    (dict(d=80), _clib.FA_ERR_HEADDIM), (dict(scale=float("inf")), _clib.FA_ERR_ARG),
    (dict(dk=FAKE + 4), _clib.FA_ERR_ARG), (dict(H=-2), _clib.FA_ERR_SHAPE),
    (dict(Hkv=3), _clib.FA_ERR_SHAPE), (dict(Hkv=0), _clib.FA_ERR_SHAPE), (dict(N=(1 << 30) + 1), _clib.FA_ERR_SHAPE),
])
def test_bwd_rejects(kw, code):
    assert bwd(**kw) == code


def decode(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, lse=None, B=2, H=4, Hkv=4, L=1000, d=128, scale=0.1, splits=8,
             dtype=_clib.FA_DTYPE_BF16, ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return _clib.lib().fa_decode(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(splits=0), _clib.FA_ERR_ARG), (dict(splits=1025), _clib.FA_ERR_ARG), (dict(L=0), _clib.FA_ERR_SHAPE),
    (dict(ws_bytes=2 * 4 * 8 * 130 * 4 - 1), _clib.FA_ERR_WORKSPACE), (dict(ws=None), _clib.FA_ERR_WORKSPACE),
    (dict(dtype=_clib.FA_DTYPE_F32), _clib.FA_ERR_DTYPE), (dict(kc=None), _clib.FA_ERR_NULL),
    (dict(d=100), _clib.FA_ERR_HEADDIM), (dict(ws=FAKE + 8), _clib.FA_ERR_ARG),
    (dict(Hkv=3), _clib.FA_ERR_SHAPE), (dict(Hkv=8), _clib.FA_ERR_SHAPE), (dict(Hkv=0), _clib.FA_ERR_SHAPE),
])
def test_decode_rejects(kw, code):
    assert decode(**kw) == code


def decode_noalloc(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, lse=None, B=2, H=4, Hkv=4, L=1000, d=128, scale=0.1, splits=8,
             dtype=_clib.FA_DTYPE_BF16, stream=None)
    a.update(kw)
    return _clib.lib().fa_decode_noalloc(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(splits=0), _clib.FA_ERR_ARG), (dict(splits=1025), _clib.FA_ERR_ARG), (dict(L=0), _clib.FA_ERR_SHAPE),
    (dict(dtype=_clib.FA_DTYPE_F32), _clib.FA_ERR_DTYPE), (dict(kc=None), _clib.FA_ERR_NULL),
    (dict(d=100), _clib.FA_ERR_HEADDIM), (dict(q=FAKE + 8), _clib.FA_ERR_ARG), (dict(Hkv=3), _clib.FA_ERR_SHAPE),
    # partials above the 64 MiB scratch: 64 * 32 * 64 * 130 * 4 bytes = 65 MiB
    (dict(B=64, H=32, Hkv=32, L=32768, splits=64), _clib.FA_ERR_SCRATCH),
    (dict(B=1 << 20, H=1 << 10, Hkv=1 << 10, L=1, splits=1024), _clib.FA_ERR_SCRATCH),
])
def test_decode_noalloc_rejects(kw, code):
    assert decode_noalloc(**kw) == code


def test_decode_noalloc_limit_is_64_mib():
    # 64 * 32 * 63 * 130 * 4 bytes fit the scratch; the same call with 64 splits does not
    assert 64 * 32 * 63 * 130 * 4 <= 64 << 20 < 64 * 32 * 64 * 130 * 4
    assert decode_noalloc(B=64, H=32, Hkv=32, L=32768, splits=64, q=None) == _clib.FA_ERR_SCRATCH
    assert decode_noalloc(B=64, H=32, Hkv=32, L=32768, splits=63, q=None) == _clib.FA_ERR_NULL


def test_decode_noalloc_empty_batch_is_a_no_op():
    assert decode_noalloc(B=0, q=None, kc=None, vc=None, o=None) == _clib.FA_OK


def decode_paged(**kw):
    a = dict(q=FAKE, kp=FAKE, vp=FAKE, table=FAKE, seqlens=FAKE, o=FAKE, lse=None, B=2, H=4, Hkv=2, d=128,
             page_size=16, num_pages=100, max_pages=20, scale=0.1, splits=8, dtype=_clib.FA_DTYPE_BF16,
             ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return _clib.lib().fa_decode_paged(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(page_size=0), _clib.FA_ERR_SHAPE), (dict(page_size=24), _clib.FA_ERR_SHAPE),
    (dict(page_size=2048), _clib.FA_ERR_SHAPE), (dict(num_pages=0), _clib.FA_ERR_SHAPE),
    (dict(max_pages=0), _clib.FA_ERR_SHAPE), (dict(max_pages=(1 << 26) + 1), _clib.FA_ERR_SHAPE),
    (dict(B=-1), _clib.FA_ERR_SHAPE), (dict(splits=0), _clib.FA_ERR_ARG),
    (dict(ws_bytes=2 * 4 * 8 * 130 * 4 - 1), _clib.FA_ERR_WORKSPACE), (dict(ws=None), _clib.FA_ERR_WORKSPACE),
    (dict(dtype=_clib.FA_DTYPE_F32), _clib.FA_ERR_DTYPE), (dict(table=None), _clib.FA_ERR_NULL),
    (dict(seqlens=None), _clib.FA_ERR_NULL), (dict(d=96), _clib.FA_ERR_HEADDIM),
    (dict(table=FAKE + 2), _clib.FA_ERR_ARG), (dict(vp=FAKE + 8), _clib.FA_ERR_ARG),
    (dict(scale=-1.0), _clib.FA_ERR_ARG), (dict(Hkv=3), _clib.FA_ERR_SHAPE), (dict(Hkv=5), _clib.FA_ERR_SHAPE),
])
def test_decode_paged_rejects(kw, code):
    assert decode_paged(**kw) == code


def test_decode_paged_empty_batch_is_a_no_op():
    # B = 0 returns before touching any pointer
    assert decode_paged(B=0, q=None, kp=None, vp=None, table=None, seqlens=None, o=None, ws=None) == _clib.FA_OK


def fwd_fp8(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, signs=None, o=FAKE, lse=FAKE, B=1, H=4, Hkv=2, N=100, d=128, scale=0.1,
             causal=1, ws=FAKE, ws_bytes=1 << 24, stream=None)
    a.update(kw)
    return _clib.lib().fa_fwd_fp8(*a.values())


def test_fwd_fp8_workspace_bytes():
    lib = _clib.lib()
    # B=1, H=4, Hkv=2, N=100 (two 64-row blocks), d=128: codes of Q, K, V then exponents,
    # each part rounded up to 256 bytes
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    q8, kv8 = 4 * 128 * 128, 2 * 128 * 128
    total = up(q8) + up(kv8) + up(kv8) + up(4 * 2 * 4) + up(2 * 2 * 4) + up(2 * 2 * 4)
    assert lib.fa_fwd_fp8_workspace_bytes(1, 4, 2, 100, 128) == total
    assert lib.fa_fwd_fp8_workspace_bytes(1, 4, 3, 100, 128) == 0
    assert lib.fa_fwd_fp8_workspace_bytes(1, 4, 2, 100, 96) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(Hkv=3), _clib.FA_ERR_SHAPE), (dict(N=-1), _clib.FA_ERR_SHAPE), (dict(d=96), _clib.FA_ERR_HEADDIM),
    (dict(scale=0.0), _clib.FA_ERR_ARG), (dict(causal=5), _clib.FA_ERR_ARG), (dict(q=None), _clib.FA_ERR_NULL),
    (dict(ws=None), _clib.FA_ERR_WORKSPACE), (dict(ws_bytes=1000), _clib.FA_ERR_WORKSPACE),
    (dict(ws=FAKE + 16), _clib.FA_ERR_ARG), (dict(signs=FAKE + 2), _clib.FA_ERR_ARG), (dict(signs=FAKE + 4), _clib.FA_ERR_ARG),
    (dict(o=FAKE + 8), _clib.FA_ERR_ARG),
])
def test_fwd_fp8_rejects(kw, code):
    assert fwd_fp8(**kw) == code


def test_python_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    import io_aware_softmax_03_amd as fa
    x = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fa.fwd(x, x, x)
