"""C-ABI checks that need no GPU: the library loads, exports every function that
include/fa3q.h declares with the binding's signature table, and rejects invalid
arguments on the host before anything is enqueued.

The argument-rejection cases pass fake non-NULL pointers; they run only where no GPU
is visible, so a validation bug can never turn into a launch on a real device.
"""
import ctypes
import os
import re

import pytest

import kv_cache_quantization_fa3q_amd as fa
from kv_cache_quantization_fa3q_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa3q.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa3q_[a-z0-9_]+)\s*\(", text)))


def _gpu_visible():
    import torch
    return torch.cuda.is_available()


no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer validation cases run only without a GPU")


def test_library_exports_every_declared_function():
    lib = fa.lib()
    declared = _declared_functions()
    assert len(declared) >= 11
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(L.SIGNATURES) == declared


def test_version_and_status_strings():
    lib = fa.lib()
    assert lib.fa3q_version() >> 16 == 1
    for code in range(12):
        s = fa.status_string(code)
        assert s.startswith("FA3Q_")
    assert fa.status_string(0) == "FA3Q_OK"
    assert "UNKNOWN" in fa.status_string(99)


def test_max_windows_cover_the_workloads():
    lib = fa.lib()
    assert lib.fa3q_calibrate_max_windows(L.FA3Q_BF16) >= 4196  # ratio 0.999 on 4M values per head
    assert lib.fa3q_calibrate_max_windows(L.FA3Q_F32) >= 22
    assert lib.fa3q_calibrate_max_windows(7) == 0


def _ratio_for_k(N: int, K: int) -> float:
    # int(ratio * N) = N - K + 1 exactly: the ratio sits half a value inside the step
    return (N - K + 1 + 0.5) / N


@pytest.mark.parametrize("dtype,S", [(L.FA3Q_BF16, 4096), (L.FA3Q_F32, 2048)])
def test_window_count_limit_is_where_the_tail_lists_stop(dtype, S):
    lib = fa.lib()
    kmax = lib.fa3q_calibrate_max_windows(dtype)
    N = S * 16
    at_cap = lib.fa3q_calibrate_workspace_bytes(dtype, 1, 2, S, 16, _ratio_for_k(N, kmax))
    past = lib.fa3q_calibrate_workspace_bytes(dtype, 1, 2, S, 16, _ratio_for_k(N, kmax + 1))
    assert at_cap > 0
    if dtype == L.FA3Q_BF16:
        # past the on-chip tail lists the histogram path takes over: a region of 65536 words per head
        assert past >= 2 * 65536 * 4
    else:
        # float32: the collect-and-sort path, two lists of N keys per head
        assert past >= 2 * 2 * N * 4


@pytest.mark.parametrize("dtype", [L.FA3Q_F32, L.FA3Q_BF16, L.FA3Q_F16])
@pytest.mark.parametrize("layout", [L.FA3Q_BHSD, L.FA3Q_BSHD])
def test_every_valid_ratio_has_a_plan(dtype, layout):
    # FA3量化 page, 原理 -> 算法流程: the window is defined for every ratio with int(ratio*N) >= 1;
    # no such ratio is refused (a workspace query of 0 would mean an error status)
    lib = fa.lib()
    cap = lib.fa3q_calibrate_max_windows(dtype)
    for (B, H, S, D) in [(1, 2, 64, 16), (2, 8, 2048, 128), (8, 128, 2048, 128), (3, 5, 777, 8)]:
        N = B * S * D
        ks = {1, 2, cap, cap + 1, N // 100, N // 10, N // 2, N - 1, N}
        ratios = {1.0, 0.9999, 0.999, 0.99, 0.9, 0.5, 0.01, 1.0 / N}
        ratios |= {_ratio_for_k(N, k) for k in ks if 1 <= k <= N - 1}
        for r in sorted(ratios):
            if r > 1.0 or int(r * N) < 1:
                continue
            ws = lib.fa3q_calibrate_ex_workspace_bytes(dtype, layout, 1, B, H, S, D, r)
            assert ws > 0, (dtype, layout, (B, H, S, D), r)


def test_bf16_calibration_takes_every_valid_ratio():
    lib = fa.lib()
    for B, H, S, D in ((1, 2, 64, 32), (8, 128, 2048, 128), (2, 128, 16384, 128)):
        N = B * S * D
        for ratio in (1.0, 0.99999, 0.9999, 0.999, 0.99, 0.9, 0.5, 0.1, 1.0 / N):
            if int(ratio * N) < 1:
                continue
            assert lib.fa3q_calibrate_workspace_bytes(L.FA3Q_BF16, B, H, S, D, ratio) > 0, (B, H, S, D, ratio)
            assert lib.fa3q_calibrate_batches_workspace_bytes(L.FA3Q_BF16, 4, B, H, S, D, ratio) > 0
    # values per head must stay below 2^32
    assert lib.fa3q_calibrate_workspace_bytes(L.FA3Q_BF16, 1 << 14, 1, 1 << 10, 1 << 8, 0.5) == 0


def test_workspace_queries():
    lib = fa.lib()
    # bf16 (8,128,2048,128), ratio 0.9999: K=211
    ws = lib.fa3q_calibrate_workspace_bytes(L.FA3Q_BF16, 8, 128, 2048, 128, 0.9999)
    assert 0 < ws < 64 * 2**20
    assert lib.fa3q_calibrate_workspace_bytes(L.FA3Q_BF16, 8, 128, 2048, 128, 0.0) == 0
    assert lib.fa3q_calibrate_workspace_bytes(9, 8, 128, 2048, 128, 0.5) == 0
    assert lib.fa3q_calibrate_workspace_bytes(L.FA3Q_BF16, 8, 128, 2048, 127, 0.9999) > 0  # S*D % 8 == 0
    assert lib.fa3q_calibrate_workspace_bytes(L.FA3Q_BF16, 1, 1, 3, 5, 0.5) == 0       # S*D = 15
    # decode: 8192 (b,h) pairs need no split; 1024 pairs over 32768 tokens do
    assert lib.fa3q_decode_attn_workspace_bytes(64, 128, 4096, 128) == 0
    assert lib.fa3q_decode_attn_workspace_bytes(8, 128, 32768, 128) > 0
    assert lib.fa3q_decode_attn_workspace_bytes(1, 1, 1, 100) == 0


FAKE = 0x10000  # never dereferenced: every case below must fail validation


def _p(off=0):
    return ctypes.c_void_p(FAKE + off)


@no_gpu_only
def test_calibrate_rejections():
    f = fa.lib().fa3q_calibrate_perhead
    big = 1 << 30
    ok = dict(x=_p(), dt=L.FA3Q_BF16, B=1, H=4, S=64, D=32, r=0.9, mn=_p(), mx=_p(), ws=_p(), wsb=big)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["dt"], a["B"], a["H"], a["S"], a["D"], a["r"], a["mn"], a["mx"], a["ws"], a["wsb"], None)

    assert call(x=None) == L.FA3Q_ERR_NULL
    assert call(mn=None) == L.FA3Q_ERR_NULL
    assert call(mx=None) == L.FA3Q_ERR_NULL
    assert call(dt=5) == L.FA3Q_ERR_DTYPE
    assert call(B=0) == L.FA3Q_ERR_SHAPE
    assert call(H=-1) == L.FA3Q_ERR_SHAPE
    assert call(S=3, D=5) == L.FA3Q_ERR_SHAPE
    assert call(r=0.0) == L.FA3Q_ERR_RATIO
    assert call(r=1.5) == L.FA3Q_ERR_RATIO
    assert call(r=float("nan")) == L.FA3Q_ERR_RATIO
    assert call(r=1e-9) == L.FA3Q_ERR_RATIO                 # int(ratio*N) = 0
    assert call(x=_p(2)) == L.FA3Q_ERR_ALIGN
    assert call(mn=_p(2)) == L.FA3Q_ERR_ALIGN
    assert call(ws=None) == L.FA3Q_ERR_WORKSPACE
    assert call(wsb=16) == L.FA3Q_ERR_WORKSPACE
    assert call(ws=_p(64)) == L.FA3Q_ERR_ALIGN


@no_gpu_only
def test_stats_rejections():
    lib = fa.lib()
    assert lib.fa3q_init_minmax(None, _p(), 4, None) == L.FA3Q_ERR_NULL
    assert lib.fa3q_init_minmax(_p(), _p(), 0, None) == L.FA3Q_ERR_SHAPE
    assert lib.fa3q_init_minmax(_p(1), _p(), 4, None) == L.FA3Q_ERR_ALIGN
    assert lib.fa3q_accumulate_minmax(_p(), _p(), None, _p(), 4, None) == L.FA3Q_ERR_NULL
    assert lib.fa3q_accumulate_minmax(_p(), _p(), _p(), _p(), -3, None) == L.FA3Q_ERR_SHAPE
    assert lib.fa3q_accumulate_minmax(_p(), _p(), _p(2), _p(), 4, None) == L.FA3Q_ERR_ALIGN
    assert lib.fa3q_qparams(_p(), None, _p(), 4, None) == L.FA3Q_ERR_NULL
    assert lib.fa3q_qparams(_p(), _p(), _p(), 0, None) == L.FA3Q_ERR_SHAPE
    assert lib.fa3q_qparams(_p(), _p(), _p(3), 4, None) == L.FA3Q_ERR_ALIGN


@no_gpu_only
def test_quantize_rejections():
    f = fa.lib().fa3q_quantize_k
    ok = dict(k=_p(), s=_p(), q=_p(), r=_p(), B=1, H=4, S=64, Dn=32, Dr=16)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["k"], a["s"], a["q"], a["r"], a["B"], a["H"], a["S"], a["Dn"], a["Dr"], None)

    assert call(k=None) == L.FA3Q_ERR_NULL
    assert call(s=None) == L.FA3Q_ERR_NULL
    assert call(q=None) == L.FA3Q_ERR_NULL
    assert call(r=None) == L.FA3Q_ERR_NULL
    assert call(S=0) == L.FA3Q_ERR_SHAPE
    assert call(Dn=24) == L.FA3Q_ERR_SHAPE
    assert call(Dn=0) == L.FA3Q_ERR_SHAPE
    assert call(Dr=12) == L.FA3Q_ERR_SHAPE
    assert call(Dr=-8) == L.FA3Q_ERR_SHAPE
    assert call(k=_p(8)) == L.FA3Q_ERR_ALIGN
    assert call(q=_p(4)) == L.FA3Q_ERR_ALIGN
    assert call(r=_p(2)) == L.FA3Q_ERR_ALIGN
    assert call(s=_p(2)) == L.FA3Q_ERR_ALIGN


@no_gpu_only
def test_decode_rejections():
    f = fa.lib().fa3q_decode_attn
    ok = dict(q=_p(), kq=_p(), s=_p(), kr=_p(), v=_p(), B=8, H=128, T=32768, Dn=128, Dr=64, Dv=128,
              sm=0.07, o=_p(), ws=_p(), wsb=1 << 30)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["kq"], a["s"], a["kr"], a["v"], a["B"], a["H"], a["T"], a["Dn"], a["Dr"], a["Dv"],
                 ctypes.c_float(a["sm"]), a["o"], a["ws"], a["wsb"], None)

    for name in ("q", "kq", "s", "kr", "v", "o"):
        assert call(**{name: None}) == L.FA3Q_ERR_NULL, name
    assert call(T=0) == L.FA3Q_ERR_SHAPE
    assert call(Dn=120) == L.FA3Q_ERR_SHAPE
    assert call(Dn=2048) == L.FA3Q_ERR_SHAPE
    assert call(Dr=60) == L.FA3Q_ERR_SHAPE
    assert call(Dv=96) == L.FA3Q_ERR_SHAPE
    assert call(Dv=1024) == L.FA3Q_ERR_SHAPE
    assert call(sm=float("inf")) == L.FA3Q_ERR_SHAPE
    assert call(v=_p(8)) == L.FA3Q_ERR_ALIGN
    assert call(o=_p(4)) == L.FA3Q_ERR_ALIGN
    assert call(ws=None) == L.FA3Q_ERR_WORKSPACE
    assert call(wsb=64) == L.FA3Q_ERR_WORKSPACE
    assert call(ws=_p(128)) == L.FA3Q_ERR_ALIGN



@no_gpu_only
def test_decode_noalloc_rejections():
    f = fa.lib().fa3q_decode_attn_noalloc
    ok = dict(q=_p(), kq=_p(), s=_p(), kr=_p(), v=_p(), B=8, H=128, T=32768, Dn=128, Dr=64, Dv=128,
              sm=0.07, o=_p())

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["kq"], a["s"], a["kr"], a["v"], a["B"], a["H"], a["T"], a["Dn"], a["Dr"], a["Dv"],
                 ctypes.c_float(a["sm"]), a["o"], None)

    for name in ("q", "kq", "s", "kr", "v", "o"):
        assert call(**{name: None}) == L.FA3Q_ERR_NULL, name
    assert call(T=0) == L.FA3Q_ERR_SHAPE
    assert call(Dn=120) == L.FA3Q_ERR_SHAPE
    assert call(Dv=96) == L.FA3Q_ERR_SHAPE
    assert call(v=_p(8)) == L.FA3Q_ERR_ALIGN
    # split states beyond the static array: rejected before any HIP call
    lib = fa.lib()
    for B, H, T, Dv in ((64, 128, 32768, 128), (8, 128, 1 << 20, 512)):
        assert lib.fa3q_decode_attn_workspace_bytes(B, H, T, Dv) > L.FA3Q_NOALLOC_SCRATCH_BYTES
        assert call(B=B, H=H, T=T, Dv=Dv) == L.FA3Q_ERR_SCRATCH
    assert fa.status_string(L.FA3Q_ERR_SCRATCH).startswith("FA3Q_ERR_SCRATCH")


def test_noalloc_scratch_covers_the_long_context_decode():
    lib = fa.lib()
    # the long-context decode (B=8, H=128, T=32768, Dv=128) and B*H=1024 up to T=65536 fit
    assert 0 < lib.fa3q_decode_attn_workspace_bytes(8, 128, 32768, 128) <= L.FA3Q_NOALLOC_SCRATCH_BYTES
    assert lib.fa3q_decode_attn_workspace_bytes(8, 128, 65536, 128) <= L.FA3Q_NOALLOC_SCRATCH_BYTES


@no_gpu_only
def test_decode_append_rejections():
    f = fa.lib().fa3q_decode_append_attn
    ok = dict(q=_p(), kn=_p(), vn=_p(), s=_p(), kq=_p(), kr=_p(), v=_p(), kl=_p(), B=8, H=128, T=32768, Dn=128,
              Dr=64, Dv=128, sm=0.07, o=_p(), ws=_p(), wsb=1 << 30)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["kn"], a["vn"], a["s"], a["kq"], a["kr"], a["v"], a["kl"], a["B"], a["H"], a["T"],
                 a["Dn"], a["Dr"], a["Dv"], ctypes.c_float(a["sm"]), a["o"], a["ws"], a["wsb"], None)

    for name in ("q", "s", "kq", "kr", "v", "kl", "o"):
        assert call(**{name: None}) == L.FA3Q_ERR_NULL, name
    # the new token comes whole or not at all
    assert call(vn=None) == L.FA3Q_ERR_NULL
    assert call(kn=None) == L.FA3Q_ERR_NULL
    assert call(T=0) == L.FA3Q_ERR_SHAPE
    assert call(Dn=120) == L.FA3Q_ERR_SHAPE
    assert call(Dv=96) == L.FA3Q_ERR_SHAPE
    assert call(sm=float("nan")) == L.FA3Q_ERR_SHAPE
    assert call(kn=_p(8)) == L.FA3Q_ERR_ALIGN
    assert call(vn=_p(8)) == L.FA3Q_ERR_ALIGN
    assert call(kl=_p(2)) == L.FA3Q_ERR_ALIGN
    assert call(ws=None) == L.FA3Q_ERR_WORKSPACE
    assert call(ws=_p(128)) == L.FA3Q_ERR_ALIGN


@no_gpu_only
def test_decode_paged_rejections():
    f = fa.lib().fa3q_decode_paged_attn
    ok = dict(q=_p(), kn=_p(), vn=_p(), s=_p(), kq=_p(), kr=_p(), v=_p(), bt=_p(), kl=_p(), B=8, H=128, NP=4096,
              P=64, MP=512, Dn=128, Dr=64, Dv=128, sm=0.07, o=_p(), ws=_p(), wsb=1 << 30)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["kn"], a["vn"], a["s"], a["kq"], a["kr"], a["v"], a["bt"], a["kl"], a["B"], a["H"],
                 a["NP"], a["P"], a["MP"], a["Dn"], a["Dr"], a["Dv"], ctypes.c_float(a["sm"]), a["o"], a["ws"],
                 a["wsb"], None)

    for name in ("q", "s", "kq", "kr", "v", "bt", "kl", "o"):
        assert call(**{name: None}) == L.FA3Q_ERR_NULL, name
    assert call(vn=None) == L.FA3Q_ERR_NULL
    for bad in (0, 8, 48, 1 << 17):                      # pages: a power of two, 16 .. 65536
        assert call(P=bad) == L.FA3Q_ERR_SHAPE, bad
    assert call(NP=0) == L.FA3Q_ERR_SHAPE
    assert call(MP=0) == L.FA3Q_ERR_SHAPE
    assert call(B=0) == L.FA3Q_ERR_SHAPE
    assert call(Dn=120) == L.FA3Q_ERR_SHAPE
    assert call(bt=_p(2)) == L.FA3Q_ERR_ALIGN
    assert call(kq=_p(8)) == L.FA3Q_ERR_ALIGN
    assert call(kl=_p(2)) == L.FA3Q_ERR_ALIGN
    # the workspace is sized for T = max_pages * page_size
    need = fa.lib().fa3q_decode_attn_workspace_bytes(8, 128, 512 * 64, 128)
    assert need > 0
    assert call(wsb=need - 1) == L.FA3Q_ERR_WORKSPACE
    assert call(ws=None) == L.FA3Q_ERR_WORKSPACE


@no_gpu_only
def test_decode_qkv8_rejections():
    f = fa.lib().fa3q_decode_attn_qkv8
    ok = dict(qq=_p(), qr=_p(), sq=_p(), kq=_p(), sk=_p(), kr=_p(), vq=_p(), sv=_p(), B=8, H=128, T=32768, Dn=128,
              Dr=64, Dv=128, sm=0.07, o=_p(), ws=_p(), wsb=1 << 30)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["qq"], a["qr"], a["sq"], a["kq"], a["sk"], a["kr"], a["vq"], a["sv"], a["B"], a["H"], a["T"],
                 a["Dn"], a["Dr"], a["Dv"], ctypes.c_float(a["sm"]), a["o"], a["ws"], a["wsb"], None)

    for name in ("qq", "qr", "sq", "kq", "sk", "kr", "vq", "sv", "o"):
        assert call(**{name: None}) == L.FA3Q_ERR_NULL, name
    assert call(Dv=8) == L.FA3Q_ERR_SHAPE      # INT8 values need 16 per lane
    assert call(Dv=96) == L.FA3Q_ERR_SHAPE
    assert call(Dn=120) == L.FA3Q_ERR_SHAPE
    assert call(qq=_p(8)) == L.FA3Q_ERR_ALIGN
    assert call(vq=_p(8)) == L.FA3Q_ERR_ALIGN
    assert call(sv=_p(2)) == L.FA3Q_ERR_ALIGN
    assert call(ws=None) == L.FA3Q_ERR_WORKSPACE

@no_gpu_only
def test_fake_quant_rejections():
    f = fa.lib().fa3q_fake_quant
    ok = dict(x=_p(), s=_p(), y=_p(1 << 20), B=1, H=4, S=64, Dn=32, Dr=16)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["s"], a["y"], a["B"], a["H"], a["S"], a["Dn"], a["Dr"], None)

    for name in ("x", "s", "y"):
        assert call(**{name: None}) == L.FA3Q_ERR_NULL, name
    assert call(B=0) == L.FA3Q_ERR_SHAPE
    assert call(Dn=24) == L.FA3Q_ERR_SHAPE
    assert call(Dr=12) == L.FA3Q_ERR_SHAPE
    assert call(x=_p(8)) == L.FA3Q_ERR_ALIGN
    assert call(y=_p(8)) == L.FA3Q_ERR_ALIGN
    assert call(s=_p(2)) == L.FA3Q_ERR_ALIGN
    # 4 * 64 rows of 48 bf16 = 24 KiB: y starting 16 bytes in (or ending 16 bytes in) overlaps x
    assert call(y=_p(16)) == L.FA3Q_ERR_ALIAS
    assert call(x=_p(16), y=_p()) == L.FA3Q_ERR_ALIAS
    assert call(y=_p(24576 - 16)) == L.FA3Q_ERR_ALIAS
    assert fa.status_string(L.FA3Q_ERR_ALIAS).startswith("FA3Q_ERR_ALIAS")


@no_gpu_only
def test_quantize_asym_rejections():
    f = fa.lib().fa3q_quantize_asym
    ok = dict(k=_p(), s=_p(), o=_p(), dt=L.FA3Q_BF16, q=_p(), r=_p(), B=1, H=4, S=64, Dn=32, Dr=16)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["k"], a["s"], a["o"], a["dt"], a["q"], a["r"], a["B"], a["H"], a["S"], a["Dn"], a["Dr"], None)

    for name in ("k", "s", "o", "q", "r"):
        assert call(**{name: None}) == L.FA3Q_ERR_NULL, name
    assert call(dt=L.FA3Q_F32) == L.FA3Q_ERR_DTYPE
    assert call(dt=7) == L.FA3Q_ERR_DTYPE
    assert call(S=0) == L.FA3Q_ERR_SHAPE
    assert call(Dn=24) == L.FA3Q_ERR_SHAPE
    assert call(Dr=12) == L.FA3Q_ERR_SHAPE
    assert call(k=_p(8)) == L.FA3Q_ERR_ALIGN
    assert call(s=_p(8)) == L.FA3Q_ERR_ALIGN   # tables are read 16 bytes at a time
    assert call(o=_p(4)) == L.FA3Q_ERR_ALIGN
    assert call(q=_p(4)) == L.FA3Q_ERR_ALIGN


@no_gpu_only
def test_decode_asym_rejections():
    f = fa.lib().fa3q_decode_attn_asym
    ok = dict(q=_p(), kq=_p(), s=_p(), of=_p(), dt=L.FA3Q_F16, kr=_p(), v=_p(), B=8, H=128, T=32768, Dn=128,
              Dr=64, Dv=128, sm=0.07, o=_p(), ws=_p(), wsb=1 << 30)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["kq"], a["s"], a["of"], a["dt"], a["kr"], a["v"], a["B"], a["H"], a["T"], a["Dn"],
                 a["Dr"], a["Dv"], ctypes.c_float(a["sm"]), a["o"], a["ws"], a["wsb"], None)

    for name in ("q", "kq", "s", "of", "kr", "v", "o"):
        assert call(**{name: None}) == L.FA3Q_ERR_NULL, name
    assert call(dt=L.FA3Q_F32) == L.FA3Q_ERR_DTYPE
    assert call(dt=3) == L.FA3Q_ERR_DTYPE
    assert call(T=0) == L.FA3Q_ERR_SHAPE
    assert call(Dn=120) == L.FA3Q_ERR_SHAPE
    assert call(Dv=96) == L.FA3Q_ERR_SHAPE
    assert call(s=_p(8)) == L.FA3Q_ERR_ALIGN
    assert call(of=_p(2)) == L.FA3Q_ERR_ALIGN
    assert call(v=_p(8)) == L.FA3Q_ERR_ALIGN
    assert call(ws=None) == L.FA3Q_ERR_WORKSPACE


@no_gpu_only
def test_decode_latent_rejections():
    lib = fa.lib()
    f = lib.fa3q_decode_latent
    ok = dict(q=_p(), c=_p(), s=_p(), kr=_p(), B=64, H=128, T=4096, Dl=512, Dr=64, sm=0.07, o=_p(), ws=_p(),
              wsb=1 << 30)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["c"], a["s"], a["kr"], a["B"], a["H"], a["T"], a["Dl"], a["Dr"], ctypes.c_float(a["sm"]),
                 a["o"], a["ws"], a["wsb"], None)

    for name in ("q", "c", "s", "kr", "o"):
        assert call(**{name: None}) == L.FA3Q_ERR_NULL, name
    assert call(kr=None, Dr=0, o=_p(4)) == L.FA3Q_ERR_ALIGN   # no RoPE part: NULL accepted, stops at `out`
    assert call(Dl=192) == L.FA3Q_ERR_SHAPE
    assert call(Dr=16) == L.FA3Q_ERR_SHAPE      # RoPE width a multiple of 32 (MFMA k-step)
    assert call(T=0) == L.FA3Q_ERR_SHAPE
    assert call(H=0) == L.FA3Q_ERR_SHAPE
    assert call(sm=float("inf")) == L.FA3Q_ERR_SHAPE
    assert call(q=_p(8)) == L.FA3Q_ERR_ALIGN
    assert call(o=_p(4)) == L.FA3Q_ERR_ALIGN
    assert call(s=_p(2)) == L.FA3Q_ERR_ALIGN
    assert call(ws=None) == L.FA3Q_ERR_WORKSPACE
    assert call(wsb=64) == L.FA3Q_ERR_WORKSPACE
    assert call(ws=_p(128)) == L.FA3Q_ERR_ALIGN
    assert lib.fa3q_decode_latent_workspace_bytes(64, 128, 4096, 512) > 0
    assert lib.fa3q_decode_latent_workspace_bytes(64, 128, 4096, 192) == 0
    # one split: no partial outputs; 128 heads or more still take one flag word per wave of the
    # 32-head kernel (which gives a split up on scores that outgrow its reference)
    assert lib.fa3q_decode_latent_workspace_bytes(1024, 64, 64, 512) == 0
    assert lib.fa3q_decode_latent_workspace_bytes(1024, 128, 64, 512) == 1024 * 4 * 4


@no_gpu_only
def test_calibrate_batches_rejections():
    lib = fa.lib()
    f = lib.fa3q_calibrate_batches
    shape = (8, 128, 2048, 128)
    need = lib.fa3q_calibrate_batches_workspace_bytes(L.FA3Q_BF16, 4, *shape, 0.9999)
    assert need >= 2 * 4 * 128 * 4  # at least the per-batch windows it keeps
    assert lib.fa3q_calibrate_batches_workspace_bytes(L.FA3Q_BF16, 0, *shape, 0.9999) == 0
    assert lib.fa3q_calibrate_batches_workspace_bytes(L.FA3Q_BF16, 17, *shape, 0.9999) == 0

    def call(xs=None, nb=4, dt=L.FA3Q_BF16, ratio=0.9999, rmin=_p(), rmax=_p(), wmin=None, wmax=None, ws=_p(),
             wsb=None):
        ptrs = (ctypes.c_void_p * 4)(*(xs if xs is not None else [FAKE] * 4))
        return f(ptrs, nb, dt, *shape, ratio, rmin, rmax, 1, wmin, wmax, ws, need if wsb is None else wsb, None)

    assert call(rmin=None) == L.FA3Q_ERR_NULL
    assert call(wmin=_p()) == L.FA3Q_ERR_NULL                 # one window array without the other
    assert call(xs=[FAKE, FAKE, 0, FAKE]) == L.FA3Q_ERR_NULL
    assert call(nb=0) == L.FA3Q_ERR_SHAPE
    assert call(nb=17) == L.FA3Q_ERR_SHAPE
    assert call(dt=9) == L.FA3Q_ERR_DTYPE
    assert call(ratio=0.0) == L.FA3Q_ERR_RATIO
    assert call(xs=[FAKE, FAKE + 8, FAKE, FAKE]) == L.FA3Q_ERR_ALIGN
    assert call(rmax=_p(2)) == L.FA3Q_ERR_ALIGN
    assert call(ws=None) == L.FA3Q_ERR_WORKSPACE
    assert call(wsb=64) == L.FA3Q_ERR_WORKSPACE
    assert call(ws=_p(128)) == L.FA3Q_ERR_ALIGN


def test_binding_refuses_mismatched_asym_tables():
    import torch
    k = torch.zeros((1, 2, 16, 48), dtype=torch.bfloat16)
    s = torch.ones((2, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa3q_quantize_asym(k, s, s.to(torch.float16), 32)     # mixed table dtypes
    with pytest.raises(ValueError):
        fa.fa3q_quantize_asym(k, s[:, :16], s[:, :16], 32)       # wrong table shape
    with pytest.raises(ValueError):
        fa.fa3q_quantize_asym(k, s.float(), s.float(), 32)       # float32 tables
    with pytest.raises(ValueError):
        fa.fa3q_quantize_asym(k, s, s, 32)                       # host tensors


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros((1, 4, 64, 32), dtype=torch.float32)
    with pytest.raises(ValueError):
        fa.fa3q_calibrate_perhead(x, 0.9)
    with pytest.raises(TypeError):
        fa.fa3q_calibrate_perhead(x.to(torch.float64), 0.9)


def test_binding_checks_every_tensor_before_a_launch():
    # host tensors throughout: each wrong dtype or size must be named before the device check
    import torch
    B, H, T, Dn, Dr, Dv = 2, 4, 32, 32, 16, 32
    q = torch.zeros((B, H, Dn + Dr), dtype=torch.bfloat16)
    kq = torch.zeros((B, H, T, Dn), dtype=torch.int8)
    kr = torch.zeros((B, H, T, Dr), dtype=torch.bfloat16)
    v = torch.zeros((B, H, T, Dv), dtype=torch.bfloat16)
    scale = torch.ones(H, dtype=torch.float32)

    def raises(match, fn, *args, **kw):
        with pytest.raises(ValueError, match=match):
            fn(*args, **kw)

    raises("scale must be float32", fa.fa3q_decode_attn, q, kq, scale.to(torch.bfloat16), kr, v, 0.1)
    raises("scale must be float32 with 4", fa.fa3q_decode_attn, q, kq, scale[:3], kr, v, 0.1)
    raises("out must be", fa.fa3q_decode_attn, q, kq, scale, kr, v, 0.1, out=torch.empty((B, H, Dv - 1)))
    raises("out must be", fa.fa3q_decode_attn, q, kq, scale, kr, v, 0.1,
           out=torch.empty((B, H, Dv), dtype=torch.float16))
    raises("v must be", fa.fa3q_decode_attn, q, kq, scale, kr, v[:, :, :-1], 0.1)
    raises("q must be", fa.fa3q_decode_attn_ex, q.float(), kq, scale, kr, v, 0.1)
    raises("v must be", fa.fa3q_decode_attn_ex, q.half(), kq, scale, kr.half(), v, 0.1)  # mixed dtypes
    raises("layout", fa.fa3q_decode_attn_ex, q, kq, scale, kr, v, 0.1, layout="SBHD")
    raises("kv_len", fa.fa3q_decode_append_attn, q, None, None, scale, kq, kr, v,
           torch.zeros(B, dtype=torch.int64), 0.1)
    k = torch.zeros((B, H, T, Dn + Dr), dtype=torch.bfloat16)
    raises("k_nope_q must be", fa.fa3q_quantize_k, k, scale, Dn, k_nope_q=torch.empty((B, H, T - 1, Dn),
                                                                                      dtype=torch.int8))
    raises("k_rope must be", fa.fa3q_quantize_k, k, scale, Dn, k_rope=torch.empty((B, H, T, Dr)))
    raises("scale must be float32", fa.fa3q_quantize_k, k, scale.double(), Dn)
    raises("k must be bfloat16", fa.fa3q_quantize_k, k.half(), scale, Dn)
    raises("k_nope_q must be", fa.fa3q_quantize_k_ex, k.transpose(1, 2).contiguous(), scale, Dn, layout="BSHD",
           k_nope_q=torch.empty((B, H, T, Dn), dtype=torch.int8))  # codes in the other layout
    f = torch.zeros(H, dtype=torch.float32)
    raises("cur_min must be float32 with 4", fa.fa3q_accumulate_minmax, f, f, f[:2], f)
    raises("run_max must be float32", fa.fa3q_qparams, f, f.half())
    raises("scale must be float32 with 4", fa.fa3q_qparams, f, f, torch.empty(5))
    raises("run_max must be float32 with 4", fa.fa3q_init_minmax, f, torch.empty(3))
    x = torch.zeros((1, H, 64, 32), dtype=torch.float32)
    raises("run_min and run_max are required", fa.fa3q_calibrate_batches, [x], 0.9, None, f)
    raises("win_min must be float32 with 8", fa.fa3q_calibrate_batches, [x, x], 0.9, f, f,
           win_min=torch.empty(4), win_max=torch.empty(8))
    raises("given together", fa.fa3q_calibrate_ex, [x], 0.9, run_min=f)


# ----------------------------------------------------------------------------- float16 and (B,S,H,D)


def test_ex_workspace_queries():
    lib = fa.lib()
    q = lib.fa3q_calibrate_ex_workspace_bytes
    r = 0.99
    for dt in (L.FA3Q_BF16, L.FA3Q_F16):
        # the (B,H,S,D) call equals the batches call; (B,S,H,D) 16-bit input takes the histogram
        assert q(dt, L.FA3Q_BHSD, 2, 1, 8, 256, 64, r) == lib.fa3q_calibrate_batches_workspace_bytes(
            dt, 2, 1, 8, 256, 64, r) > 0
        assert q(dt, L.FA3Q_BSHD, 2, 1, 8, 256, 64, r) >= 2 * 8 * 65536 * 4
        assert q(dt, L.FA3Q_BSHD, 1, 2, 4, 16, 12, r) == 0  # rows of 12 values: not whole vectors
    assert q(L.FA3Q_F32, L.FA3Q_BHSD, 1, 1, 8, 256, 64, r) > 0
    # float32 (B,S,H,D) with rows of a power-of-two width and K within the tail lists' cap: the
    # tail lists, the same workspace as (B,H,S,D) slabs
    assert q(L.FA3Q_F32, L.FA3Q_BSHD, 2, 1, 8, 256, 64, r) == q(L.FA3Q_F32, L.FA3Q_BHSD, 2, 1, 8, 256, 64, r) > 0
    # other widths (96) and larger K: the collect-and-sort path, one region of two N-key lists per
    # head for any number of batches (they take it in turn), plus the windows of every batch
    one = q(L.FA3Q_F32, L.FA3Q_BSHD, 1, 1, 8, 256, 96, r)
    assert one >= 2 * 8 * (256 * 96) * 4
    assert 0 <= q(L.FA3Q_F32, L.FA3Q_BSHD, 4, 1, 8, 256, 96, r) - one < 4096
    assert q(L.FA3Q_F32, L.FA3Q_BSHD, 1, 4, 8, 4096, 64, 0.9) >= 2 * 8 * (4 * 4096 * 64) * 4
    assert q(L.FA3Q_F32, L.FA3Q_BSHD, 1, 2, 4, 16, 6, r) == 0  # rows of 6 float32 values: not whole vectors
    assert q(L.FA3Q_BF16, 2, 1, 1, 8, 256, 64, r) == 0
    assert q(7, L.FA3Q_BHSD, 1, 1, 8, 256, 64, r) == 0
    assert q(L.FA3Q_F16, L.FA3Q_BHSD, 17, 1, 8, 256, 64, r) == 0
    # float16 heads follow bf16's routing: the same windows cap, the same workspace
    assert lib.fa3q_calibrate_max_windows(L.FA3Q_F16) == lib.fa3q_calibrate_max_windows(L.FA3Q_BF16)
    assert lib.fa3q_calibrate_workspace_bytes(L.FA3Q_F16, 2, 8, 4096, 128, 0.999) == \
        lib.fa3q_calibrate_workspace_bytes(L.FA3Q_BF16, 2, 8, 4096, 128, 0.999)


@no_gpu_only
def test_calibrate_ex_rejections():
    f = fa.lib().fa3q_calibrate_ex
    xs = (ctypes.c_void_p * 2)(1 << 20, 2 << 20)
    ok = dict(xs=xs, nb=2, dt=L.FA3Q_F16, lay=L.FA3Q_BSHD, B=1, H=8, S=256, D=64, r=0.99, rmin=_p(), rmax=_p(),
              init=1, wmin=None, wmax=None, ws=_p(), wb=1 << 40)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["xs"], a["nb"], a["dt"], a["lay"], a["B"], a["H"], a["S"], a["D"], a["r"], a["rmin"], a["rmax"],
                 a["init"], a["wmin"], a["wmax"], a["ws"], a["wb"], None)

    assert call(lay=2) == L.FA3Q_ERR_LAYOUT
    assert call(dt=5) == L.FA3Q_ERR_DTYPE
    assert call(dt=L.FA3Q_F32, D=6) == L.FA3Q_ERR_SHAPE  # float32 rows of whole 16-byte vectors
    assert call(D=12) == L.FA3Q_ERR_SHAPE
    assert call(nb=0) == L.FA3Q_ERR_SHAPE
    assert call(r=0.0) == L.FA3Q_ERR_RATIO
    assert call(rmin=None, rmax=None) == L.FA3Q_ERR_NULL  # neither statistics nor windows
    assert call(rmax=None) == L.FA3Q_ERR_NULL
    assert call(rmin=None, rmax=None, wmin=_p(), wmax=None) == L.FA3Q_ERR_NULL
    assert call(ws=None) == L.FA3Q_ERR_WORKSPACE
    assert call(wb=16) == L.FA3Q_ERR_WORKSPACE
    assert call(xs=(ctypes.c_void_p * 2)(1 << 20, (2 << 20) + 8)) == L.FA3Q_ERR_ALIGN


@no_gpu_only
def test_quantize_k_ex_rejections():
    f = fa.lib().fa3q_quantize_k_ex
    ok = dict(k=_p(), s=_p(), kq=_p(), kr=_p(), dt=L.FA3Q_F16, lay=L.FA3Q_BSHD, B=2, H=4, S=16, Dn=128, Dr=64)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["k"], a["s"], a["kq"], a["kr"], a["dt"], a["lay"], a["B"], a["H"], a["S"], a["Dn"], a["Dr"], None)

    assert call(lay=7) == L.FA3Q_ERR_LAYOUT
    assert call(dt=L.FA3Q_F32) == L.FA3Q_ERR_DTYPE
    for name in ("k", "s", "kq", "kr"):
        assert call(**{name: None}) == L.FA3Q_ERR_NULL, name
    assert call(Dn=120) == L.FA3Q_ERR_SHAPE
    assert call(kr=_p(8)) == L.FA3Q_ERR_ALIGN


@no_gpu_only
def test_decode_ex_rejections():
    lib = fa.lib()
    ok = dict(q=_p(), kq=_p(), s=_p(), kr=_p(), v=_p(), dt=L.FA3Q_F16, lay=L.FA3Q_BSHD, B=2, H=4, T=512, Dn=128,
              Dr=64, Dv=128, sm=0.07, o=_p(), ws=_p(), wb=1 << 30)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.fa3q_decode_attn_ex(a["q"], a["kq"], a["s"], a["kr"], a["v"], a["dt"], a["lay"], a["B"], a["H"],
                                       a["T"], a["Dn"], a["Dr"], a["Dv"], ctypes.c_float(a["sm"]), a["o"], a["ws"],
                                       a["wb"], None)

    def append(**kw):
        a = dict(ok, **kw)
        return lib.fa3q_decode_append_attn_ex(a["q"], _p(), _p(), a["s"], a["kq"], a["kr"], a["v"], _p(), a["dt"],
                                              a["lay"], a["B"], a["H"], a["T"], a["Dn"], a["Dr"], a["Dv"],
                                              ctypes.c_float(a["sm"]), a["o"], a["ws"], a["wb"], None)

    for fn in (call, append):
        assert fn(lay=-1) == L.FA3Q_ERR_LAYOUT
        assert fn(dt=L.FA3Q_F32) == L.FA3Q_ERR_DTYPE
        assert fn(q=None) == L.FA3Q_ERR_NULL
        assert fn(Dv=96) == L.FA3Q_ERR_SHAPE
        assert fn(v=_p(8)) == L.FA3Q_ERR_ALIGN
