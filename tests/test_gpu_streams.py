"""The binding on a side stream: outputs and workspaces allocated by the wrapper belong to
the stream the kernels run on, and the results equal those of the same calls on torch's
current stream (bit for bit: same kernels, same plans)."""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_bits_equal, log

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def fa():
    import kv_cache_quantization_fa3q_amd as m
    return m


def _path(fa, stream):
    """calibration, statistics, scale, quantisation and decode, every output and workspace made
    by the wrapper on `stream`."""
    B, H, S, D = 2, 8, 1024, 64
    T, Dn, Dr, Dv = 6000, 128, 64, 128
    sigma = synth.head_sigmas(H, seed=31)
    x = synth.activations((B, H, S, D), sigma, outlier_frac=0.001, dtype=torch.bfloat16, seed=32).to(DEV)
    k = synth.activations((B, H, T, Dn + Dr), sigma, dtype=torch.bfloat16, seed=33).to(DEV)
    v = synth.activations((B, H, T, Dv), sigma, dtype=torch.bfloat16, seed=34).to(DEV)
    q = synth.normal_tensor((B, H, Dn + Dr), dtype=torch.bfloat16, seed=35).to(DEV)
    torch.cuda.synchronize()  # inputs ready before a side stream reads them
    wmin, wmax = fa.fa3q_calibrate_perhead(x, 0.999, stream=stream)
    scale = fa.fa3q_qparams(wmin, wmax, stream=stream)
    kq, kr = fa.fa3q_quantize_k(k, scale, Dn, stream=stream)
    out = fa.fa3q_decode_attn(q, kq, scale, kr, v, 1.0 / math.sqrt(Dn + Dr), stream=stream)
    return [wmin, wmax, scale, kq, kr.view(torch.int16), out]


def test_side_stream_results_equal_current_stream(fa):
    log("binding on the current stream")
    ref = [t.cpu().numpy() for t in _path(fa, None)]
    torch.cuda.synchronize()
    for kind in ("torch stream", "raw handle"):
        s = torch.cuda.Stream()
        log(f"binding on a side stream ({kind})")
        got = _path(fa, s if kind == "torch stream" else s.cuda_stream)
        s.synchronize()
        for i, (g, r) in enumerate(zip(got, ref)):
            assert_bits_equal(g.cpu().numpy(), r, f"{kind}: output {i}")


def test_side_stream_workspace_is_not_reused_early(fa):
    # many back-to-back calls on a side stream whose workspaces the wrapper frees at once: each
    # result must still be that of its own inputs
    B, H, T, Dn, Dr, Dv = 4, 16, 8192, 128, 64, 128  # several splits: a workspace is needed
    assert fa.fa3q_decode_attn_workspace_bytes(B, H, T, Dv) > 0
    g = np.random.default_rng(36)
    kq = torch.from_numpy(g.integers(-127, 128, size=(B, H, T, Dn)).astype(np.int8)).to(DEV)
    sigma = synth.head_sigmas(H, seed=37)
    kr = synth.activations((B, H, T, Dr), sigma, dtype=torch.bfloat16, seed=38).to(DEV)
    v = synth.activations((B, H, T, Dv), sigma, dtype=torch.bfloat16, seed=39).to(DEV)
    scale = (sigma * 4.0 / 127.0).to(torch.float32).to(DEV)
    qs = [synth.normal_tensor((B, H, Dn + Dr), dtype=torch.bfloat16, seed=40 + i).to(DEV) for i in range(8)]
    sm = 1.0 / math.sqrt(Dn + Dr)
    torch.cuda.synchronize()
    ref = [fa.fa3q_decode_attn(q, kq, scale, kr, v, sm).cpu().numpy() for q in qs]
    s = torch.cuda.Stream()
    log("eight decode calls on a side stream, wrapper-owned workspaces")
    outs = [fa.fa3q_decode_attn(q, kq, scale, kr, v, sm, stream=s) for q in qs]
    s.synchronize()
    for i, (o, r) in enumerate(zip(outs, ref)):
        assert_bits_equal(o.cpu().numpy(), r, f"call {i}")
