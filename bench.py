#!/usr/bin/env python3
"""Benchmark of the FA3 per-head INT8 hot path on one MI355X.

One step runs every stage once, on inputs already resident in HBM:
  1. calibrate   4 batches of bf16 activations (8,128,2048,128), Student-t(3) tails,
                 ratio 0.9999 (N = 2,097,152 values and K = 211 windows per head)
  2. accumulate  running per-head min/max over the 4 batches (after an init)
  3. qparams     scale[h] = abs_max / 127
  4. quantize    K of 64 sequences x 4096 tokens, H=128, 128 nope + 64 rope dims, bf16
                 -> int8 K-nope cache + bf16 K-rope (scales from step 3)
  5. decode      batch 64, 128 heads, one query each over the 4096 cached tokens of
                 step 4 plus bf16 V (128 dims), softmax scale 1/sqrt(192)

Prints one JSON line.  ``value`` is the step's algorithmic HBM bytes divided by its
wall time (GB/s); per-stage figures (calib Gelem/s, quantize GB/s, decode KV GB/s, each
as a fraction of the 8 TB/s HBM peak) are under ``breakdown``; ``roofline`` is for the
kernel that takes the most time, timed with HIP events on the stream it runs on;
``cpu_baseline`` is the CPU oracle timed on a bounded sample of the same workload, on a
pool of worker processes (one per host core the process may use, at most 16).

Measurements outside the step (``breakdown`` entries after the four stages) can be
narrowed with ``--only name,name`` for profiling runs.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
METRIC = "calib Gelem/s; quantize GB/s; decode-attn KV GB/s (fraction of HBM peak)"

# workload shapes
H = 128
CAL_SHAPE = (8, H, 2048, 128)
CAL_BATCHES = 4
RATIO = 0.9999
QB, QS, DN, DR = 64, 4096, 128, 64
DV = 128

CAL_BYTES = 2 * math.prod(CAL_SHAPE)                            # per batch, bf16 read once
QUANT_BYTES = QB * H * QS * (2 * (DN + DR) + DN + 2 * DR)       # 640 B per (token, head)
DEC_BYTES = QB * H * QS * (DN + 2 * DR + 2 * DV) + QB * H * (2 * (DN + DR) + 4 * DV)  # 512 B per (b,h,t) + q + out
COPY_BYTES = 1 << 30  # device-to-device copy reference (read + write of 1 GiB each)
LONG_SHAPE = (2, H, 16384, 128)  # long-context calibration tensor
LONG_RATIOS = (0.999, 0.9999, 0.99999)

# kernel -> the sources its code comes from (the committed counter summary names their hash)
KERNEL_SOURCES = {
    "quantize_k_kernel": ("quantize.hip", "fa3q_internal.hpp"),
    "decode_split_kernel": ("decode.hip", "fa3q_internal.hpp"),
    "calib_hist_kernel": ("calib_hist.hip", "calib_hist.hpp", "calibrate.hip", "fa3q_internal.hpp"),
}
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "fa3q_step_hbm_traffic.md")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of CPU oracle work for the baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="comma-separated measurements outside the step to run (default: all): " + ", ".join(EXTRAS))
    return ap.parse_args()


def source_hash(kernel: str) -> str:
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "kv_cache_quantization_fa3q_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_summary(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when the
    summary is missing or was taken on different kernel sources."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None, "no counter summary"
    start = text.find("```json")
    if start < 0:
        return None, "counter summary has no json block"
    end = text.find("```", start + 7)
    try:
        entries = json.loads(text[start + 7:end])
    except ValueError:
        return None, "counter summary json unreadable"
    e = entries.get(kernel)
    if not e:
        return None, f"no counters for {kernel}"
    if e.get("source_sha256_16") != source_hash(kernel):
        return None, f"{kernel} changed since its counters were taken"
    return float(e["hbm_bytes_per_launch"]), f"{os.path.relpath(TRAFFIC_SUMMARY, ROOT)} (sources {e['source_sha256_16']})"


# ----------------------------------------------------------------------------- CPU oracle baseline
#
# The oracle as it stands, timed on the host's cores: a pool of spawned worker processes
# (one BLAS/OpenMP thread each) reads the same synthetic inputs from shared memory and runs
# the oracle's own functions on whole heads (calibration), (sequence, 8 heads) slices
# (quantisation) and (sequence, 4 heads) slices (decode).  Each stage runs rounds of one
# task per worker until its share of the budget is spent; its rate is the work done over
# the stage's wall time.

_SHM = {}


def _cpu_worker_init():
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        os.environ[var] = "1"


def _shm_array(name, shape, dtype):
    import numpy as np
    from multiprocessing import shared_memory

    if name not in _SHM:
        _SHM[name] = shared_memory.SharedMemory(name=name)
    return np.ndarray(shape, dtype=dtype, buffer=_SHM[name].buf)


def _cpu_task(task):
    """One oracle call in a worker on inputs in shared memory; returns the units it covered."""
    import numpy as np

    import oracle

    kind, spec, arg = task
    if kind == "calib":
        x = _shm_array(*spec["x"])
        head = oracle.bf16_bits_to_f32(x[:, arg].reshape(-1))
        oracle.recall_window(head, RATIO)
        return head.size
    if kind == "quant":
        b, h0 = arg
        k = _shm_array(*spec["k"])
        scale = _shm_array(*spec["scale"])
        kb = np.ascontiguousarray(k[b:b + 1, h0:h0 + 8])
        oracle.quantize_k(kb, scale[h0:h0 + 8], DN)
        return kb.size // (DN + DR) * (2 * (DN + DR) + DN + 2 * DR)
    if kind == "decode":
        b, h0 = arg
        kq, kr, v, q = (_shm_array(*spec[n]) for n in ("kq", "kr", "v", "q"))
        scale = _shm_array(*spec["scale"])
        sl = (slice(b, b + 1), slice(h0, h0 + 4))
        oracle.decode_attn(q[sl], kq[sl], scale[h0:h0 + 4], kr[sl], v[sl], 1.0 / math.sqrt(DN + DR))
        return 4 * kq.shape[2] * (DN + 2 * DR + 2 * DV)
    raise ValueError(kind)


def _host_info():
    model, mem = None, None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    mem = int(line.split()[1]) * 1024
                    break
    except OSError:
        pass
    return model or platform.processor() or platform.machine(), mem


def cpu_pool(workers: int):
    """The worker pool, started before the GPU is touched (spawned interpreters that only run the oracle)."""
    import multiprocessing as mp

    return mp.get_context("spawn").Pool(workers, initializer=_cpu_worker_init)


def cpu_baseline(pool, workers: int, inputs, budget_s: float):
    """Oracle throughput on `workers` host processes over the same workload (bounded sample)."""
    import numpy as np
    import torch
    from multiprocessing import shared_memory

    owned = []

    def share(name, t):
        a = t.detach().contiguous().cpu()
        if a.dtype in (torch.bfloat16, torch.float16):
            a = a.view(torch.int16)
        arr = a.numpy()
        if arr.dtype == np.int16:
            arr = arr.view(np.uint16)
        shm = shared_memory.SharedMemory(create=True, size=max(1, arr.nbytes))
        owned.append(shm)
        np.ndarray(arr.shape, dtype=arr.dtype, buffer=shm.buf)[...] = arr
        return (shm.name, arr.shape, arr.dtype.str)

    NS = 4  # sequences of the quantisation / decode workload shared with the workers
    try:
        spec = {
            "x": share("x", inputs["calib"][0]),
            "k": share("k", inputs["k"][:NS]),
            "scale": share("scale", inputs["scale"]),
            "kq": share("kq", inputs["kq"][:NS]),
            "kr": share("kr", inputs["kr"][:NS]),
            "v": share("v", inputs["v"][:NS]),
            "q": share("q", inputs["q"][:NS]),
        }
        per_stage = budget_s / 3.0

        def stage(kind, args):
            # one task per worker first (it also attaches the shared inputs), then as many more as
            # the stage's budget allows at that pace, in one map so no worker waits on a round
            t0 = time.perf_counter()
            done = sum(pool.map(_cpu_task, [(kind, spec, a) for a in args[:workers]], chunksize=1))
            first = time.perf_counter() - t0
            rounds = int(max(0.0, per_stage - first) / max(first, 1e-3))
            rest = args[workers:workers + workers * rounds]
            if rest:
                done += sum(pool.map(_cpu_task, [(kind, spec, a) for a in rest], chunksize=1))
            return done / (time.perf_counter() - t0), min(len(args), workers) + len(rest)

        cal_rate, n_heads = stage("calib", list(range(H)))
        q_rate, n_q = stage("quant", [(b, h0) for b in range(NS) for h0 in range(0, H, 8)])
        d_rate, n_d = stage("decode", [(b, h0) for b in range(NS) for h0 in range(0, H, 4)])
    finally:
        for shm in owned:
            shm.close()
            shm.unlink()
    step_s = CAL_BATCHES * CAL_BYTES / (2 * cal_rate) + QUANT_BYTES / q_rate + DEC_BYTES / d_rate
    total = CAL_BATCHES * CAL_BYTES + QUANT_BYTES + DEC_BYTES
    model, mem = _host_info()
    return {
        "value": total / step_s / 1e9,
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"{n_heads} whole heads of one calibration batch (2,097,152 values each), {n_q} x "
                   f"(sequence, 8 heads x 4096 tokens) of K quantisation, {n_d} x (sequence, 4 heads) decode slices "
                   f"over 4096 tokens, on {workers} worker processes with one BLAS thread each; rates scaled to one "
                   "full step by the step's bytes per stage"),
        "stages": {"calib_gelem_s": cal_rate / 1e9, "quantize_gbs": q_rate / 1e9, "decode_kv_gbs": d_rate / 1e9},
        "cpu": model,
        "host_mem_bytes": mem,
        "host_threads_available": len(os.sched_getaffinity(0)),
    }


EXTRAS = ("decode_append", "decode_qkv8", "asym", "fake_quant", "decode_latent", "calibrate_long",
          "calibrate_largek", "calibrate_f32", "decode_long", "decode_noalloc", "decode_paged", "f16_bshd")


def main() -> int:
    args = parse()
    if args.gpus != 1:
        log("bench.py measures one GPU: this build has no multi-GPU path (each GPU would run its own "
            "heads or sequences with no exchange); run with --gpus 1")
        return 2
    only = set(EXTRAS) if args.only is None else {e for e in args.only.split(",") if e}
    unknown = only - set(EXTRAS)
    if unknown:
        log(f"unknown --only entries {sorted(unknown)}; choose from {', '.join(EXTRAS)}")
        return 2
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    pool = None if args.no_cpu_baseline else cpu_pool(workers)  # before the GPU is touched
    try:
        return run(args, only, pool, workers)
    finally:
        if pool is not None:
            pool.terminate()
            pool.join()


def run(args, only, pool, workers) -> int:
    import torch

    import kv_cache_quantization_fa3q_amd as fa
    import synth

    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} CUs={props.multi_processor_count} mem={props.total_memory / 2**30:.0f} GiB "
        f"lib={fa.library_path()}")

    t_setup = time.perf_counter()
    sigma = synth.head_sigmas(H, seed=2024)
    calib = [synth.activations(CAL_SHAPE, sigma, law="t3", dtype=torch.bfloat16, seed=100 + i, device=dev)
             for i in range(CAL_BATCHES)]
    k = synth.activations((QB, H, QS, DN + DR), sigma, law="normal", outlier_frac=0.0005, outlier_mult=40.0,
                          dtype=torch.bfloat16, seed=200, device=dev)
    v = synth.activations((QB, H, QS, DV), sigma, law="normal", dtype=torch.bfloat16, seed=300, device=dev)
    q = synth.normal_tensor((QB, H, DN + DR), dtype=torch.bfloat16, seed=400, device=dev)
    kq = torch.empty((QB, H, QS, DN), dtype=torch.int8, device=dev)
    kr = torch.empty((QB, H, QS, DR), dtype=torch.bfloat16, device=dev)
    out = torch.empty((QB, H, DV), dtype=torch.float32, device=dev)
    run_min = torch.empty(H, dtype=torch.float32, device=dev)
    run_max = torch.empty(H, dtype=torch.float32, device=dev)
    scale = torch.empty(H, dtype=torch.float32, device=dev)
    ws_cal = torch.empty(max(1, fa.fa3q_calibrate_batches_workspace_bytes(torch.bfloat16, CAL_BATCHES, *CAL_SHAPE,
                                                                          RATIO)), dtype=torch.uint8, device=dev)
    dec_ws_bytes = fa.fa3q_decode_attn_workspace_bytes(QB, H, QS, DV)
    ws_dec = torch.empty(dec_ws_bytes, dtype=torch.uint8, device=dev) if dec_ws_bytes else None
    sm = 1.0 / math.sqrt(DN + DR)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t_setup:.1f} s")

    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        # every calibration batch's windows folded into the running min/max, in one call
        fa.fa3q_calibrate_batches(calib, RATIO, run_min, run_max, True, workspace=ws_cal, stream=stream)
        if ev:
            ev[1].record(stream)
        fa.fa3q_qparams(run_min, run_max, scale, stream=stream)
        if ev:
            ev[2].record(stream)
        fa.fa3q_quantize_k(k, scale, DN, kq, kr, stream=stream)
        if ev:
            ev[3].record(stream)
        fa.fa3q_decode_attn(q, kq, scale, kr, v, sm, out, ws_dec, stream=stream)
        if ev:
            ev[4].record(stream)

    for i in range(args.warmup):
        step()
        log(f"warmup step {i + 1}/{args.warmup} enqueued")
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall:.3f} s")

    def avg(a, b):
        return sum(events[i][a].elapsed_time(events[i][b]) for i in range(args.steps)) / args.steps  # ms

    cal_ms, qp_ms, quant_ms, dec_ms = avg(0, 1), avg(1, 2), avg(2, 3), avg(3, 4)
    ms_per_step = wall * 1e3 / args.steps
    total_bytes = CAL_BATCHES * CAL_BYTES + QUANT_BYTES + DEC_BYTES
    value = total_bytes / (ms_per_step * 1e-3) / 1e9

    def gbs(nbytes, ms):
        return nbytes / (ms * 1e-3) / 1e9

    cal_gbs = gbs(CAL_BATCHES * CAL_BYTES, cal_ms)
    quant_gbs = gbs(QUANT_BYTES, quant_ms)
    dec_gbs = gbs(DEC_BYTES, dec_ms)
    breakdown = {
        "calibrate": {"ms": cal_ms, "gelem_s": CAL_BATCHES * CAL_BYTES / 2 / (cal_ms * 1e-3) / 1e9,
                      "gbs": cal_gbs, "frac_hbm": cal_gbs / HBM_PEAK_GBS,
                      "note": "4 batches in one fa3q_calibrate_batches call: per-head histograms, windows, accumulate"},
        "qparams": {"ms": qp_ms},
        "quantize": {"ms": quant_ms, "gbs": quant_gbs, "frac_hbm": quant_gbs / HBM_PEAK_GBS},
        "decode": {"ms": dec_ms, "kv_gbs": dec_gbs, "frac_hbm": dec_gbs / HBM_PEAK_GBS},
    }
    # the kernel with the largest share of the step; its events bracket exactly one launch
    stages = {"quantize_k_kernel": (quant_ms, QUANT_BYTES, 1), "decode_split_kernel": (dec_ms, DEC_BYTES, 1),
              "calib_hist_kernel": (cal_ms, CAL_BATCHES * CAL_BYTES, 1)}
    dom = max(stages, key=lambda s: stages[s][0] * stages[s][2])
    d_ms, d_bytes, _ = stages[dom]
    achieved = gbs(d_bytes, d_ms)
    traffic, traffic_src = traffic_from_summary(dom)
    roofline = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "traffic_source": traffic_src,
                "algorithmic_bytes_per_launch": d_bytes, "avg_launch_ms": d_ms}
    if dom == "calib_hist_kernel":
        roofline["note"] = "calibration: histogram, window and accumulate kernels, events around all of them"

    def timed(fn, reps=5):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def hbm_row(ms, nbytes, note, key="gbs", **extra):
        r = {"ms": ms, key: gbs(nbytes, ms), "frac_hbm": gbs(nbytes, ms) / HBM_PEAK_GBS, "note": note}
        r.update(extra)
        return r

    def per_head_scale(x4):
        nh = int(x4.shape[1])
        mn = torch.empty(nh, dtype=torch.float32, device=dev)
        mx = torch.empty(nh, dtype=torch.float32, device=dev)
        rmin = torch.empty(nh, dtype=torch.float32, device=dev)
        rmax = torch.empty(nh, dtype=torch.float32, device=dev)
        fa.fa3q_init_minmax(rmin, rmax, stream=stream)
        fa.fa3q_calibrate_perhead(x4, RATIO, mn, mx, stream=stream)
        fa.fa3q_accumulate_minmax(rmin, rmax, mn, mx, stream=stream)
        return fa.fa3q_qparams(rmin, rmax, stream=stream)

    # ------------------------------------------------------------------ measurements outside the step
    if "decode_append" in only:
        # one new token per (b,h) written into the cache at position T-1, then attention over all
        # T tokens: the cache reads of decode plus one row written per (b,h)
        k_new = synth.normal_tensor((QB, H, DN + DR), dtype=torch.bfloat16, seed=410, device=dev)
        v_new = synth.normal_tensor((QB, H, DV), dtype=torch.bfloat16, seed=420, device=dev)
        kv_len = torch.full((QB,), QS - 1, dtype=torch.int32, device=dev)
        app_ms = timed(lambda: fa.fa3q_decode_append_attn(q, k_new, v_new, scale, kq, kr, v, kv_len, sm, out, ws_dec,
                                                          stream=stream))
        breakdown["decode_append"] = hbm_row(app_ms, DEC_BYTES, "append one token per (b,h) at position T-1, then "
                                             "attention over T (outside the step)", key="kv_gbs")
        del k_new, v_new, kv_len

    if "decode_qkv8" in only:
        # Q (non-RoPE part), K-nope and V all INT8: V and Q get per-head scales from the library's
        # own calibration (V: sequence 0 of the cache; Q: its non-RoPE part); 384 B per cached token
        scale_v = per_head_scale(v[:1].contiguous())
        scale_q = per_head_scale(q[:, :, :DN].contiguous().view(QB, H, 1, DN))
        vq, _ = fa.fa3q_quantize_k(v, scale_v, DV, stream=stream)
        qc, qrope = fa.fa3q_quantize_k(q.view(QB, H, 1, DN + DR), scale_q, DN, stream=stream)
        qc, qrope = qc.view(QB, H, DN), qrope.view(QB, H, DR)
        q8_ms = timed(lambda: fa.fa3q_decode_attn_qkv8(qc, qrope, scale_q, kq, scale, kr, vq, scale_v, sm, out,
                                                       ws_dec, stream=stream))
        q8_bytes = QB * H * (QS * (DN + 2 * DR + DV) + DN + 2 * DR + 4 * DV)
        breakdown["decode_qkv8"] = hbm_row(q8_ms, q8_bytes, "Q (non-RoPE), K-nope and V INT8 with per-head scales; "
                                           "384 B per cached token (outside the step)", key="kv_gbs", bytes=q8_bytes)
        del vq

    if "asym" in only:
        # asymmetric K cache with a scale and an offset per (head, dim) (float16 tables derived with
        # torch from per-channel min/max of sequence 0), quantised then decoded
        kn0 = k[0, :, :, :DN].float()
        lo, hi = kn0.amin(dim=1), kn0.amax(dim=1)
        a_scale = ((hi - lo) / 255.0).clamp_min(1e-6)
        a_offset = -128.0 - lo / a_scale
        a_scale, a_offset = a_scale.to(torch.float16).contiguous(), a_offset.to(torch.float16).contiguous()
        del kn0, lo, hi
        akq = torch.empty_like(kq)
        akr = torch.empty_like(kr)
        aq_ms = timed(lambda: fa.fa3q_quantize_asym(k, a_scale, a_offset, DN, akq, akr, stream=stream))
        ad_ms = timed(lambda: fa.fa3q_decode_attn_asym(q, akq, a_scale, a_offset, akr, v, sm, out, ws_dec,
                                                       stream=stream))
        breakdown["quantize_asym"] = hbm_row(aq_ms, QUANT_BYTES, "scale and offset per (head, dim), float16 tables "
                                             "(outside the step)")
        breakdown["decode_asym"] = hbm_row(ad_ms, DEC_BYTES, "attention over the asymmetric K-nope cache (outside "
                                           "the step)", key="kv_gbs")
        del akq, akr

    if "fake_quant" in only:
        # out of place (768 B per (token, head)), then in place on the result (512 B: the RoPE part is
        # neither read nor written; the operation is idempotent, so every call does the same work)
        fq_y = torch.empty_like(k)
        fq_ms = timed(lambda: fa.fa3q_fake_quant(k, scale, DN, fq_y, stream=stream))
        fqi_ms = timed(lambda: fa.fa3q_fake_quant(fq_y, scale, DN, fq_y, stream=stream))
        breakdown["fake_quant"] = hbm_row(fq_ms, QB * H * QS * 4 * (DN + DR), "K (64,128,4096,128+64) bf16 -> bf16, "
                                          "out of place (outside the step)")
        breakdown["fake_quant_in_place"] = hbm_row(fqi_ms, QB * H * QS * 4 * DN, "the same in place: only the "
                                                   "non-RoPE part is touched")
        del fq_y

    if "decode_latent" in only:
        # shared-latent (absorbed MLA) cache: per token one latent row of 512 features (+ 64 RoPE)
        # shared by all 128 heads, built by the library's own path with one head; both products on
        # MFMA: 2 * H * (Dl + Dr + Dl) flop per (b, t)
        LAT_DL = 512
        lat_rows = synth.activations((QB, 1, QS, LAT_DL + DR), sigma[:1], law="normal", outlier_frac=0.0005,
                                     outlier_mult=40.0, dtype=torch.bfloat16, seed=500, device=dev)
        lat_scale = per_head_scale(lat_rows[:, :, :, :LAT_DL].contiguous())
        lat_c, lat_r = fa.fa3q_quantize_k(lat_rows, lat_scale, LAT_DL, stream=stream)
        del lat_rows
        lat_q = synth.normal_tensor((QB, H, LAT_DL + DR), dtype=torch.bfloat16, seed=510, device=dev)
        lat_out = torch.empty((QB, H, LAT_DL), dtype=torch.float32, device=dev)
        lat_ws = torch.empty(max(1, fa.fa3q_decode_latent_workspace_bytes(QB, H, QS, LAT_DL)), dtype=torch.uint8,
                             device=dev)
        lt_ms = timed(lambda: fa.fa3q_decode_latent(lat_q, lat_c, lat_scale, lat_r, sm, lat_out, lat_ws,
                                                    stream=stream))
        lat_flop = QB * H * QS * 2 * (2 * LAT_DL + DR)
        lat_bytes = QB * QS * (LAT_DL + 2 * DR) + QB * H * (2 * (LAT_DL + DR) + 4 * LAT_DL)
        breakdown["decode_latent"] = {
            "ms": lt_ms, "tflops": lat_flop / (lt_ms * 1e-3) / 1e12,
            "frac_mfma_bf16": lat_flop / (lt_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "cache_gbs": gbs(lat_bytes, lt_ms),
            "note": "shared-latent MLA cache, B=64 H=128 T=4096 Dl=512 Dr=64, MFMA bf16 (outside the step)"}
        del lat_c, lat_r, lat_q, lat_out, lat_ws

    long_bytes = 2 * math.prod(LONG_SHAPE)
    n_long = LONG_SHAPE[0] * LONG_SHAPE[2] * LONG_SHAPE[3]
    if "calibrate_long" in only or "calibrate_largek" in only:
        # one (2,128,16384,128) bf16 tensor (Student-t(3) tails, 1e-4 outliers at +-60 sigma)
        long_x = synth.activations(LONG_SHAPE, synth.head_sigmas(H, seed=77), law="t3", outlier_frac=1e-4,
                                   outlier_mult=60.0, dtype=torch.bfloat16, seed=501, device=dev)
        long_min = torch.empty(H, dtype=torch.float32, device=dev)
        long_max = torch.empty(H, dtype=torch.float32, device=dev)

        def calib_row(x, r, key, note):
            B_, H_, S_, D_ = x.shape
            ws = torch.empty(max(1, fa.fa3q_calibrate_workspace_bytes(torch.bfloat16, B_, H_, S_, D_, r)),
                             dtype=torch.uint8, device=dev)
            n = B_ * S_ * D_
            c_ms = timed(lambda: fa.fa3q_calibrate_perhead(x, r, long_min, long_max, ws, stream=stream))
            k_win = n - int(r * n) + 1
            hist = k_win > fa.fa3q_calibrate_max_windows(torch.bfloat16) or n >= 1 << 20  # the header's routing
            breakdown[key] = hbm_row(c_ms, 2 * x.numel(), note, K=k_win, path="histogram" if hist else "tail lists")
            del ws

        if "calibrate_long" in only:
            for r in LONG_RATIOS:
                calib_row(long_x, r, f"calibrate_long_{r}", f"one (2,128,16384,128) bf16 tensor at ratio {r} "
                          "(outside the step)")
        if "calibrate_largek" in only:
            calib_row(long_x, 0.99, "calibrate_largek_long_0.99", "one (2,128,16384,128) bf16 tensor at ratio 0.99 "
                      "(K past the on-chip tail lists: histogram path; outside the step)")
            for r in (0.99, 0.9):
                calib_row(calib[0], r, f"calibrate_largek_{r}", f"one (8,128,2048,128) bf16 batch at ratio {r} "
                          "(histogram path; outside the step)")
        del long_x

    if "calibrate_f32" in only:
        # one float32 calibration batch (8,128,2048,128): the tail lists at ratio 0.9999 (rows of
        # 128 values, a power of two, take them in (B,S,H,D) too), the collect-and-sort path past
        # them (0.99, 0.9)
        x32 = synth.activations(CAL_SHAPE, synth.head_sigmas(H, seed=2024), law="t3", dtype=torch.float32, seed=100,
                                device=dev)
        w32_min = torch.empty((1, H), dtype=torch.float32, device=dev)
        w32_max = torch.empty((1, H), dtype=torch.float32, device=dev)
        n32 = CAL_SHAPE[0] * CAL_SHAPE[2] * CAL_SHAPE[3]
        for layout, xl, ratios in (("BHSD", x32, (0.9999, 0.99, 0.9)), ("BSHD", None, (0.9999, 0.99))):
            if layout == "BSHD":
                xl = x32.transpose(1, 2).contiguous()
            for r in ratios:
                ws = torch.empty(max(1, fa.fa3q_calibrate_ex_workspace_bytes(torch.float32, layout, 1, *CAL_SHAPE, r)),
                                 dtype=torch.uint8, device=dev)
                c_ms = timed(lambda: fa.fa3q_calibrate_ex([xl], r, layout=layout, win_min=w32_min, win_max=w32_max,
                                                          workspace=ws, stream=stream))
                k_win = n32 - int(r * n32) + 1
                sort = k_win > fa.fa3q_calibrate_max_windows(torch.float32)  # D = 128: rows take the tail lists
                tag = "" if layout == "BHSD" else "_bshd"
                breakdown[f"calibrate_f32{tag}_{r}"] = hbm_row(
                    c_ms, 4 * x32.numel(), f"one (8,128,2048,128) float32 batch, {layout}, at ratio {r} "
                    "(bytes: the batch read once; outside the step)", K=k_win,
                    path="collect and sort" if sort else "tail lists")
                del ws
            del xl
        del x32

    LB, LT = 8, QB * QS // 8
    long_dec_bytes = LB * H * LT * (DN + 2 * DR + 2 * DV) + LB * H * (2 * (DN + DR) + 4 * DV)
    kq_l, kr_l, v_l = kq.view(LB, H, LT, DN), kr.view(LB, H, LT, DR), v.view(LB, H, LT, DV)
    q_l, out_l = q[:LB], out[:LB]
    if "decode_long" in only:
        # decode with B=8, T=32768 over the step's cache bytes read as 8 sequences of 32768 tokens
        ld_ws = torch.empty(max(1, fa.fa3q_decode_attn_workspace_bytes(LB, H, LT, DV)), dtype=torch.uint8,
                            device=dev)
        ld_ms = timed(lambda: fa.fa3q_decode_attn(q_l, kq_l, scale, kr_l, v_l, sm, out_l, ld_ws, stream=stream))
        breakdown["decode_long"] = hbm_row(ld_ms, long_dec_bytes, "B=8 H=128 T=32768 Dv=128, split over the tokens "
                                           "(outside the step)", key="kv_gbs")
        del ld_ws
    if "decode_noalloc" in only:
        # the same long-context decode through the entry point that keeps its split states in the
        # library's static scratch array
        nd_ms = timed(lambda: fa.fa3q_decode_attn_noalloc(q_l, kq_l, scale, kr_l, v_l, sm, out_l, stream=stream))
        breakdown["decode_noalloc"] = hbm_row(nd_ms, long_dec_bytes, "B=8 H=128 T=32768 through "
                                              "fa3q_decode_attn_noalloc (outside the step)", key="kv_gbs")

    if "decode_paged" in only:
        # the step's cache bytes read as pools of 64-token pages, each sequence's 64 pages scattered by
        # a seeded permutation; attention over all 4096 tokens of every sequence through the table
        PG = 64
        n_pages = QB * QS // PG
        gen = torch.Generator(device="cpu")
        gen.manual_seed(700)
        table = torch.randperm(n_pages, generator=gen).to(torch.int32).view(QB, QS // PG).to(dev)
        full_len = torch.full((QB,), QS, dtype=torch.int32, device=dev)
        kq_p, kr_p, v_p = kq.view(n_pages, H, PG, DN), kr.view(n_pages, H, PG, DR), v.view(n_pages, H, PG, DV)
        pg_ms = timed(lambda: fa.fa3q_decode_paged_attn(q, None, None, scale, kq_p, kr_p, v_p, table, full_len, sm,
                                                        out, ws_dec, stream=stream))
        breakdown["decode_paged"] = hbm_row(pg_ms, DEC_BYTES + table.numel() * 4, "B=64 H=128 T=4096 in 64-token "
                                            "pages through a permuted block table (outside the step)", key="kv_gbs")
        del table

    if "f16_bshd" in only:
        # the step's three streaming stages on float16 tensors in the (B,S,H,D) layout, drawn in float16
        # with the step's recipes and laid out once, outside the timing
        def f16_bshd(t):
            return t.transpose(1, 2).contiguous()

        calib_t = [f16_bshd(synth.activations(CAL_SHAPE, sigma, law="t3", dtype=torch.float16, seed=100 + i,
                                              device=dev)) for i in range(CAL_BATCHES)]
        ws_t = torch.empty(max(1, fa.fa3q_calibrate_ex_workspace_bytes(torch.float16, "BSHD", CAL_BATCHES,
                                                                       *CAL_SHAPE, RATIO)),
                           dtype=torch.uint8, device=dev)
        rmin_t = torch.empty(H, dtype=torch.float32, device=dev)
        rmax_t = torch.empty(H, dtype=torch.float32, device=dev)
        ct_ms = timed(lambda: fa.fa3q_calibrate_ex(calib_t, RATIO, "BSHD", rmin_t, rmax_t, True, workspace=ws_t,
                                                   stream=stream))
        breakdown["calibrate_f16_bshd"] = hbm_row(ct_ms, CAL_BATCHES * CAL_BYTES, "4 batches (8,2048,128,128) "
                                                  "float16 (B,S,H,D) through fa3q_calibrate_ex (histogram path; "
                                                  "outside the step)")
        del calib_t, ws_t
        k_t = f16_bshd(synth.activations((QB, H, QS, DN + DR), sigma, law="normal", outlier_frac=0.0005,
                                         outlier_mult=40.0, dtype=torch.float16, seed=200, device=dev))
        kq_t = torch.empty((QB, QS, H, DN), dtype=torch.int8, device=dev)
        kr_t = torch.empty((QB, QS, H, DR), dtype=torch.float16, device=dev)
        qt_ms = timed(lambda: fa.fa3q_quantize_k_ex(k_t, scale, DN, "BSHD", kq_t, kr_t, stream=stream))
        breakdown["quantize_f16_bshd"] = hbm_row(qt_ms, QUANT_BYTES, "K (64,4096,128,128+64) float16 (B,S,H,D) "
                                                 "through fa3q_quantize_k_ex (outside the step)")
        del k_t
        v_t = f16_bshd(synth.activations((QB, H, QS, DV), sigma, law="normal", dtype=torch.float16, seed=300,
                                         device=dev))
        q_t = synth.normal_tensor((QB, H, DN + DR), dtype=torch.float16, seed=400, device=dev)
        dt_ms = timed(lambda: fa.fa3q_decode_attn_ex(q_t, kq_t, scale, kr_t, v_t, sm, "BSHD", out, ws_dec,
                                                     stream=stream))
        breakdown["decode_f16_bshd"] = hbm_row(dt_ms, DEC_BYTES, "B=64 H=128 T=4096 cache in (B,T,H,.) with float16 "
                                               "q, K-rope and V through fa3q_decode_attn_ex (outside the step)",
                                               key="kv_gbs")
        del kq_t, kr_t, v_t, q_t

    # device-to-device copy of COPY_BYTES: a reference ceiling for read+write streaming, and the
    # known-size kernel the HBM byte counters are scaled by
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1.0)
    copy_ms = timed(lambda: dst.copy_(src))
    copy_ref = {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES, "ms": copy_ms,
                "gbs_read_plus_write": 2 * COPY_BYTES / (copy_ms * 1e-3) / 1e9}
    del src, dst

    cpu = None
    if pool is not None:
        log(f"timing the CPU oracle on a bounded sample with {workers} worker processes ...")
        cpu = cpu_baseline(pool, workers, {"calib": calib, "k": k, "scale": scale, "kq": kq, "kr": kr, "v": v,
                                           "q": q}, args.cpu_budget)

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("fa3q hot path: calibrate 4 x bf16 (8,128,2048,128) ratio 0.9999 -> accumulate -> qparams "
                         "-> quantize K (64,128,4096,128+64) -> decode attention B=64 H=128 T=4096 Dv=128"),
            "storage": "bf16 activations/K-rope/V, int8 K-nope cache, float32 stats and scales",
            "arithmetic": "integer keys and float32 (window lengths, scales, quotients, attention)",
            "algorithmic_bytes_per_step": total_bytes,
        },
        "breakdown": breakdown,
        "roofline": roofline,
        "copy_reference": copy_ref,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
