"""Benchmark of the MI355X linear-attention library (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one la_forward call over the bf16 prefill workload B=4, H=8,
T=8192, d=64 (chunk 64, fp32 state): the whole hot path of that workload.
The line printed is one JSON object:

* value / unit: prefill tokens per second (B*T per step) of the timed steps;
* roofline: HBM roofline of the la_forward call -- algorithmic bytes (inputs
  read once, outputs and final state written once) over the mean duration
  measured with HIP events on the launch stream;
* cpu_baseline: the fp64 oracle (C, OpenMP over heads) timed on the host on
  the same workload;
* extra: the other measured paths -- the long-stream LA workload, the LA
  backward pass on the bench workload, a packed serving batch of mixed
  request lengths, the delta, gated delta and
  scalar-decay (SSD) prefills and the 1000-step decode chains of the four
  rules (state-update GB/s) -- each with its own roofline fraction.

Inputs are synthetic (seeded, generated on the device) and rotate among
several copies so that each step reads data evicted from the 256 MB
Infinity Cache.  --gpus above 1 is refused: the benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_MFMA_PEAK_TFS = 2516.6  # MI355X dense bf16 MFMA, published (2.5 PFLOP/s)
METRIC = "prefill tokens/sec (MFMA % peak); decode state-update GB/s (% HBM peak)"

# HBM traffic of one la_fused_kernel launch on the bf16 prefill workload:
# rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch, mean of the
# dispatches of `bench.py --only la --steps 5 --warmup 2 --no-cpu`), each
# scaled by what the same counter reads for a 1 GiB device copy
# (`bench.py --calibrate-copy`: FETCH_SIZE 524302 KiB -> x2.0, WRITE_SIZE
# 1048576 KiB -> x1.0).  Valid only for the kernel sources it was measured
# on (their SHA-256 below); the roofline reports null traffic otherwise.
LA_TRAFFIC = {
    "sources": ["weight_recurrent_memory_amd/csrc/la_prefill.hip",
                "weight_recurrent_memory_amd/csrc/common.hpp",
                "weight_recurrent_memory_amd/csrc/kernels.hpp",
                "weight_recurrent_memory_amd/csrc/segments.hpp"],
    "sha256": "8a1c05f785bc34ee923c50a50735c4808e955abc50d893e23f3736166ef11e64",
    "fetch_kib": 70050.5, "fetch_scale": 2.0,
    "write_kib": 48397.1, "write_scale": 1.0,
}


def la_traffic_bytes():
    import hashlib
    h = hashlib.sha256()
    for f in LA_TRAFFIC["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != LA_TRAFFIC["sha256"]:
        return None
    return 1024 * (LA_TRAFFIC["fetch_kib"] * LA_TRAFFIC["fetch_scale"]
                   + LA_TRAFFIC["write_kib"] * LA_TRAFFIC["write_scale"])


def la_bytes(B, H, T, dk, dv, el):
    return B * H * T * (2 * dk + dv) * el + B * H * T * dv * el + B * H * (dk * dv + dk) * 4


def la_flops(B, H, T, dk, dv, C=64):
    # per token-head at chunk C: (C+1)(dk+dv) + 4 dk dv (causal half of the
    # intra-chunk products, the inter-chunk read and the state update)
    return B * H * T * ((C + 1) * (dk + dv) + 4 * dk * dv)


def delta_bytes(B, H, T, dk, dv, el, gated=False):
    # q, k, v, beta read, o written, final state written; gated: alpha (fp32) read
    return (B * H * T * (2 * dk + dv) * el + B * H * T * el + B * H * T * dv * el + B * H * dk * dv * 4
            + (B * H * T * 4 if gated else 0))


def delta_flops(B, H, T, dk, dv, C=64):
    return B * H * T * ((C - 1) * dk + C * C // 3 + (C + 1) * (dk + 2 * dv) + 6 * dk * dv)


def ssd_bytes(B, H, T, dk, dv, el):
    # q, k, v and alpha (fp32) read once, o written once, the final state written
    return B * H * T * (2 * dk + dv) * el + B * H * T * 4 + B * H * T * dv * el + B * H * dk * dv * 4


def ssd_flops(B, H, T, dk, dv, C=64):
    # per token-head: causal half of Q K^T and of P V, the state read and the update
    return B * H * T * ((C + 1) * (dk + dv) + 4 * dk * dv)


def decode_bytes(N, H, dk, dv, el):
    return N * H * (2 * dk * dv * 4 + 2 * dk * 4 + (2 * dk + dv) * el + dv * el)


def delta_decode_bytes(N, H, dk, dv, el, gated=False):
    # S read and written (fp32); q, k, v, beta read; o written; gated: alpha (fp32) read
    return N * H * (2 * dk * dv * 4 + (2 * dk + dv + 1) * el + dv * el + (4 if gated else 0))


def ssd_decode_bytes(N, H, dk, dv, el):
    # S read and written (fp32); q, k, v, alpha (fp32) read; o written
    return N * H * (2 * dk * dv * 4 + (2 * dk + dv) * el + 4 + dv * el)


def _events(n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def time_calls(fn, n_calls, warmup, stream):
    """Run fn(i) warmup + n_calls times; returns (wall seconds of the timed
    calls, mean device time per call in ms).  The device time comes from two
    HIP events on the launch stream around the whole timed region, so it is
    the average launch duration including the gaps between launches, and the
    host's own per-call overhead overlaps the device work."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, end = _events(2)
    # A garbage-collection pause while the calls are being queued would leave
    # the device idle inside the timed region.
    gc_was_on = gc.isenabled()
    gc.collect()
    gc.disable()
    try:
        t0 = time.perf_counter()
        start.record(stream)
        for i in range(n_calls):
            fn(i)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    finally:
        if gc_was_on:
            gc.enable()
    return wall, start.elapsed_time(end) / n_calls


def bench_la(w, steps, warmup, copies, lin, wl):
    dev = torch.device("cuda:0")
    el = 2 if w.dtype == torch.bfloat16 else 4
    sets = [wl.la_inputs(w.B, w.H, w.T, w.dk, w.dv, w.dtype, w.seed + 17 * i, dev) for i in range(copies)]
    outs = [torch.empty((w.B, w.H, w.T, w.dv), dtype=w.dtype, device=dev) for _ in range(copies)]
    S = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    z = torch.empty((w.B, w.H, w.dk), dtype=torch.float32, device=dev)
    ws = torch.empty(lin.la_forward_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv), dtype=torch.uint8, device=dev)

    def step(i):
        q, k, v = sets[i % copies]
        lin.la_forward(q, k, v, eps=1e-6, o=outs[i % copies], S_out=S, z_out=z, workspace=ws)

    stream = torch.cuda.current_stream(dev)
    wall, mean_ms = time_calls(step, steps, warmup, stream)
    nbytes = la_bytes(w.B, w.H, w.T, w.dk, w.dv, el)
    return {
        "wall_s": wall, "ms_per_step": 1e3 * wall / steps, "event_ms_mean": mean_ms,
        "tokens_per_s": w.B * w.T * steps / wall,
        "bytes": nbytes, "flops": la_flops(w.B, w.H, w.T, w.dk, w.dv),
        "gbs": nbytes / (mean_ms * 1e-3) / 1e9,
        "tflops": la_flops(w.B, w.H, w.T, w.dk, w.dv) / (mean_ms * 1e-3) / 1e12,
    }


def bench_delta(w, steps, warmup, copies, lin, wl):
    """delta_forward, or gated_delta_forward for a gated workload."""
    dev = torch.device("cuda:0")
    el = 2
    gated = w.kind == "gated_delta"
    sets = [wl.delta_inputs(w.B, w.H, w.T, w.dk, w.dv, w.dtype, w.seed + 17 * i, dev)
            + ((wl.gates((w.B, w.H, w.T), w.seed + 17 * i, dev),) if gated else ()) for i in range(copies)]
    outs = [torch.empty((w.B, w.H, w.T, w.dv), dtype=w.dtype, device=dev) for _ in range(copies)]
    S = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(lin.delta_forward_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv), dtype=torch.uint8, device=dev)

    def step(i):
        if gated:
            q, k, v, beta, alpha = sets[i % copies]
            lin.gated_delta_forward(q, k, v, beta, alpha, o=outs[i % copies], S_out=S, workspace=ws)
        else:
            q, k, v, beta = sets[i % copies]
            lin.delta_forward(q, k, v, beta, o=outs[i % copies], S_out=S, workspace=ws)

    wall, mean_ms = time_calls(step, steps, warmup, torch.cuda.current_stream(dev))
    nbytes = delta_bytes(w.B, w.H, w.T, w.dk, w.dv, el, gated)
    fl = delta_flops(w.B, w.H, w.T, w.dk, w.dv)
    return {"ms_per_step": 1e3 * wall / steps, "event_ms_mean": mean_ms, "tokens_per_s": w.B * w.T * steps / wall,
            "bytes": nbytes, "flops": fl, "gbs": nbytes / (mean_ms * 1e-3) / 1e9,
            "tflops": fl / (mean_ms * 1e-3) / 1e12}


def bench_ssd(w, steps, warmup, copies, lin, wl):
    dev = torch.device("cuda:0")
    el = 2
    sets = [wl.la_inputs(w.B, w.H, w.T, w.dk, w.dv, w.dtype, w.seed + 17 * i, dev)
            + (wl.gates((w.B, w.H, w.T), w.seed + 17 * i, dev),) for i in range(copies)]
    outs = [torch.empty((w.B, w.H, w.T, w.dv), dtype=w.dtype, device=dev) for _ in range(copies)]
    S = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(lin.ssd_forward_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv), dtype=torch.uint8, device=dev)

    def step(i):
        q, k, v, alpha = sets[i % copies]
        lin.ssd_forward(q, k, v, alpha, o=outs[i % copies], S_out=S, workspace=ws)

    wall, mean_ms = time_calls(step, steps, warmup, torch.cuda.current_stream(dev))
    nbytes = ssd_bytes(w.B, w.H, w.T, w.dk, w.dv, el)
    fl = ssd_flops(w.B, w.H, w.T, w.dk, w.dv)
    return {"ms_per_step": 1e3 * wall / steps, "event_ms_mean": mean_ms, "tokens_per_s": w.B * w.T * steps / wall,
            "bytes": nbytes, "flops": fl, "gbs": nbytes / (mean_ms * 1e-3) / 1e9,
            "tflops": fl / (mean_ms * 1e-3) / 1e12}


def bench_ssd_decode(w, lin, wl, n_steps=None):
    dev = torch.device("cuda:0")
    S, Q, K, V, At = wl.make(w, dev)
    n = w.T if n_steps is None else n_steps
    o = torch.empty((w.B, w.H, w.dv), dtype=w.dtype, device=dev)

    def step(i):
        j = i % w.T
        lin.ssd_decode_step(Q[j], K[j], V[j], At[j], S, o=o)

    wall, mean_ms = time_calls(step, n, 10, torch.cuda.current_stream(dev))
    per = ssd_decode_bytes(w.B, w.H, w.dk, w.dv, 2)
    return {"steps": n, "ms_per_step": 1e3 * wall / n, "event_ms_mean": mean_ms, "bytes_per_step": per,
            "gbs_wall": per * n / wall / 1e9, "gbs": per / (mean_ms * 1e-3) / 1e9}


def la_backward_bytes(B, H, T, dk, dv, el):
    # q, k, v, dO read once; dq, dk, dv written once
    return B * H * T * (2 * dk + 2 * dv) * el + B * H * T * (2 * dk + dv) * el


def bench_la_backward(w, steps, warmup, copies, lin, wl):
    """la_backward on the LA prefill workload (gradients of a random dO)."""
    dev = torch.device("cuda:0")
    sets = [wl.la_inputs(w.B, w.H, w.T, w.dk, w.dv, w.dtype, w.seed + 17 * i, dev)
            + (wl.la_inputs(w.B, w.H, w.T, w.dv, w.dv, w.dtype, w.seed + 17 * i + 1, dev)[0],) for i in range(copies)]
    grads = [tuple(torch.empty_like(x) for x in st[:3]) for st in sets]
    ws = torch.empty(lin.la_backward_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv), dtype=torch.uint8, device=dev)

    def step(i):
        q, k, v, dO = sets[i % copies]
        dq, dk, dv = grads[i % copies]
        lin.la_backward(q, k, v, dO, eps=1e-6, dq=dq, dk=dk, dv=dv, return_state_grads=False, workspace=ws)

    wall, mean_ms = time_calls(step, steps, warmup, torch.cuda.current_stream(dev))
    nbytes = la_backward_bytes(w.B, w.H, w.T, w.dk, w.dv, 2)
    return {"ms_per_step": 1e3 * wall / steps, "event_ms_mean": mean_ms, "tokens_per_s": w.B * w.T * steps / wall,
            "bytes": nbytes, "gbs": nbytes / (mean_ms * 1e-3) / 1e9}


def delta_backward_bytes(B, H, T, dk, dv, el, gated):
    # q, k, v, dO, beta read once, dq, dk, dv written once, dbeta (fp32)
    # written; gated: alpha read and dalpha written (fp32)
    return (B * H * T * (2 * dk + 2 * dv + 1) * el + B * H * T * (2 * dk + dv) * el + B * H * T * 4
            + (2 * B * H * T * 4 if gated else 0))


def bench_delta_backward(w, steps, warmup, copies, lin, wl):
    """delta_backward (gated for a gated workload): gradients of a random dO."""
    dev = torch.device("cuda:0")
    gated = w.kind == "gated_delta"
    sets = []
    for i in range(copies):
        q, k, v, beta = wl.delta_inputs(w.B, w.H, w.T, w.dk, w.dv, w.dtype, w.seed + 17 * i, dev)
        dO = wl.la_inputs(w.B, w.H, w.T, w.dv, w.dv, w.dtype, w.seed + 17 * i + 1, dev)[0]
        alpha = wl.gates((w.B, w.H, w.T), w.seed + 17 * i, dev) if gated else None
        sets.append((q, k, v, beta, dO, alpha))
    grads = [tuple(torch.empty_like(x) for x in st[:3]) for st in sets]
    ws = torch.empty(lin.delta_backward_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv), dtype=torch.uint8, device=dev)

    def step(i):
        q, k, v, beta, dO, alpha = sets[i % copies]
        dq, dk, dv = grads[i % copies]
        lin.delta_backward(q, k, v, beta, dO, alpha, dq=dq, dk=dk, dv=dv, return_state_grad=False, workspace=ws)

    wall, mean_ms = time_calls(step, steps, warmup, torch.cuda.current_stream(dev))
    nbytes = delta_backward_bytes(w.B, w.H, w.T, w.dk, w.dv, 2, gated)
    return {"ms_per_step": 1e3 * wall / steps, "event_ms_mean": mean_ms, "tokens_per_s": w.B * w.T * steps / wall,
            "bytes": nbytes, "gbs": nbytes / (mean_ms * 1e-3) / 1e9}


def bench_la_packed(w, steps, warmup, lin, wl):
    """la_forward_packed on a serving batch of mixed request lengths."""
    dev = torch.device("cuda:0")
    q, k, v, cu = wl.make(w, dev)
    cu_dev = cu.to(dev)
    o = torch.empty((w.H, w.T, w.dv), dtype=w.dtype, device=dev)
    S = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    z = torch.empty((w.B, w.H, w.dk), dtype=torch.float32, device=dev)
    ws = torch.empty(lin.la_forward_packed_workspace_bytes(cu, w.H, w.dk, w.dv), dtype=torch.uint8, device=dev)

    def step(i):
        lin.la_forward_packed(q, k, v, cu_dev, eps=1e-6, cu_seqlens_host=cu, o=o, S_out=S, z_out=z, workspace=ws)

    wall, mean_ms = time_calls(step, steps, warmup, torch.cuda.current_stream(dev))
    nbytes = la_bytes(1, w.H, w.T, w.dk, w.dv, 2) + (w.B - 1) * w.H * (w.dk * w.dv + w.dk) * 4
    lengths = (cu[1:] - cu[:-1]).tolist()
    return {"ms_per_step": 1e3 * wall / steps, "event_ms_mean": mean_ms, "tokens_per_s": w.T * steps / wall,
            "gbs": nbytes / (mean_ms * 1e-3) / 1e9, "requests": w.B, "min_len": min(lengths),
            "max_len": max(lengths)}


def bench_decode(w, lin, wl, n_steps=None):
    dev = torch.device("cuda:0")
    S, z, Q, K, V = wl.make(w, dev)
    n = w.T if n_steps is None else n_steps
    o = torch.empty((w.B, w.H, w.dv), dtype=w.dtype, device=dev)

    def step(i):
        lin.la_decode_step(Q[i % w.T], K[i % w.T], V[i % w.T], S, z, eps=1e-6, o=o)

    wall, mean_ms = time_calls(step, n, 10, torch.cuda.current_stream(dev))
    per = decode_bytes(w.B, w.H, w.dk, w.dv, 2)
    return {"steps": n, "ms_per_step": 1e3 * wall / n, "event_ms_mean": mean_ms, "bytes_per_step": per,
            "gbs_wall": per * n / wall / 1e9, "gbs": per / (mean_ms * 1e-3) / 1e9}


def bench_delta_decode(w, lin, wl, n_steps=None):
    """delta_decode_step, or gated_delta_decode_step for a gated workload."""
    dev = torch.device("cuda:0")
    gated = w.kind == "gated_delta_decode"
    if gated:
        S, Q, K, V, Bt, At = wl.make(w, dev)
    else:
        S, Q, K, V, Bt = wl.make(w, dev)
    n = w.T if n_steps is None else n_steps
    o = torch.empty((w.B, w.H, w.dv), dtype=w.dtype, device=dev)

    def step(i):
        j = i % w.T
        if gated:
            lin.gated_delta_decode_step(Q[j], K[j], V[j], Bt[j], At[j], S, o=o)
        else:
            lin.delta_decode_step(Q[j], K[j], V[j], Bt[j], S, o=o)

    wall, mean_ms = time_calls(step, n, 10, torch.cuda.current_stream(dev))
    per = delta_decode_bytes(w.B, w.H, w.dk, w.dv, 2, gated)
    return {"steps": n, "ms_per_step": 1e3 * wall / n, "event_ms_mean": mean_ms, "bytes_per_step": per,
            "gbs_wall": per * n / wall / 1e9, "gbs": per / (mean_ms * 1e-3) / 1e9}


def cpu_baseline(w, oracle, wl, heads=None):
    """The fp64 oracle on the host, same workload recipe (generated on the CPU)."""
    q, k, v = wl.la_inputs(w.B, w.H, w.T, w.dk, w.dv, w.dtype, w.seed, "cpu")
    BH = w.B * w.H
    heads = BH if heads is None else heads
    flat = lambda t: t.reshape(BH, *t.shape[2:])[:heads][None]
    qs, ks, vs = (oracle._f64(flat(t)) for t in (q, k, v))
    # Whole passes until about a second has run (at most 30 passes), so that
    # a fast pass is not timed once on its own.
    passes, total = 0, 0.0
    while passes < 30 and (passes == 0 or total < 1.0):
        t0 = time.perf_counter()
        oracle.la_forward(qs, ks, vs, eps=1e-6)
        total += time.perf_counter() - t0
        passes += 1
    dt = total / passes
    tokens = w.T * heads / w.H  # token rate scaled to the metric's B*T per step
    return {"value": tokens / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{heads} of {BH} heads x T={w.T} (all heads = the whole workload), {passes} passes; "
                      f"{total:.2f} s wall in total, {dt:.3f} s per pass", "seconds": dt}


def calibrate_copy(nbytes=1 << 30):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    dev = torch.device("cuda:0")
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": nbytes, "launches": 3}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=4, help="input copies rotated through (cache eviction)")
    ap.add_argument("--only", choices=["all", "la", "la_long", "la_packed", "la_backward", "delta", "gated_delta",
                                       "delta_backward", "ssd", "decode", "delta_decode", "gated_delta_decode",
                                       "ssd_decode"],
                    default="all")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} refused: the benchmark runs on one GPU "
              "(sharding is described, not run)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy()
        return

    from weight_recurrent_memory_amd import binding as lin
    from weight_recurrent_memory_amd import workloads as wl

    lin.lib()  # fail loudly if the HIP library is missing
    w = wl.LA_BF16_PREFILL
    main_res = None
    extra = {}
    if args.only in ("all", "la"):
        main_res = bench_la(w, args.steps, args.warmup, args.copies, lin, wl)
    if args.only in ("all", "la_long"):
        wl_ = wl.LA_BF16_LONG
        r = bench_la(wl_, max(3, args.steps // 10), 2, 2, lin, wl)
        extra[wl_.name] = {"tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"],
                           "hbm_gbs": r["gbs"], "hbm_frac": r["gbs"] / HBM_PEAK_GBS,
                           "mfma_tflops": r["tflops"], "mfma_frac": r["tflops"] / BF16_MFMA_PEAK_TFS}
    if args.only in ("all", "la_backward"):
        r = bench_la_backward(w, max(3, args.steps // 2), 3, args.copies, lin, wl)
        extra["la_backward_" + w.name] = {"tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"],
                                          "us_per_call": 1e3 * r["event_ms_mean"], "hbm_gbs": r["gbs"],
                                          "hbm_frac": r["gbs"] / HBM_PEAK_GBS, "bytes_per_call": r["bytes"]}
    if args.only in ("all", "la_packed"):
        wp = wl.PACKED_LA_BF16
        r = bench_la_packed(wp, max(3, args.steps // 2), 3, lin, wl)
        extra[wp.name] = {"tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"],
                          "hbm_gbs": r["gbs"], "hbm_frac": r["gbs"] / HBM_PEAK_GBS, "requests": r["requests"],
                          "request_len_min_max": [r["min_len"], r["max_len"]]}
    for key, wd in (("delta", wl.DELTA_BF16_PREFILL), ("gated_delta", wl.GATED_DELTA_BF16_PREFILL)):
        if args.only not in ("all", key):
            continue
        try:
            r = bench_delta(wd, max(5, args.steps // 2), 5, 2, lin, wl)
            extra[wd.name] = {"tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"],
                              "hbm_gbs": r["gbs"], "hbm_frac": r["gbs"] / HBM_PEAK_GBS,
                              "mfma_tflops": r["tflops"], "mfma_frac": r["tflops"] / BF16_MFMA_PEAK_TFS}
        except lin.LinAttnError as e:
            extra[wd.name] = {"error": str(e)}
    if args.only in ("all", "delta_backward"):
        for wd in (wl.DELTA_BF16_PREFILL, wl.GATED_DELTA_BF16_PREFILL):
            r = bench_delta_backward(wd, max(5, args.steps // 5), 3, 2, lin, wl)
            extra["delta_backward_" + wd.name] = {"tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"],
                                                  "us_per_call": 1e3 * r["event_ms_mean"], "hbm_gbs": r["gbs"],
                                                  "hbm_frac": r["gbs"] / HBM_PEAK_GBS, "bytes_per_call": r["bytes"]}
    if args.only in ("all", "ssd"):
        ws_ = wl.SSD_BF16_PREFILL
        r = bench_ssd(ws_, max(3, args.steps // 2), 3, args.copies, lin, wl)
        extra[ws_.name] = {"tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"],
                           "hbm_gbs": r["gbs"], "hbm_frac": r["gbs"] / HBM_PEAK_GBS,
                           "mfma_tflops": r["tflops"], "mfma_frac": r["tflops"] / BF16_MFMA_PEAK_TFS}
    if args.only in ("all", "decode"):
        wdec = wl.DECODE_BF16
        r = bench_decode(wdec, lin, wl)
        extra[wdec.name] = {"state_update_gbs": r["gbs"], "hbm_frac": r["gbs"] / HBM_PEAK_GBS,
                            "gbs_wall_incl_launch_gaps": r["gbs_wall"], "us_per_step": 1e3 * r["event_ms_mean"],
                            "steps": r["steps"], "bytes_per_step": r["bytes_per_step"]}

    for key, wdd in (("delta_decode", wl.DELTA_DECODE_BF16), ("gated_delta_decode", wl.GATED_DELTA_DECODE_BF16)):
        if args.only not in ("all", key):
            continue
        r = bench_delta_decode(wdd, lin, wl)
        extra[wdd.name] = {"state_update_gbs": r["gbs"], "hbm_frac": r["gbs"] / HBM_PEAK_GBS,
                           "gbs_wall_incl_launch_gaps": r["gbs_wall"], "us_per_step": 1e3 * r["event_ms_mean"],
                           "steps": r["steps"], "bytes_per_step": r["bytes_per_step"]}
    if args.only in ("all", "ssd_decode"):
        wsd = wl.SSD_DECODE_BF16
        r = bench_ssd_decode(wsd, lin, wl)
        extra[wsd.name] = {"state_update_gbs": r["gbs"], "hbm_frac": r["gbs"] / HBM_PEAK_GBS,
                           "gbs_wall_incl_launch_gaps": r["gbs_wall"], "us_per_step": 1e3 * r["event_ms_mean"],
                           "steps": r["steps"], "bytes_per_step": r["bytes_per_step"]}

    if main_res is None:
        print(json.dumps({"extra": extra}))
        return

    cpu = None
    if not args.no_cpu:
        import oracle  # test infrastructure, used only for this CPU baseline leg
        cpu = cpu_baseline(w, oracle, wl)

    gbs = main_res["gbs"]
    traffic = la_traffic_bytes()
    line = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q,k,v; generated on device; %d rotating copies)" % args.copies,
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv, "chunk": 64,
                   "state": "fp32"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_unit": "bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
                     "kernel": "la_fused_kernel<bf16, 64, 64> (the one launch of la_forward)",
                     "algorithmic_bytes_per_launch": main_res["bytes"],
                     "event_ms_mean": main_res["event_ms_mean"],
                     "mfma_tflops": main_res["tflops"], "mfma_frac": main_res["tflops"] / BF16_MFMA_PEAK_TFS},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
