"""Benchmark of the MI355X linear-attention library (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one la_forward call over the long-stream workload B=1, H=32,
T=65536, d=64 (bf16 inputs, fp32 state, chunk 64, outputs plus the final
S/z): the whole prefill hot path of the largest configuration.  The line
printed is one JSON object:

* value / unit: prefill tokens per second (B*T per step) over the wall time
  of the K timed steps;
* roofline: HBM roofline of la_fused_kernel (la_forward's one launch) --
  algorithmic bytes (inputs read once, outputs and final state written once)
  over the mean per-call duration from HIP event pairs on the launch stream;
  traffic from rocprofv3 FETCH_SIZE / WRITE_SIZE counters of the same
  kernel on the same workload, while the sources still match;
* cpu_baseline: the fp64 oracle (C, OpenMP over heads) timed on the host on
  every head of the same workload;
* decode: the other half of the metric -- the 1000-step decode chain (256
  sequences x 32 heads, d = 128, resident fp32 state) as state-update GB/s,
  with its own roofline and oracle baseline;
* extra: the other measured paths -- the bf16 prefill B=4 H=8 T=8192, the LA
  backward pass, a packed serving batch of mixed request lengths, the delta,
  gated delta and scalar-decay (SSD) prefills, the delta backward and the
  decode chains of the other three rules -- each with its own roofline
  fraction.

Timing: after the warm-up calls (by default enough to bring a cold device
to its steady clocks; the secondary workloads warm up for at least 60 ms,
and nothing idles the device between the warm-up and the timed calls), K
calls enqueued back to back between one
HIP event pair on the launch stream give the wall-clock throughput and the
average launch duration (what a kernel trace of the calls averages); K more
calls, each bracketed by its own event pair, give the median per call.
Inputs are synthetic (seeded, generated on the
device) and rotate among copies whose total exceeds the 256 MB Infinity
Cache, so each step reads from HBM.  --gpus above 1 is refused: the
benchmark runs on one GPU.
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
# Warm-up floor of the secondary workloads: a device that idled for a few
# milliseconds (input generation, the previous workload's bookkeeping) drops
# its clocks, and some 50 ms of sustained load bring them back.
WARM_S = 0.06

# Counter readings per (kernel, workload): rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch, mean over the dispatches of the command in
# the profile of the same name under profiles/), each scaled by what the same
# counter reads for a 1 GiB device copy (`bench.py --calibrate-copy`:
# FETCH_SIZE 524302 KiB -> x2.0, WRITE_SIZE 1048576 KiB -> x1.0), so that
# traffic is HBM-side bytes per launch.  A reading is valid only for the
# kernel sources it was taken on (their SHA-256 below); the roofline reports
# null traffic otherwise.
_CSRC = "weight_recurrent_memory_amd/csrc/"
LA_SOURCES = [_CSRC + f for f in ("la_prefill.hip", "common.hpp", "kernels.hpp", "segments.hpp")]
LA_DECODE_SOURCES = [_CSRC + f for f in ("la_decode.hip", "common.hpp", "kernels.hpp")]
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
COUNTERS = {
    # workload name -> kernel, sources, sha256 of the sources, KiB per dispatch
    "la_bf16_b1_h32_t65536_d64": {"kernel": "la_fused_kernel", "sources": LA_SOURCES,
                                  "sha256": "dea79e9da54a16e00c32689de5d002d36447d767b570acbf82e9d40877a9f156",
                                  "fetch_kib": 572178.1, "write_kib": 350713.0},
    "la_bf16_b4_h8_t8192_d64": {"kernel": "la_fused_kernel", "sources": LA_SOURCES,
                                "sha256": "dea79e9da54a16e00c32689de5d002d36447d767b570acbf82e9d40877a9f156",
                                "fetch_kib": 66439.5, "write_kib": 48397.0},
    "decode_bf16_n256_h32_d128_1000steps": {"kernel": "la_decode_kernel", "sources": LA_DECODE_SOURCES,
                                            "sha256": "3f6ff15dd06ccadb10a9e713196c85c9a832099ca4ea57f6b52e4ba8e306e996",
                                            "fetch_kib": 267306.9, "write_kib": 530466.8},
}


def sources_sha256(sources):
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_bytes(workload):
    """HBM bytes per launch from the stored counters, or None when none were
    taken on the current sources."""
    c = COUNTERS.get(workload)
    if not c or c["fetch_kib"] is None or c["sha256"] != sources_sha256(c["sources"]):
        return None
    return 1024 * (c["fetch_kib"] * FETCH_SCALE + c["write_kib"] * WRITE_SCALE)


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


def time_calls(fn, n_calls, warmup, stream, warm_s=0.0):
    """Run fn(i) warmup + 2 n_calls times (more warm-up calls, in groups of
    ten, while less than warm_s seconds of warm-up have run: the secondary
    workloads' calls are short, and a fixed count of them would not bring the
    device back to its steady clocks).  Returns (wall seconds of the first
    n_calls timed calls, mean device time per call in ms over that region,
    and the mean and median of per-call device times in ms).

    The first timed pass enqueues the calls back to back between one pair of
    HIP events on the launch stream: its wall time is the throughput figure
    and its event time divided by the calls is the average launch duration
    (the gaps between consecutive launches included, about a microsecond),
    which is what a kernel trace of the same calls averages.  The second
    pass brackets each call with its own event pair, for the median of at
    least 20 repetitions; each pair adds a few microseconds of its own, so
    those per-call figures run a little above the trace's."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_calls)]
    # A garbage-collection pause while the calls are being queued would leave
    # the device idle inside the timed region; it is taken before the warm-up,
    # so that only the synchronisation separates the warm-up from the timed
    # calls (an idle device drops its clocks within milliseconds).
    gc_was_on = gc.isenabled()
    gc.collect()
    gc.disable()
    try:
        t0 = time.perf_counter()
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        while time.perf_counter() - t0 < warm_s:
            for i in range(10):
                fn(i)
            torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for i in range(n_calls):
            fn(i)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for i in range(n_calls):
            ev[i][0].record(stream)
            fn(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
    finally:
        if gc_was_on:
            gc.enable()
    d = sorted(a.elapsed_time(b) for a, b in ev)
    med = d[len(d) // 2] if len(d) % 2 else 0.5 * (d[len(d) // 2 - 1] + d[len(d) // 2])
    return wall, start.elapsed_time(end) / n_calls, sum(d) / len(d), med


def bench_la(w, steps, warmup, copies, lin, wl, warm_s=0.0):
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
    wall, mean_ms, pc_mean, med_ms = time_calls(step, steps, warmup, stream, warm_s)
    nbytes = la_bytes(w.B, w.H, w.T, w.dk, w.dv, el)
    return {
        "wall_s": wall, "ms_per_step": 1e3 * wall / steps, "event_ms_mean": mean_ms, "event_ms_median": med_ms, "event_ms_mean_per_call": pc_mean,
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

    wall, mean_ms, pc_mean, med_ms = time_calls(step, steps, warmup, torch.cuda.current_stream(dev), WARM_S)
    nbytes = delta_bytes(w.B, w.H, w.T, w.dk, w.dv, el, gated)
    fl = delta_flops(w.B, w.H, w.T, w.dk, w.dv)
    return {"ms_per_step": 1e3 * wall / steps, "event_ms_mean": mean_ms, "event_ms_median": med_ms, "event_ms_mean_per_call": pc_mean, "tokens_per_s": w.B * w.T * steps / wall,
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

    wall, mean_ms, pc_mean, med_ms = time_calls(step, steps, warmup, torch.cuda.current_stream(dev), WARM_S)
    nbytes = ssd_bytes(w.B, w.H, w.T, w.dk, w.dv, el)
    fl = ssd_flops(w.B, w.H, w.T, w.dk, w.dv)
    return {"ms_per_step": 1e3 * wall / steps, "event_ms_mean": mean_ms, "event_ms_median": med_ms, "event_ms_mean_per_call": pc_mean, "tokens_per_s": w.B * w.T * steps / wall,
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

    wall, mean_ms, pc_mean, med_ms = time_calls(step, n, 10, torch.cuda.current_stream(dev), WARM_S)
    per = ssd_decode_bytes(w.B, w.H, w.dk, w.dv, 2)
    return {"steps": n, "ms_per_step": 1e3 * wall / n, "event_ms_mean": mean_ms, "event_ms_median": med_ms, "event_ms_mean_per_call": pc_mean, "bytes_per_step": per,
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

    wall, mean_ms, pc_mean, med_ms = time_calls(step, steps, warmup, torch.cuda.current_stream(dev), WARM_S)
    nbytes = la_backward_bytes(w.B, w.H, w.T, w.dk, w.dv, 2)
    return {"ms_per_step": 1e3 * wall / steps, "event_ms_mean": mean_ms, "event_ms_median": med_ms, "event_ms_mean_per_call": pc_mean, "tokens_per_s": w.B * w.T * steps / wall,
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

    wall, mean_ms, pc_mean, med_ms = time_calls(step, steps, warmup, torch.cuda.current_stream(dev), WARM_S)
    nbytes = delta_backward_bytes(w.B, w.H, w.T, w.dk, w.dv, 2, gated)
    return {"ms_per_step": 1e3 * wall / steps, "event_ms_mean": mean_ms, "event_ms_median": med_ms, "event_ms_mean_per_call": pc_mean, "tokens_per_s": w.B * w.T * steps / wall,
            "bytes": nbytes, "gbs": nbytes / (mean_ms * 1e-3) / 1e9}


def bench_delta_train(w, steps, warmup, copies, lin, wl):
    """One training step of the delta rule (gated for a gated workload):
    the forward and the backward of a random dO, timed twice -- as
    delta_forward + delta_backward (the backward recomputes the forward's
    context) and as delta_forward_train + delta_backward_after_forward (the
    forward keeps it)."""
    dev = torch.device("cuda:0")
    gated = w.kind == "gated_delta"
    sets = []
    for i in range(copies):
        q, k, v, beta = wl.delta_inputs(w.B, w.H, w.T, w.dk, w.dv, w.dtype, w.seed + 17 * i, dev)
        dO = wl.la_inputs(w.B, w.H, w.T, w.dv, w.dv, w.dtype, w.seed + 17 * i + 1, dev)[0]
        alpha = wl.gates((w.B, w.H, w.T), w.seed + 17 * i, dev) if gated else None
        sets.append((q, k, v, beta, dO, alpha))
    outs = [torch.empty((w.B, w.H, w.T, w.dv), dtype=w.dtype, device=dev) for _ in range(copies)]
    grads = [tuple(torch.empty_like(x) for x in st[:3]) for st in sets]
    S = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(lin.delta_backward_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv), dtype=torch.uint8, device=dev)

    def separate(i):
        q, k, v, beta, dO, alpha = sets[i % copies]
        dq, dk, dv = grads[i % copies]
        if gated:
            lin.gated_delta_forward(q, k, v, beta, alpha, o=outs[i % copies], S_out=S, workspace=ws)
        else:
            lin.delta_forward(q, k, v, beta, o=outs[i % copies], S_out=S, workspace=ws)
        lin.delta_backward(q, k, v, beta, dO, alpha, dq=dq, dk=dk, dv=dv, return_state_grad=False, workspace=ws)

    def paired(i):
        q, k, v, beta, dO, alpha = sets[i % copies]
        dq, dk, dv = grads[i % copies]
        lin.delta_forward_train(q, k, v, beta, alpha, o=outs[i % copies], S_out=S, workspace=ws)
        lin.delta_backward_after_forward(q, k, v, beta, dO, ws, alpha, dq=dq, dk=dk, dv=dv, return_state_grad=False)

    def forward_only(i):  # the training forward alone: the pair less this is the backward
        q, k, v, beta, dO, alpha = sets[i % copies]
        lin.delta_forward_train(q, k, v, beta, alpha, o=outs[i % copies], S_out=S, workspace=ws)

    stream = torch.cuda.current_stream(dev)
    res = {}
    for name, fn in (("separate", separate), ("training_pair", paired), ("forward_train", forward_only)):
        wall, mean_ms, pc_mean, med_ms = time_calls(fn, steps, warmup, stream, WARM_S)
        res[name] = {"ms_per_step": 1e3 * wall / steps, "us_per_step": 1e3 * mean_ms,
                     "us_per_step_median": 1e3 * med_ms, "tokens_per_s": w.B * w.T * steps / wall}
    res["backward_after_forward_us"] = res["training_pair"]["us_per_step"] - res["forward_train"]["us_per_step"]
    return res


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

    wall, mean_ms, pc_mean, med_ms = time_calls(step, steps, warmup, torch.cuda.current_stream(dev), WARM_S)
    nbytes = la_bytes(1, w.H, w.T, w.dk, w.dv, 2) + (w.B - 1) * w.H * (w.dk * w.dv + w.dk) * 4
    lengths = (cu[1:] - cu[:-1]).tolist()
    return {"ms_per_step": 1e3 * wall / steps, "event_ms_mean": mean_ms, "event_ms_median": med_ms, "event_ms_mean_per_call": pc_mean, "tokens_per_s": w.T * steps / wall,
            "gbs": nbytes / (mean_ms * 1e-3) / 1e9, "requests": w.B, "min_len": min(lengths),
            "max_len": max(lengths)}


def bench_decode(w, lin, wl, n_steps=None):
    dev = torch.device("cuda:0")
    S, z, Q, K, V = wl.make(w, dev)
    n = w.T if n_steps is None else n_steps
    o = torch.empty((w.B, w.H, w.dv), dtype=w.dtype, device=dev)

    def step(i):
        lin.la_decode_step(Q[i % w.T], K[i % w.T], V[i % w.T], S, z, eps=1e-6, o=o)

    wall, mean_ms, pc_mean, med_ms = time_calls(step, n, 10, torch.cuda.current_stream(dev), WARM_S)
    per = decode_bytes(w.B, w.H, w.dk, w.dv, 2)
    return {"steps": n, "ms_per_step": 1e3 * wall / n, "event_ms_mean": mean_ms, "event_ms_median": med_ms, "event_ms_mean_per_call": pc_mean, "bytes_per_step": per,
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

    wall, mean_ms, pc_mean, med_ms = time_calls(step, n, 10, torch.cuda.current_stream(dev), WARM_S)
    per = delta_decode_bytes(w.B, w.H, w.dk, w.dv, 2, gated)
    return {"steps": n, "ms_per_step": 1e3 * wall / n, "event_ms_mean": mean_ms, "event_ms_median": med_ms, "event_ms_mean_per_call": pc_mean, "bytes_per_step": per,
            "gbs_wall": per * n / wall / 1e9, "gbs": per / (mean_ms * 1e-3) / 1e9}


def _timed_passes(run, min_seconds, max_passes):
    """Whole passes of run() until min_seconds of wall time (at least one)."""
    passes, total = 0, 0.0
    while passes < max_passes and (passes == 0 or total < min_seconds):
        t0 = time.perf_counter()
        run()
        total += time.perf_counter() - t0
        passes += 1
    return passes, total


def cpu_baseline(w, oracle, wl, min_seconds=5.0):
    """The fp64 oracle on the host over every head of the prefill workload
    (inputs from the same recipe, generated on the CPU), repeated in whole
    passes until about min_seconds have run."""
    q, k, v = wl.la_inputs(w.B, w.H, w.T, w.dk, w.dv, w.dtype, w.seed, "cpu")
    qs, ks, vs = (oracle._f64(t) for t in (q, k, v))
    del q, k, v
    passes, total = _timed_passes(lambda: oracle.la_forward(qs, ks, vs, eps=1e-6), min_seconds, 30)
    dt = total / passes
    return {"value": w.B * w.T / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the whole workload (all {w.B * w.H} heads x T={w.T}), {passes} passes; "
                      f"{total:.2f} s wall in total, {dt:.3f} s per pass", "seconds": dt}


def cpu_baseline_decode(w, oracle, wl, min_seconds=5.0):
    """The fp64 oracle's decode step on the host over every state of the
    decode workload, step after step, until about min_seconds have run;
    reported as steps/s and as the equivalent state-update GB/s."""
    S, z = wl.decode_state(w.B, w.H, w.dk, w.dv, w.seed, "cpu")
    nt = 8
    Q, K, V = wl.decode_tokens(nt, w.B, w.H, w.dk, w.dv, w.dtype, w.seed, "cpu")
    st = {"S": oracle._f64(S), "z": oracle._f64(z), "i": 0}
    toks = [tuple(oracle._f64(x[j]) for x in (Q, K, V)) for j in range(nt)]

    def one():
        q, k, v = toks[st["i"] % nt]
        _, st["S"], st["z"] = oracle.la_decode_step(q, k, v, st["S"], st["z"], eps=1e-6)
        st["i"] += 1

    steps, total = _timed_passes(one, min_seconds, 200)
    per = decode_bytes(w.B, w.H, w.dk, w.dv, 2)
    return {"value": per * steps / total / 1e9, "unit": "GB/s", "steps_per_s": steps / total,
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"all {w.B * w.H} states, {steps} consecutive steps (of the chain's {w.T}); "
                      f"{total:.2f} s wall in total", "seconds_per_step": total / steps}


def calibrate_copy(nbytes=1 << 30):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    dev = torch.device("cuda:0")
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": nbytes, "launches": 3}))


def copy_reference(nbytes=1 << 30, calls=20):
    """What a plain device copy reaches on this GPU (bytes read + bytes
    written per second), as the practical ceiling the HBM fractions above
    are read against."""
    dev = torch.device("cuda:0")
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    wall, mean_ms, pc_mean, med_ms = time_calls(lambda i: b.copy_(a), calls, 5, torch.cuda.current_stream(dev))
    gbs = 2 * nbytes / (mean_ms * 1e-3) / 1e9
    return {"bytes_moved_per_copy": 2 * nbytes, "gbs": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS,
            "us_per_copy": 1e3 * mean_ms}


def hbm_roofline(nbytes, r, workload, kernel):
    """The HBM roofline object of one launch: algorithmic bytes over the mean
    per-call duration, and the counter traffic when taken on these sources."""
    gbs = nbytes / (r["event_ms_mean"] * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": traffic_bytes(workload),
            "traffic_unit": "HBM bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
            "kernel": kernel, "algorithmic_bytes_per_launch": nbytes,
            "event_ms_mean": r["event_ms_mean"],
            "event_ms_per_call": {"median": r["event_ms_median"], "mean": r["event_ms_mean_per_call"],
                                  "note": "one event pair per call; each pair adds a few microseconds"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # A cold device takes about 100 back-to-back launches (some 30 ms of
    # sustained load) to reach its steady clocks: on the long-stream
    # workload groups of ten launches measured 524, 321, 309, 294, 280 ... us
    # each, then 262-268 us from the ninth group on.  The default warm-up
    # covers that, so the timed steps measure the sustained rate.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--only", choices=["all", "la", "la_long", "la_packed", "la_backward", "delta", "gated_delta",
                                       "delta_backward", "delta_train", "copy", "ssd", "decode", "delta_decode",
                                       "gated_delta_decode", "ssd_decode"],
                    default="all")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baselines")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="steps of each decode chain (default: the workload's 1000; fewer for profiling runs)")
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
    head = wl.LA_BF16_LONG
    main_res = dec_res = None
    extra = {}
    if args.only in ("all", "la_long"):
        # two rotating copies of the inputs (1.6 GB) keep every step's reads out of the Infinity Cache
        main_res = bench_la(head, args.steps, args.warmup, 2, lin, wl)
    if args.only in ("all", "decode"):
        dec_res = bench_decode(wl.DECODE_BF16, lin, wl, args.decode_steps)
    if args.only in ("all", "la"):
        w = wl.LA_BF16_PREFILL
        r = bench_la(w, max(20, args.steps), args.warmup, 4, lin, wl, WARM_S)
        extra[w.name] = {"tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"],
                         "roofline": hbm_roofline(r["bytes"], r, w.name, "la_fused_kernel<bf16, 64, 64>"),
                         "mfma_tflops": r["tflops"], "mfma_frac": r["tflops"] / BF16_MFMA_PEAK_TFS}
    if args.only in ("all", "la_backward"):
        w = wl.LA_BF16_PREFILL
        r = bench_la_backward(w, max(3, args.steps // 2), 3, 4, lin, wl)
        extra["la_backward_" + w.name] = {"tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"],
                                          "us_per_call": 1e3 * r["event_ms_mean"],
                                          "us_per_call_median": 1e3 * r["event_ms_median"], "hbm_gbs": r["gbs"],
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
        r = bench_delta(wd, max(5, args.steps // 2), 5, 2, lin, wl)
        extra[wd.name] = {"tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"],
                          "us_per_call": 1e3 * r["event_ms_mean"], "us_per_call_median": 1e3 * r["event_ms_median"],
                          "hbm_gbs": r["gbs"], "hbm_frac": r["gbs"] / HBM_PEAK_GBS,
                          "mfma_tflops": r["tflops"], "mfma_frac": r["tflops"] / BF16_MFMA_PEAK_TFS}
    if args.only in ("all", "delta_backward"):
        for wd in (wl.DELTA_BF16_PREFILL, wl.GATED_DELTA_BF16_PREFILL):
            r = bench_delta_backward(wd, max(5, args.steps // 5), 3, 2, lin, wl)
            extra["delta_backward_" + wd.name] = {"tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"],
                                                  "us_per_call": 1e3 * r["event_ms_mean"],
                                                  "us_per_call_median": 1e3 * r["event_ms_median"],
                                                  "hbm_gbs": r["gbs"],
                                                  "hbm_frac": r["gbs"] / HBM_PEAK_GBS, "bytes_per_call": r["bytes"]}
    if args.only in ("all", "delta_train"):
        for wd in (wl.DELTA_BF16_PREFILL, wl.GATED_DELTA_BF16_PREFILL):
            extra["train_step_" + wd.name] = bench_delta_train(wd, max(5, args.steps // 5), 3, 2, lin, wl)
    if args.only in ("all", "copy"):
        extra["hbm_copy_reference_1gib"] = copy_reference()
    if args.only in ("all", "ssd"):
        ws_ = wl.SSD_BF16_PREFILL
        r = bench_ssd(ws_, max(3, args.steps // 2), 3, 4, lin, wl)
        extra[ws_.name] = {"tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"],
                           "us_per_call": 1e3 * r["event_ms_mean"], "hbm_gbs": r["gbs"],
                           "hbm_frac": r["gbs"] / HBM_PEAK_GBS,
                           "mfma_tflops": r["tflops"], "mfma_frac": r["tflops"] / BF16_MFMA_PEAK_TFS}
    for key, wdd in (("delta_decode", wl.DELTA_DECODE_BF16), ("gated_delta_decode", wl.GATED_DELTA_DECODE_BF16)):
        if args.only not in ("all", key):
            continue
        r = bench_delta_decode(wdd, lin, wl, args.decode_steps)
        extra[wdd.name] = {"state_update_gbs": r["gbs"], "hbm_frac": r["gbs"] / HBM_PEAK_GBS,
                           "gbs_wall_incl_launch_gaps": r["gbs_wall"], "us_per_step": 1e3 * r["event_ms_mean"],
                           "us_per_step_median": 1e3 * r["event_ms_median"],
                           "steps": r["steps"], "bytes_per_step": r["bytes_per_step"]}
    if args.only in ("all", "ssd_decode"):
        wsd = wl.SSD_DECODE_BF16
        r = bench_ssd_decode(wsd, lin, wl, args.decode_steps)
        extra[wsd.name] = {"state_update_gbs": r["gbs"], "hbm_frac": r["gbs"] / HBM_PEAK_GBS,
                           "gbs_wall_incl_launch_gaps": r["gbs_wall"], "us_per_step": 1e3 * r["event_ms_mean"],
                           "us_per_step_median": 1e3 * r["event_ms_median"],
                           "steps": r["steps"], "bytes_per_step": r["bytes_per_step"]}

    decode = None
    if dec_res is not None:
        wd = wl.DECODE_BF16
        decode = {"metric": "decode state-update GB/s", "value": dec_res["gbs_wall"], "unit": "GB/s",
                  "workload": wd.name, "steps": dec_res["steps"], "us_per_step": 1e3 * dec_res["ms_per_step"],
                  "roofline": hbm_roofline(dec_res["bytes_per_step"], dec_res, wd.name,
                                           "la_decode_kernel<bf16, 128, 128> (the one launch of la_decode_step)"),
                  "cpu_baseline": None}
        if not args.no_cpu:
            import oracle  # test infrastructure, used only for the CPU baseline legs
            decode["cpu_baseline"] = cpu_baseline_decode(wd, oracle, wl)
    if main_res is None:
        print(json.dumps({"decode": decode, "extra": extra}))
        return

    cpu = None
    if not args.no_cpu:
        import oracle  # test infrastructure, used only for the CPU baseline legs
        cpu = cpu_baseline(head, oracle, wl)

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
        "data": "synthetic (seeded N(0,1) q,k,v; generated on device; 2 rotating copies)",
        "config": {"workload": head.name, "B": head.B, "H": head.H, "T": head.T, "dk": head.dk, "dv": head.dv,
                   "chunk": 64, "state": "fp32"},
        "roofline": dict(hbm_roofline(main_res["bytes"], main_res, head.name,
                                      "la_fused_kernel<bf16, 64, 64> (the one launch of la_forward)"),
                         mfma_tflops=main_res["tflops"], mfma_frac=main_res["tflops"] / BF16_MFMA_PEAK_TFS),
        "cpu_baseline": cpu,
        "decode": decode,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
