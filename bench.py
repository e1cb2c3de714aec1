"""Benchmark of the EXL3 linear layer on one MI355X.

Headline workload: the dense decode GEMV of a k=5120 x n=17408 EXL3 tensor at
K=4 bits with one activation row (M=1): one step is one exl3_linear call
(input sign + transform, trellis stream and decode, contraction, split-k sum,
output transform + svh, cast).  25 copies of the trellis (1.11 GB) are used
in rotation so that successive steps read HBM, not the 256 MB last-level
cache.  `value` is the whole-job rate of the metric (algorithmic bytes of the
call per second); `roofline` reports the call's kernel pair (the persistent
decode/contraction kernel and the small split-k finishing kernel after it on
the same stream), timed per call with HIP events on the launch stream.  The
float64 oracle is timed on the host on the same workload as the CPU baseline.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                [--no-secondary] [--profile-pass [gemv|prefill|prefill_int8|moe4096|moe1|mixed1]]

--profile-pass runs a short fixed sequence for counter collection instead of
the benchmark: a plain 256 MiB device copy (the scale of the HBM byte
counters), then a few calls of one leg.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix, published
MFMA_I8_PEAK_TOPS = 5000.0     # MI355X dense int8 matrix, published
METRIC = "EXL3 GEMV HBM GB/s (% of 8 TB/s) at M=1; prefill GEMM TFLOPS (% MFMA)"
GEMV_SOURCES = ["gemm_exl3_linear_amd/csrc/exl3_device.hpp", "gemm_exl3_linear_amd/csrc/exl3_gemv_mf.hpp",
                "gemm_exl3_linear_amd/csrc/exl3_sk_split.hpp", "gemm_exl3_linear_amd/csrc/exl3_gemv.hip"]
GEMV_KERNELS = "gemv_mf_kernel<4, 1> + gemv_mf_finish<true>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_dense_5120x17408_k4_m1_traffic.json")


def gemv_source_hash() -> str:
    h = hashlib.sha256()
    for p in GEMV_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def linear_bytes(k, n, bits, m, out_bytes=2):
    """Algorithmic bytes of one call: trellis + suh + svh + x + y, each once."""
    return k * n * bits // 8 + 2 * k + 2 * n + 2 * m * k + out_bytes * m * n


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the GEMV sources changed after the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemv_source_hash") != gemv_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def time_calls(fn, steps, warmup, stream, median=False):
    """Returns (mean per-launch time from per-call event pairs, whole-loop time),
    and with median=True also the median of the per-call event pairs.

    Two timed passes over the same `steps` calls: the whole-loop time comes
    from one event pair around back-to-back calls (nothing recorded between
    them), the per-launch time from an event pair around each call."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        fn(warmup + i)
    t1.record(stream)
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1) * 1e-3
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        fn(warmup + i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    times = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    per = sum(times) / steps
    if median:
        return per * 1e-3, total, times[steps // 2] * 1e-3
    return per * 1e-3, total


def time_graph(calls, replays, stream):
    """Per-call time of `calls` (a list of functions taking a stream) captured
    into one graph and replayed: the GPU time of the calls without the host's
    per-call cost."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        g.capture_begin()
        for c in calls:
            c(side)
        g.capture_end()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(3):
            g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        t0.record(stream)
        for _ in range(replays):
            g.replay()
        t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e-3 / (replays * len(calls))


def bench_lib():
    """The benchmark's measurement kernels (libexl3_bench.so)."""
    import ctypes
    path = os.path.join(ROOT, "gemm_exl3_linear_amd", "libexl3_bench.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build first (python -m gemm_exl3_linear_amd.build)")
    L = ctypes.CDLL(path)
    L.exl3_bench_stream_read.restype = ctypes.c_int
    L.exl3_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_void_p]
    return L


def host_call_times(X, weights, x, y, ws, stream, calls=200):
    """Seconds of host time per exl3_linear call: (Python binding, direct C
    ABI call through ctypes with prepared arguments)."""
    import ctypes
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(calls):
        X.exl3_linear(x, weights[i % len(weights)], out=y, workspace=ws, stream=stream)
    py = (time.perf_counter() - t0) / calls
    torch.cuda.synchronize()
    L = X.lib()
    recs = [w._c() for w in weights]
    refs = [ctypes.byref(r) for r in recs]
    xp, yp, wp = x.data_ptr(), y.data_ptr(), ws.data_ptr()
    ldx, ldy, nws, sp = x.stride(0), y.stride(0), ws.numel(), stream.cuda_stream
    t0 = time.perf_counter()
    for i in range(calls):
        L.exl3_linear(refs[i % len(refs)], xp, 1, ldx, yp, ldy, 0, wp, nws, sp)
    c = (time.perf_counter() - t0) / calls
    torch.cuda.synchronize()
    return py, c


def read_ceiling(buffers, nbytes, stream, reps=200):
    """Practical HBM read ceiling: a plain streaming-read kernel over the same
    rotated buffers the GEMV reads, back to back; the best of a few launch
    shapes."""
    import torch
    B = bench_lib()
    sink = torch.empty(1 << 13, dtype=torch.int32, device=buffers[0].device)
    best = None
    for wg in (1024, 2048, 4096):
        for un in (4, 8):
            def call(i, wg=wg, un=un):
                rc = B.exl3_bench_stream_read(buffers[i % len(buffers)].data_ptr(), nbytes, sink.data_ptr(), wg, un,
                                              stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"stream read launch failed ({rc})")
            per, total, med = time_calls(call, reps, 20, stream, median=True)
            gbs = nbytes * reps / total / 1e9
            if best is None or gbs > best["GB/s"]:
                best = {"GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                        "us_per_read": round(total / reps * 1e6, 3), "us_per_read_event_median": round(med * 1e6, 3),
                        "workgroups": wg, "loads_in_flight_per_thread": un, "bytes": nbytes,
                        "kernel": f"stream_read_kernel<{un}>"}
    return best


def moe_id_sets(ids, experts, torch, dev):
    """Routing for the one-token legs: the drawn token's top-k slots mapped
    onto `experts / topk` disjoint expert sets that together cover every
    expert (a seeded permutation), so that rotating through them makes each
    call read its experts' weights from HBM, not from the last-level cache."""
    import numpy as np
    topk = ids.shape[1]
    perm = np.random.default_rng(11).permutation(experts).astype(np.int32)
    return [torch.from_numpy(perm[i * topk:(i + 1) * topk].reshape(1, topk).copy()).to(dev)
            for i in range(experts // topk)]


def moe_t1_bytes(mo):
    """Algorithmic bytes of one routed-expert call at one token: the trellis
    and signs of the gate, up and down tensors of the topk experts it
    reaches, x, the fp32 output and the routing, each once."""
    t, topk = mo["ids"].shape
    gu, dn = mo["gate_up"], mo["down"]
    per_expert = 0
    for arena, slots in ((gu, 2), (dn, 1)):
        k, n, b = arena["k"], arena["n"], arena["bits"]
        per_expert += slots * (k * n * b // 8 + 2 * k + 2 * n)
    return topk * t * per_expert + 2 * t * gu["k"] + 4 * t * gu["k"] + 8 * t * topk


def mixed_layer_leg(X, torch, synth, dev, stream, reps=50):
    """The mixed-width decoder layer: q, k, v, o (5120 x 5120), gate, up
    (5120 x 17408), down (17408 x 5120) with per-tensor widths drawn from 2..8.
    M = 1: the seven projections run in layer order, repeatedly, each call
    timed with its own event pair (between two calls of one tensor the other
    six stream about 220 MB, so each call reads mostly HBM), then again with
    the projections that read one input fused into one exl3_linear_multi call
    each ((q, k, v), o, (gate, up), down); M = 4096: each projection timed
    alone (the MFMA-bound prefill), through the fp16 and the int8 path."""
    out = {"bits": {}, "m1": {}, "m4096": {}, "m4096_int8": {}}
    d1 = synth.mixed_layer_inputs(synth.SEED_MIXED_LAYER, 1)
    names = [nm for nm, _, _ in synth.MIXED_LAYER_SHAPES]
    ws, xs, ys = {}, {}, {}
    for nm in names:
        d = d1[nm]
        out["bits"][nm] = d["bits"]
        ws[nm] = X.Exl3Weight.from_numpy(d["trellis"], d["suh"], d["svh"], d["bits"], device=dev)
        xs[nm] = torch.from_numpy(d["x"]).to(dev)
        ys[nm] = torch.empty((1, d["n"]), dtype=torch.float16, device=dev)
    wsp = torch.zeros(max(X.exl3_linear_workspace_size(ws[nm], 4096) for nm in names),
                      dtype=torch.uint8, device=dev)
    for _ in range(3):
        for nm in names:
            X.exl3_linear(xs[nm], ws[nm], out=ys[nm], workspace=wsp, stream=stream)
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in names]
          for _ in range(reps)]
    for r in range(reps):
        for i, nm in enumerate(names):
            ev[r][i][0].record(stream)
            X.exl3_linear(xs[nm], ws[nm], out=ys[nm], workspace=wsp, stream=stream)
            ev[r][i][1].record(stream)
    torch.cuda.synchronize()
    tot_b = tot_t = 0.0
    for i, nm in enumerate(names):
        d = d1[nm]
        t = sum(ev[r][i][0].elapsed_time(ev[r][i][1]) for r in range(reps)) / reps * 1e-3
        b = linear_bytes(d["k"], d["n"], d["bits"], 1)
        tot_b += b
        tot_t += t
        out["m1"][nm] = {"us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                         "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 4)}
    out["m1"]["layer"] = {"us": round(tot_t * 1e6, 2), "GB/s": round(tot_b / tot_t / 1e9, 1),
                          "frac_hbm": round(tot_b / tot_t / 1e9 / HBM_PEAK_GBS, 4)}
    # the seven calls captured into one graph and replayed: the layer's GPU
    # time without the host's per-call cost
    layer_calls = [lambda st, nm=nm: X.exl3_linear(xs[nm], ws[nm], out=ys[nm], workspace=wsp, stream=st)
                   for nm in names]
    tg = time_graph(layer_calls, 20, stream) * len(names)
    out["m1"]["layer_graph_replay"] = {"us": round(tg * 1e6, 2), "GB/s": round(tot_b / tg / 1e9, 1),
                                       "frac_hbm": round(tot_b / tg / 1e9 / HBM_PEAK_GBS, 4)}
    # the same layer with the projections that share an input fused into one
    # exl3_linear_multi call each: (q, k, v), o, (gate, up), down
    groups = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    gouts = {g: [ys[nm] for nm in g] for g in groups}
    gws = {g: [ws[nm] for nm in g] for g in groups}
    wsm = torch.zeros(max(X.exl3_linear_multi_workspace_size(gws[g], 1) for g in groups), dtype=torch.uint8,
                      device=dev)
    def gcall(g):
        X.exl3_linear_multi(xs[g[0]], gws[g], outs=gouts[g], workspace=wsm, stream=stream)
    for _ in range(3):
        for g in groups:
            gcall(g)
    torch.cuda.synchronize()
    evg = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in groups]
           for _ in range(reps)]
    for r in range(reps):
        for i, g in enumerate(groups):
            evg[r][i][0].record(stream)
            gcall(g)
            evg[r][i][1].record(stream)
    torch.cuda.synchronize()
    out["m1_fused"] = {}
    tot_t = 0.0
    for i, g in enumerate(groups):
        t = sum(evg[r][i][0].elapsed_time(evg[r][i][1]) for r in range(reps)) / reps * 1e-3
        b = sum(linear_bytes(d1[nm]["k"], d1[nm]["n"], d1[nm]["bits"], 1) for nm in g)
        tot_t += t
        out["m1_fused"]["+".join(g)] = {"us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                                        "frac_hbm": round(b / t / 1e9 / HBM_PEAK_GBS, 4)}
    out["m1_fused"]["layer"] = {"us": round(tot_t * 1e6, 2), "GB/s": round(tot_b / tot_t / 1e9, 1),
                                "frac_hbm": round(tot_b / tot_t / 1e9 / HBM_PEAK_GBS, 4)}
    tg = time_graph([lambda st, g=g: X.exl3_linear_multi(xs[g[0]], gws[g], outs=gouts[g], workspace=wsm, stream=st)
                     for g in groups], 20, stream) * len(groups)
    out["m1_fused"]["layer_graph_replay"] = {"us": round(tg * 1e6, 2), "GB/s": round(tot_b / tg / 1e9, 1),
                                             "frac_hbm": round(tot_b / tg / 1e9 / HBM_PEAK_GBS, 4)}
    del wsm
    del xs, ys
    d4 = synth.mixed_layer_inputs(synth.SEED_MIXED_LAYER, 4096)
    ws8 = torch.empty(max(X.exl3_linear_int8_workspace_size(ws[nm], 4096) for nm in names), dtype=torch.uint8,
                      device=dev)
    tot_f = tot_t = tot_t8 = 0.0
    for nm in names:
        d = d4[nm]
        x4 = torch.from_numpy(d["x"]).to(dev)
        y4 = torch.empty((4096, d["n"]), dtype=torch.float16, device=dev)
        pl, _ = time_calls(lambda i: X.exl3_linear(x4, ws[nm], out=y4, workspace=wsp, stream=stream),
                           10, 2, stream)
        pl8, _ = time_calls(lambda i: X.exl3_linear_int8(x4, ws[nm], out=y4, workspace=ws8, stream=stream),
                            10, 2, stream)
        f = 2.0 * 4096 * d["k"] * d["n"]
        tot_f += f
        tot_t += pl
        tot_t8 += pl8
        out["m4096"][nm] = {"ms": round(pl * 1e3, 3), "TFLOP/s": round(f / pl / 1e12, 1),
                            "frac_mfma_f16": round(f / pl / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}
        out["m4096_int8"][nm] = {"ms": round(pl8 * 1e3, 3), "TOP/s": round(f / pl8 / 1e12, 1),
                                 "frac_mfma_i8": round(f / pl8 / 1e12 / MFMA_I8_PEAK_TOPS, 4)}
        del x4, y4
    out["m4096"]["layer"] = {"ms": round(tot_t * 1e3, 3), "TFLOP/s": round(tot_f / tot_t / 1e12, 1),
                             "frac_mfma_f16": round(tot_f / tot_t / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}
    out["m4096_int8"]["layer"] = {"ms": round(tot_t8 * 1e3, 3), "TOP/s": round(tot_f / tot_t8 / 1e12, 1),
                                  "frac_mfma_i8": round(tot_f / tot_t8 / 1e12 / MFMA_I8_PEAK_TOPS, 4)}
    del ws, wsp, ws8, d1, d4
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--profile-pass", nargs="?", const="gemv", default=None,
                    choices=["gemv", "prefill", "prefill_int8", "moe4096", "moe1", "mixed1"],
                    help="short run for counter collection: a plain copy of known size, then a few calls of "
                         "one leg (gemv: 50 M=1 calls; prefill / prefill_int8: 10 M=4096 calls; moe4096: 5 "
                         "routed-expert calls at T=4096; moe1: 64 at T=1, routing rotated over all experts; "
                         "mixed1: the mixed-width layer's seven M=1 projections, 10 times in layer order)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gemm_exl3_linear_amd as X
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    X.lib()  # fail loudly if the library is missing
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    k, n, bits = 5120, 17408, 4
    d = synth.linear_inputs(synth.SEED_DENSE_5120x17408, 16, k, n, bits)
    trellis_bytes = k * n * bits // 8
    copies = -(-(1 << 30) // trellis_bytes)
    t_host = torch.from_numpy(d["trellis"].view(np.int16).copy())
    trellis = [t_host.to(dev) for _ in range(copies)]
    suh = torch.from_numpy(d["suh"]).to(dev)
    svh = torch.from_numpy(d["svh"]).to(dev)
    xs = torch.from_numpy(d["x"]).to(dev)
    weights = [X.Exl3Weight(t, suh, svh, bits) for t in trellis]
    ws = torch.zeros(max(X.exl3_linear_workspace_size(weights[0], m) for m in (1, 4, 16)),
                     dtype=torch.uint8, device=dev)
    y = torch.empty((16, n), dtype=torch.float16, device=dev)

    def gemv(m):
        def call(i):
            X.exl3_linear(xs[:m], weights[i % copies], out=y[:m], workspace=ws, stream=stream)
        return call

    if args.profile_pass:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        kind = args.profile_pass
        if kind == "gemv":
            for i in range(50):
                gemv(1)(i)
            calls = 50
        elif kind in ("prefill", "prefill_int8"):
            dp = synth.linear_inputs(synth.SEED_PREFILL_4096x5120x17408, 4096, k, n, bits)
            wp = X.Exl3Weight.from_numpy(dp["trellis"], dp["suh"], dp["svh"], bits, device=dev)
            xp = torch.from_numpy(dp["x"]).to(dev)
            yp = torch.empty((4096, n), dtype=torch.float16, device=dev)
            if kind == "prefill":
                wsp = torch.zeros(X.exl3_linear_workspace_size(wp, 4096), dtype=torch.uint8, device=dev)
                fn = lambda: X.exl3_linear(xp, wp, out=yp, workspace=wsp, stream=stream)
            else:
                wsp = torch.empty(X.exl3_linear_int8_workspace_size(wp, 4096), dtype=torch.uint8, device=dev)
                fn = lambda: X.exl3_linear_int8(xp, wp, out=yp, workspace=wsp, stream=stream)
            calls = 10
            for _ in range(calls):
                fn()
        elif kind == "moe1":
            # one token, routing rotated over the disjoint id sets that cover
            # all 256 experts (each call reads its experts from HBM)
            mo = synth.moe_inputs(synth.SEED_MOE_256x2048x512, 1)
            gu = X.Exl3Arena.from_numpy(mo["gate_up"], dev)
            dn = X.Exl3Arena.from_numpy(mo["down"], dev)
            xm = torch.from_numpy(mo["x"]).to(dev)
            ids_list = moe_id_sets(mo["ids"], 256, torch, dev)
            wt = torch.from_numpy(mo["weights"]).to(dev)
            wsm = torch.zeros(X.exl3_grouped_experts_workspace_size(gu, dn, 1, 8), dtype=torch.uint8, device=dev)
            ym = torch.empty((1, 2048), dtype=torch.float32, device=dev)
            calls = 2 * len(ids_list)
            for i in range(calls):
                X.exl3_grouped_experts(xm, ids_list[i % len(ids_list)], wt, gu, dn, out=ym, workspace=wsm,
                                       stream=stream)
        elif kind == "mixed1":
            # the mixed-width layer at M=1: the seven projections in layer order
            d1 = synth.mixed_layer_inputs(synth.SEED_MIXED_LAYER, 1)
            names = [nm for nm, _, _ in synth.MIXED_LAYER_SHAPES]
            wl = {nm: X.Exl3Weight.from_numpy(d1[nm]["trellis"], d1[nm]["suh"], d1[nm]["svh"], d1[nm]["bits"],
                                              device=dev) for nm in names}
            xl = {nm: torch.from_numpy(d1[nm]["x"]).to(dev) for nm in names}
            yl = {nm: torch.empty((1, d1[nm]["n"]), dtype=torch.float16, device=dev) for nm in names}
            wsl = torch.zeros(max(X.exl3_linear_workspace_size(wl[nm], 1) for nm in names), dtype=torch.uint8,
                              device=dev)
            calls = 10
            for _ in range(calls):
                for nm in names:
                    X.exl3_linear(xl[nm], wl[nm], out=yl[nm], workspace=wsl, stream=stream)
        else:
            mo = synth.moe_inputs(synth.SEED_MOE_256x2048x512, 4096)
            gu = X.Exl3Arena.from_numpy(mo["gate_up"], dev)
            dn = X.Exl3Arena.from_numpy(mo["down"], dev)
            xm = torch.from_numpy(mo["x"]).to(dev)
            ids = torch.from_numpy(mo["ids"]).to(dev)
            wt = torch.from_numpy(mo["weights"]).to(dev)
            wsm = torch.zeros(X.exl3_grouped_experts_workspace_size(gu, dn, 4096, 8), dtype=torch.uint8, device=dev)
            ym = torch.empty((4096, 2048), dtype=torch.float32, device=dev)
            calls = 5
            for _ in range(calls):
                X.exl3_grouped_experts(xm, ids, wt, gu, dn, out=ym, workspace=wsm, stream=stream)
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass": kind, "copy_bytes": 256 << 20, "calls": calls,
                          "gemv_source_hash": gemv_source_hash()}))
        return

    per_launch, total, per_median = time_calls(gemv(1), args.steps, args.warmup, stream, median=True)
    nbytes = linear_bytes(k, n, bits, 1)
    value = nbytes * args.steps / total / 1e9
    achieved = nbytes / per_launch / 1e9
    # the same calls replayed from one graph (one call per weight copy), and
    # the plain streaming read of the same copies
    graph_t = time_graph([lambda st, w=w: X.exl3_linear(xs[:1], w, out=y[:1], workspace=ws, stream=st)
                          for w in weights], 40, stream)
    # host time to enqueue one call (wall clock over a burst of 200 launches
    # while the GPU works through them): through the Python binding, and
    # through ctypes straight into the C ABI with the arguments prepared
    host_py, host_c = host_call_times(X, weights, xs[:1], y[:1], ws, stream)
    ceiling = read_ceiling(trellis, trellis_bytes, stream)

    secondary = {}
    if not args.no_secondary:
        for m in (4, 16):
            pl, tot = time_calls(gemv(m), 200, 20, stream)
            gb = linear_bytes(k, n, bits, m) / pl / 1e9
            secondary[f"gemv_m{m}"] = {"GB/s": round(gb, 1), "frac_hbm": round(gb / HBM_PEAK_GBS, 4),
                                       "us_per_call": round(pl * 1e6, 2),
                                       "us_per_call_back_to_back": round(tot / 200 * 1e6, 2)}
        # The stream-k v_dot2 kernel at M=1 (the several-tensor call with one
        # tensor): the cost of giving every row count 1..16 one contraction is
        # the difference between this and the headline call on the same box.
        wsd = torch.zeros(X.exl3_linear_multi_workspace_size([weights[0]], 1), dtype=torch.uint8, device=dev)
        pl, tot = time_calls(lambda i: X.exl3_linear_multi(xs[:1], [weights[i % copies]], outs=[y[:1]], workspace=wsd,
                                                           stream=stream), 200, 20, stream)
        gb = nbytes * 200 / tot / 1e9
        secondary["gemv_m1_v_dot2_one_tensor"] = {"GB/s": round(gb, 1), "frac_hbm": round(gb / HBM_PEAK_GBS, 4),
                                                  "us_per_call": round(pl * 1e6, 2),
                                                  "us_per_call_back_to_back": round(tot / 200 * 1e6, 2)}
        del wsd
        # prefill: M=4096 (input transform kernel + fused decode/MFMA GEMM kernel)
        dp = synth.linear_inputs(synth.SEED_PREFILL_4096x5120x17408, 4096, k, n, bits)
        wp = X.Exl3Weight.from_numpy(dp["trellis"], dp["suh"], dp["svh"], bits, device=dev)
        xp = torch.from_numpy(dp["x"]).to(dev)
        wsp = torch.zeros(X.exl3_linear_workspace_size(wp, 4096), dtype=torch.uint8, device=dev)
        yp = torch.empty((4096, n), dtype=torch.float16, device=dev)
        pl, _ = time_calls(lambda i: X.exl3_linear(xp, wp, out=yp, workspace=wsp, stream=stream), 20, 3, stream)
        tf = 2.0 * 4096 * k * n / pl / 1e12
        secondary["prefill_m4096"] = {"TFLOP/s": round(tf, 1), "frac_mfma_f16": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                                      "ms_per_call": round(pl * 1e3, 3)}
        # the same prefill through the int8 path (row-quantizing input transform
        # + fused decode-to-int8 / int8 MFMA GEMM)
        ws8 = torch.empty(X.exl3_linear_int8_workspace_size(wp, 4096), dtype=torch.uint8, device=dev)
        pl8, _ = time_calls(lambda i: X.exl3_linear_int8(xp, wp, out=yp, workspace=ws8, stream=stream), 20, 3,
                            stream)
        to = 2.0 * 4096 * k * n / pl8 / 1e12
        secondary["prefill_int8_m4096"] = {"TOP/s": round(to, 1), "frac_mfma_i8": round(to / MFMA_I8_PEAK_TOPS, 4),
                                           "ms_per_call": round(pl8 * 1e3, 3),
                                           "speedup_vs_fp16": round(pl / pl8, 3)}
        del wp, xp, wsp, yp, ws8
        secondary["mixed_layer"] = mixed_layer_leg(X, torch, synth, dev, stream)
        # routed experts: 256 experts, top-8, hidden 2048, intermediate 512, K=3
        for t in (1, 4096):
            mo = synth.moe_inputs(synth.SEED_MOE_256x2048x512, t)
            gu = X.Exl3Arena.from_numpy(mo["gate_up"], dev)
            dn = X.Exl3Arena.from_numpy(mo["down"], dev)
            xm = torch.from_numpy(mo["x"]).to(dev)
            ids_list = moe_id_sets(mo["ids"], 256, torch, dev) if t == 1 else [torch.from_numpy(mo["ids"]).to(dev)]
            wt = torch.from_numpy(mo["weights"]).to(dev)
            wsm = torch.zeros(X.exl3_grouped_experts_workspace_size(gu, dn, t, 8), dtype=torch.uint8, device=dev)
            ym = torch.empty((t, 2048), dtype=torch.float32, device=dev)
            reps = 200 if t == 1 else 10
            pl, _ = time_calls(lambda i: X.exl3_grouped_experts(xm, ids_list[i % len(ids_list)], wt, gu, dn, out=ym,
                                                                workspace=wsm, stream=stream), reps, 3, stream)
            flops = 2.0 * t * 8 * 3 * 2048 * 512
            leg = {"us_per_call": round(pl * 1e6, 2), "TFLOP/s": round(flops / pl / 1e12, 2)}
            if t == 1:
                b = moe_t1_bytes(mo)
                leg.update({"GB/s": round(b / pl / 1e9, 1), "frac_hbm": round(b / pl / 1e9 / HBM_PEAK_GBS, 4),
                            "algorithmic_bytes": b, "routing": f"{len(ids_list)} id sets rotated over all 256 experts"})
                leg["us_per_call_graph"] = round(time_graph(
                    [lambda st, ids=ids: X.exl3_grouped_experts(xm, ids, wt, gu, dn, out=ym, workspace=wsm, stream=st)
                     for ids in ids_list], 20, stream) * 1e6, 2)
            else:
                leg["frac_mfma_f16"] = round(flops / pl / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)
            secondary[f"moe_t{t}"] = leg
            del gu, dn, xm, ids_list, wt, wsm, ym
        # the same shape with a width per expert drawn from {2, 3, 4}
        for t in (1, 4096):
            mo = synth.moe_mixed_inputs(synth.SEED_MOE_MIXED_WIDTHS, t, widths=(2, 3, 4))
            gu = X.Exl3MixedArena.from_numpy(mo["gate_up"], dev)
            dn = X.Exl3MixedArena.from_numpy(mo["down"], dev)
            xm = torch.from_numpy(mo["x"]).to(dev)
            ids_list = moe_id_sets(mo["ids"], 256, torch, dev) if t == 1 else [torch.from_numpy(mo["ids"]).to(dev)]
            wt = torch.from_numpy(mo["weights"]).to(dev)
            wsm = torch.zeros(X.exl3_grouped_experts_mixed_workspace_size(gu, dn, t, 8), dtype=torch.uint8,
                              device=dev)
            ym = torch.empty((t, 2048), dtype=torch.float32, device=dev)
            reps = 200 if t == 1 else 10
            pl, _ = time_calls(lambda i: X.exl3_grouped_experts_mixed(xm, ids_list[i % len(ids_list)], wt, gu, dn,
                                                                      out=ym, workspace=wsm, stream=stream),
                               reps, 3, stream)
            flops = 2.0 * t * 8 * 3 * 2048 * 512
            leg = {"us_per_call": round(pl * 1e6, 2), "TFLOP/s": round(flops / pl / 1e12, 2)}
            if t == 1:
                leg["routing"] = f"{len(ids_list)} id sets rotated over all 256 experts"
            else:
                leg["frac_mfma_f16"] = round(flops / pl / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)
            secondary[f"moe_mixed_widths_t{t}"] = leg
            del gu, dn, xm, ids_list, wt, wsm, ym

    cpu = None
    if not args.no_cpu_baseline:
        import threadpoolctl
        from oracle import exl3_oracle as O
        x1 = d["x"][:1]
        reps, t_cpu = 0, 0.0
        while reps < 20 and (reps == 0 or t_cpu < 10.0):
            t0 = time.perf_counter()
            O.linear(x1, d["trellis"], d["suh"], d["svh"], bits)
            t_cpu += time.perf_counter() - t0
            reps += 1
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] + [1])
        cpu = {"value": round(nbytes * reps / t_cpu / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"full workload (k=5120, n=17408, K=4, M=1), {reps} pass(es) of the float64 oracle "
                         f"(vectorised decode single-threaded, matrix product on {threads} BLAS threads), "
                         f"{t_cpu:.1f} s, host os.cpu_count()={os.cpu_count()}"}

    traffic = measured_traffic()
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "dense decode GEMV, EXL3 k=5120 n=17408 K=4, M=1, fp16 in/out",
                   "k": k, "n": n, "bits": bits, "m": 1, "weight_copies_rotated": copies,
                   "algorithmic_bytes_per_call": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": GEMV_KERNELS, "us_per_launch": round(per_launch * 1e6, 3),
                     "us_per_launch_median": round(per_median * 1e6, 3),
                     "us_per_call_back_to_back": round(total / args.steps * 1e6, 3),
                     "us_per_call_graph_replay": round(graph_t * 1e6, 3),
                     "host_us_per_call_python": round(host_py * 1e6, 2),
                     "host_us_per_call_c_abi": round(host_c * 1e6, 2),
                     "read_ceiling": ceiling,
                     "frac_of_read_ceiling": round(achieved / ceiling["GB/s"], 4)},
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
