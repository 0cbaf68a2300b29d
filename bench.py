"""Throughput of the WKV operator (RWKV-4 time mixing) on one MI355X.

A step is one forward and one backward pass over one batch of the 3B-class layer shape
(B=8, T=4096, C=2560, fp32): wkv_forward fills y and its workspace, wkv_backward reads
that workspace and writes dk, dv, dw, du. Inputs are synthetic and seeded (the
distributions of the 3B-class layer workload in wkv_inputs.py) and resident in HBM
before timing starts; the step reuses preallocated outputs and workspaces.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-state]
                    [--no-gated] [--no-bf16] [--no-shift]

prints one JSON line. `value` is B*T*C / step time (elements per second of fwd+bwd);
`roofline` describes the kernel that takes most of the step, with its algorithmic bytes
(20 B per element for the backward: k, v, dy read, dk, dv written; 12 B for the
forward: k, v read, y written) over its mean duration from HIP events on the stream the
library launches on. `traffic` comes from a committed rocprofv3 counter summary and is
reported only while the kernel sources still hash to the value recorded there.
`cpu_baseline` times the fp64 CPU oracle (test infrastructure, OpenMP over all host
threads) on the same workload. `decode` reports the batched decode step separately
(B=256, C=5120, 40 layer states, 36 B per element per call; the step's 40 calls replayed
from a captured HIP graph, with the eager Python-launched rate beside it); `forward_state`
the forward
from a given state that also returns the final state (prompt prefill), on the same layer;
`gated` the receptance-gated forward + backward (out = sigma(r) y) on the same layer; `bf16`
the step with the [B, T, C] tensors stored as bfloat16 (reported apart: the benchmark's own
workload is fp32); `token_shift` the mix that produces the projections' inputs.

The default warm-up (200 steps, about 0.12 s) runs the step long enough under sustained
load for the GPU's clocks to settle: over the first ~100 back-to-back steps after idle the
kernels run up to a third slower before they reach a steady rate, and the default timed
steps (100) are taken there.

Helpers for the counter summaries:
    python bench.py --with-copy ...        also runs a 1 GiB device copy (known bytes)
    python bench.py --summarize-counters FETCH_DIR WRITE_DIR
        reads two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` output folders of a
        `--with-copy` run and prints the summary JSON (per-dispatch KiB, copy scaling).
    python bench.py --summarize-trace TRACE_DIR [--warmup W --steps K]
        prints the step's kernel durations from a `rocprofv3 --kernel-trace` folder of a run
        with the same W and K (all dispatches, and the timed ones alone).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
PKG_DIR = os.path.join(HERE, "rwkv_linear_attention_forward_amd")
CSRC = os.path.join(PKG_DIR, "csrc")
COUNTERS = os.path.join(HERE, "profiles", "wkv_l3b_counters.json")
METRIC = ("WKV fwd+bwd elements/sec (B·T·C) and achieved HBM GB/s vs peak, "
          "T=4096 C=2560")
PEAK_GBPS = 8000.0
COPY_BYTES = 1 << 30
# The step's kernels as rocprofv3 names them (the fp32, ungated instances that keep the
# backward's states; the other legs run other instances, or come after the step's
# dispatches).
KERNELS = {"forward": "wkv_forward_kernel<2, 32, false, (wkvdev::Io)0, true>",
           "backward": "wkv_backward_kernel<2, 32, false, (wkvdev::Io)0>"}
REDUCE_KERNEL = "wkv_reduce_kernel"
BYTES_PER_ELEM = {"forward": 12, "backward": 20}


# Sources the forward and backward kernels (and their workspace layout) are built from; the
# decode and token-shift kernels do not change their traffic.
TRAFFIC_SOURCES = ("wkv_api.hip", "wkv_backward.hip", "wkv_chunk.h", "wkv_device.h",
                   "wkv_forward.hip", "wkv_launch.h")


def source_hash() -> str:
    """sha256 over the sources of the forward and backward kernels, in name order."""
    h = hashlib.sha256()
    for path in sorted(os.path.join(CSRC, f) for f in TRAFFIC_SOURCES):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# ---------------------------------------------------------------------------------------
# counter summaries
# ---------------------------------------------------------------------------------------
def _read_counter_rows(folder):
    rows = []
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit("no *counter_collection.csv under %s" % folder)
    return rows


def _per_dispatch(rows, counter):
    """{kernel_name: [value per dispatch]} for one counter (values summed per dispatch)."""
    per = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        key = (r.get("Dispatch_Id"), r.get("Kernel_Name"))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (_, name), val in per.items():
        out.setdefault(name, []).append(val)
    return out


def _match(per, needle):
    vals = [v for name, vs in per.items() if needle in name for v in vs]
    return statistics.median(vals) if vals else None


def summarize_counters(fetch_dir, write_dir):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the WKV kernels, each scaled by what the
    same counter reads for the 1 GiB device copy of a --with-copy run (the runtime's
    copyBuffer kernel: reads and writes exactly COPY_BYTES)."""
    fetch = _per_dispatch(_read_counter_rows(fetch_dir), "FETCH_SIZE")
    write = _per_dispatch(_read_counter_rows(write_dir), "WRITE_SIZE")
    big = COPY_BYTES / 1024 / 4  # the copy's dispatches, not the runtime's small blits
    copy_f = statistics.median(v for n, vs in fetch.items() if "copyBuffer" in n for v in vs
                               if v > big)
    copy_w = statistics.median(v for n, vs in write.items() if "copyBuffer" in n for v in vs
                               if v > big)
    out = {"source_sha256": source_hash(),
           "copy_kib_expected": COPY_BYTES / 1024,
           "copy_fetch_kib": copy_f, "copy_write_kib": copy_w,
           "fetch_scale": (COPY_BYTES / 1024) / copy_f,
           "write_scale": (COPY_BYTES / 1024) / copy_w,
           "kernels": {}}
    for op, name in KERNELS.items():
        f, w = _match(fetch, name), _match(write, name)
        if f is not None and w is not None:
            out["kernels"][op] = {"fetch_kib": f, "write_kib": w,
                                  "traffic_bytes": 1024 * (f * out["fetch_scale"]
                                                           + w * out["write_scale"])}
    return out


def counter_traffic(op):
    """HBM bytes per launch of `op` from the committed counter summary, or None if absent or
    taken on different kernel sources."""
    try:
        with open(COUNTERS) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_hash():
        return None
    k = rec.get("kernels", {}).get(op)
    return None if k is None else k["traffic_bytes"]


def summarize_trace(folder, warmup, steps):
    """Markdown table of the step's kernel durations from a `rocprofv3 --kernel-trace` folder
    of a bench.py run with the same --warmup and --steps: every dispatch of each kernel, and
    the timed ones alone (the step runs first, so they are dispatches warmup .. warmup+steps-1
    of each of its kernels, in launch order)."""
    rows = []
    for path in glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit("no *kernel_trace.csv under %s" % folder)
    import wkv_inputs
    wl = wkv_inputs.WORKLOADS["l3b"]
    n = wl["B"] * wl["T"] * wl["C"]
    lines = ["| kernel | dispatches | mean us (all) | timed dispatches | mean us (timed) | "
             "min us (timed) | max us (timed) | algorithmic GB/s (timed mean) |",
             "|---|---|---|---|---|---|---|---|"]
    timed_sum = 0.0
    for op, needle in (("forward", KERNELS["forward"]), ("backward", KERNELS["backward"]),
                       ("reduce", REDUCE_KERNEL)):
        d = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
                   if needle in r["Kernel_Name"])
        if not d:
            continue
        us = [(e - s0) / 1e3 for s0, e in d]
        tw = us[warmup:warmup + steps]
        if op != "forward":
            timed_sum += statistics.mean(tw)
        gbs = ("%.0f" % (BYTES_PER_ELEM[op] * n / (statistics.mean(tw) * 1e-6) / 1e9)
               if op in BYTES_PER_ELEM else "-")
        lines.append("| `%s` | %d | %.1f | %d | %.1f | %.1f | %.1f | %s |" % (
            needle, len(us), statistics.mean(us), len(tw), statistics.mean(tw), min(tw),
            max(tw), gbs))
    lines.append("")
    lines.append("backward call (backward kernel + reduce kernel), timed means: %.1f us" % timed_sum)
    return "\n".join(lines)


# ---------------------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the same workload
# ---------------------------------------------------------------------------------------
def cpu_baseline(x, budget_s=10.0, max_runs=3):
    import oracle
    B, T, C = x["k"].shape
    times = []
    t_start = time.perf_counter()
    while len(times) < max_runs:
        t0 = time.perf_counter()
        oracle.forward_recurrent(x["w"], x["u"], x["k"], x["v"])
        oracle.backward_recurrent(x["w"], x["u"], x["k"], x["v"], x["dy"])
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s:
            break
    t = statistics.median(times)
    return {"value": B * T * C / t, "unit": "elem/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "full workload B=%d T=%d C=%d, fp64 plain recurrence forward + linear-time "
                      "backward (OpenMP over b, c), median of %d runs" % (B, T, C, len(times))}


# ---------------------------------------------------------------------------------------
# GPU measurement
# ---------------------------------------------------------------------------------------
def bench_step(wkv, torch, dev, x, steps, warmup):
    t = {n: torch.from_numpy(x[n]).to(dev) for n in ("w", "u", "k", "v", "dy")}
    B, T, C = t["k"].shape
    fws = wkv.forward_workspace(B, T, C, dev)
    bws = torch.empty(max(16, wkv.backward_workspace_size(B, T, C, True)), dtype=torch.uint8,
                      device=dev)
    y = torch.empty_like(t["k"])
    outs = (torch.empty_like(t["k"]), torch.empty_like(t["k"]), torch.empty_like(t["w"]),
            torch.empty_like(t["u"]))

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        wkv.forward(t["w"], t["u"], t["k"], t["v"], workspace=fws, out=y)
        if ev is not None:
            ev[1].record()
        wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"], fwd_workspace=fws, workspace=bws,
                     out=outs)
        if ev is not None:
            ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    span_ms = evs[0][0].elapsed_time(evs[-1][2])
    ok = all(bool(torch.isfinite(a).all()) for a in (y,) + outs)
    return {"B": B, "T": T, "C": C, "fwd_ms": fwd_ms, "bwd_ms": bwd_ms, "span_ms": span_ms,
            "wall_s": wall, "finite": ok}


def bench_copy(torch, dev, reps=3):
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize(dev)
        ms.append(e0.elapsed_time(e1))
    return {"bytes": 2 * COPY_BYTES, "ms": statistics.median(ms),
            "gbps": 2 * COPY_BYTES / (statistics.median(ms) * 1e-3) / 1e9}


def bench_decode(wkv, torch, dev, steps=20, warmup=3, dtype=None):
    import wkv_inputs
    dtype = torch.float32 if dtype is None else dtype
    cfg = wkv_inputs.DECODE
    B, C, L = cfg["B"], cfg["C"], cfg["layers"]
    params = [wkv_inputs.decode_layer_params(l) for l in range(L)]
    w = [torch.from_numpy(pw).to(dev) for pw, _ in params]
    u = [torch.from_numpy(pu).to(dev) for _, pu in params]
    st = [tuple(torch.from_numpy(a).to(dev) for a in wkv_inputs.empty_decode_state(B, C))
          for _ in range(L)]
    y = torch.empty(B, C, dtype=dtype, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1005)
    kv = torch.empty(L, 2, B, C, dtype=dtype, device=dev)

    def calls():
        for l in range(L):
            a, b, p = st[l]
            wkv.decode_step(w[l], u[l], kv[l, 0], kv[l, 1], a, b, p, out=y)

    def timed(run):
        ms = []
        for s in range(warmup + steps):
            kv.normal_(generator=gen)  # the step's tokens, outside the timed region
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize(dev)
            if s >= warmup:
                ms.append(e0.elapsed_time(e1))
        return statistics.median(ms) * 1e3 / L

    # eager: 40 launches from Python per step (host launch cost included where it exceeds
    # the kernels'); graph: the step's 40 calls captured once and replayed, as a serving
    # loop runs them
    eager_us = timed(calls)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream(dev).wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    per_call_us = timed(graph.replay)
    if dtype != torch.float32:  # the 16-bit form: only its graph-replayed rate
        gbps = 30 * B * C / (per_call_us * 1e-6) / 1e9
        return {"us_per_call": per_call_us, "algorithmic_gbps": gbps,
                "frac_of_peak": gbps / PEAK_GBPS, "bytes_per_elem": 30}
    gbps = 36 * B * C / (per_call_us * 1e-6) / 1e9
    return {"workload": "batched decode B=%d C=%d, %d layer states, k, v ~ N(0,1)" % (B, C, L),
            "us_per_call": per_call_us, "elem_per_s": B * C / (per_call_us * 1e-6),
            "algorithmic_gbps": gbps, "frac_of_peak": gbps / PEAK_GBPS,
            "us_per_call_eager": eager_us, "timing": "graph replay of the step's calls",
            "steps": steps, "calls_per_step": L}


def bench_forward_state(wkv, torch, dev, x, steps=100, warmup=100):
    """The forward from a state on the benchmark layer (prompt prefill), back to back as the
    step is timed: each call starts from the state the previous one left (random at first)
    and leaves y and the final state; 12 B per element plus 24 B of state per (b, c). Timed
    for the training entry point (wkv_forward_state, whose workspace serves a backward) and
    for the inference one (wkv_forward_infer, which keeps no states for a backward)."""
    import wkv_inputs
    t = {n: torch.from_numpy(x[n]).to(dev) for n in ("w", "u", "k", "v")}
    B, T, C = t["k"].shape
    st = [torch.from_numpy(a).to(dev) for a in wkv_inputs.random_state(B, C, seed=1006)]
    ws = wkv.forward_workspace(B, T, C, dev)
    y = torch.empty_like(t["k"])

    def timed(call):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize(dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for e0, e1 in evs:
            e0.record()
            call()
            e1.record()
        torch.cuda.synchronize(dev)
        return statistics.mean(e0.elapsed_time(e1) for e0, e1 in evs) * 1e3

    us = timed(lambda: wkv.forward_state(t["w"], t["u"], t["k"], t["v"], *st, workspace=ws,
                                         out=y))
    us_inf = timed(lambda: wkv.forward_infer(t["w"], t["u"], t["k"], t["v"], state=st,
                                             workspace=ws, out=y))
    ok = bool(torch.isfinite(y).all()) and all(bool(torch.isfinite(a).all()) for a in st)
    # its backward (a sequence trained in pieces): the state gradient alone, then with the
    # next piece's cotangent of the final state (a second pass over k, v, dk, dv)
    wkv.forward_state(t["w"], t["u"], t["k"], t["v"], *st, workspace=ws, out=y)
    dy = torch.from_numpy(x["dy"]).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(1007)
    dstate = tuple(torch.randn(B, C, device=dev, generator=g) * 0.1 for _ in range(2))
    bws = torch.empty(max(16, wkv.backward_workspace_size(B, T, C, True)), dtype=torch.uint8,
                      device=dev)
    grads = wkv.backward_state(t["w"], t["u"], t["k"], t["v"], dy, ws, workspace=bws)
    us_b = timed(lambda: wkv.backward_state(t["w"], t["u"], t["k"], t["v"], dy, ws,
                                            workspace=bws, out=grads))
    us_bc = timed(lambda: wkv.backward_state(t["w"], t["u"], t["k"], t["v"], dy, ws,
                                             dstate=dstate, workspace=bws, out=grads))
    ok = ok and all(bool(torch.isfinite(a).all()) for a in grads)
    alg = 12 * B * T * C + 24 * B * C
    gbps = alg / (us * 1e-6) / 1e9
    gbps_inf = alg / (us_inf * 1e-6) / 1e9
    return {"workload": "forward from a state, B=%d T=%d C=%d" % (B, T, C),
            "us": us, "elem_per_s": B * T * C / (us * 1e-6), "algorithmic_gbps": gbps,
            "frac_of_peak": gbps / PEAK_GBPS, "infer_us": us_inf,
            "infer_elem_per_s": B * T * C / (us_inf * 1e-6),
            "infer_frac_of_peak": gbps_inf / PEAK_GBPS, "backward_state_us": us_b,
            "backward_state_cotangent_us": us_bc, "steps": steps, "outputs_finite": ok}


def bench_gated(wkv, torch, dev, x, steps=100, warmup=100):
    """The receptance-gated step on the benchmark layer, back to back: forward_gated
    (k, v, r read, out written: 16 B per element) and backward_gated (k, v, r, dout read;
    dk, dv, dr written: 28 B per element)."""
    t = {n: torch.from_numpy(x[n]).to(dev) for n in ("w", "u", "k", "v", "dy")}
    B, T, C = t["k"].shape
    gen = torch.Generator(device=dev)
    gen.manual_seed(1007)
    r = torch.randn(B, T, C, dtype=torch.float32, device=dev, generator=gen)
    fws = wkv.forward_workspace(B, T, C, dev)
    bws = torch.empty(max(16, wkv.backward_workspace_size(B, T, C, True)), dtype=torch.uint8,
                      device=dev)
    o = torch.empty_like(t["k"])
    outs = (torch.empty_like(t["k"]), torch.empty_like(t["k"]), torch.empty_like(t["k"]),
            torch.empty_like(t["w"]), torch.empty_like(t["u"]))

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        wkv.forward_gated(t["w"], t["u"], t["k"], t["v"], r, workspace=fws, out=o)
        if ev is not None:
            ev[1].record()
        wkv.backward_gated(t["w"], t["u"], t["k"], t["v"], r, t["dy"], fwd_workspace=fws,
                           workspace=bws, out=outs)
        if ev is not None:
            ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize(dev)
    f_us = statistics.mean(e[0].elapsed_time(e[1]) for e in evs) * 1e3
    b_us = statistics.mean(e[1].elapsed_time(e[2]) for e in evs) * 1e3
    n = B * T * C
    ok = all(bool(torch.isfinite(a).all()) for a in (o,) + outs)
    return {"workload": "receptance-gated forward + backward, B=%d T=%d C=%d" % (B, T, C),
            "forward_us": f_us, "backward_us": b_us,
            "elem_per_s": n / ((f_us + b_us) * 1e-6),
            "forward_frac_of_peak": 16 * n / (f_us * 1e-6) / 1e9 / PEAK_GBPS,
            "backward_frac_of_peak": 28 * n / (b_us * 1e-6) / 1e9 / PEAK_GBPS,
            "steps": steps, "outputs_finite": ok}


def bench_bf16(wkv, torch, dev, x, steps=100, warmup=100):
    """The step with k, v, dy, y, dk, dv stored as bfloat16 (state and arithmetic as in fp32),
    back to back: forward 6 B and backward 10 B per element."""
    t = {n: torch.from_numpy(x[n]).to(dev) for n in ("w", "u", "k", "v", "dy")}
    for n in ("k", "v", "dy"):
        t[n] = t[n].to(torch.bfloat16)
    B, T, C = t["k"].shape
    fws = wkv.forward_workspace(B, T, C, dev)
    bws = torch.empty(max(16, wkv.backward_workspace_size(B, T, C, True)), dtype=torch.uint8,
                      device=dev)
    y = torch.empty_like(t["k"])
    outs = (torch.empty_like(t["k"]), torch.empty_like(t["k"]), torch.empty_like(t["w"]),
            torch.empty_like(t["u"]))

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        wkv.forward(t["w"], t["u"], t["k"], t["v"], workspace=fws, out=y)
        if ev is not None:
            ev[1].record()
        wkv.backward(t["w"], t["u"], t["k"], t["v"], t["dy"], fwd_workspace=fws, workspace=bws,
                     out=outs)
        if ev is not None:
            ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize(dev)
    f_us = statistics.mean(e[0].elapsed_time(e[1]) for e in evs) * 1e3
    b_us = statistics.mean(e[1].elapsed_time(e[2]) for e in evs) * 1e3
    n = B * T * C
    ok = all(bool(torch.isfinite(a).all()) for a in (y,) + outs)
    return {"workload": "bfloat16 k, v, dy, y, dk, dv, B=%d T=%d C=%d" % (B, T, C),
            "forward_us": f_us, "backward_us": b_us,
            "elem_per_s": n / ((f_us + b_us) * 1e-6),
            "forward_frac_of_peak": 6 * n / (f_us * 1e-6) / 1e9 / PEAK_GBPS,
            "backward_frac_of_peak": 10 * n / (b_us * 1e-6) / 1e9 / PEAK_GBPS,
            "steps": steps, "outputs_finite": ok}


def bench_shift(wkv, torch, dev, steps=100, warmup=50):
    """The token-shift mix on the benchmark layer's shape, back to back: forward 16 B
    (x read, three mixes written) and backward 20 B per element (three cotangents and x
    read, dx written)."""
    B, T, C = 8, 4096, 2560
    gen = torch.Generator(device=dev)
    gen.manual_seed(1008)
    x = torch.randn(B, T, C, device=dev, generator=gen)
    mu = torch.rand(3, C, device=dev, generator=gen)
    prev = torch.randn(B, C, device=dev, generator=gen)
    dout = [torch.randn(B, T, C, device=dev, generator=gen) for _ in range(3)]
    for _ in range(warmup):
        wkv.token_shift(x, mu, prev)
        wkv.token_shift_backward(x, mu, dout, prev)
    torch.cuda.synchronize(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        e[0].record()
        wkv.token_shift(x, mu, prev)
        e[1].record()
        wkv.token_shift_backward(x, mu, dout, prev)
        e[2].record()
    torch.cuda.synchronize(dev)
    f_us = statistics.mean(e[0].elapsed_time(e[1]) for e in evs) * 1e3
    b_us = statistics.mean(e[1].elapsed_time(e[2]) for e in evs) * 1e3
    n = B * T * C
    return {"workload": "token-shift mix, B=%d T=%d C=%d" % (B, T, C), "forward_us": f_us,
            "backward_us": b_us,
            "forward_frac_of_peak": 16 * n / (f_us * 1e-6) / 1e9 / PEAK_GBPS,
            "backward_frac_of_peak": 20 * n / (b_us * 1e-6) / 1e9 / PEAK_GBPS, "steps": steps}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    ap.add_argument("--no-state", action="store_true",
                    help="skip the forward-from-a-state measurement")
    ap.add_argument("--no-gated", action="store_true",
                    help="skip the receptance-gated measurement")
    ap.add_argument("--no-bf16", action="store_true", help="skip the bfloat16 measurement")
    ap.add_argument("--no-shift", action="store_true", help="skip the token-shift measurement")
    ap.add_argument("--with-copy", action="store_true",
                    help="also time a 1 GiB device copy (scales rocprofv3 byte counters)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="print the step's kernel durations from a rocprofv3 --kernel-trace "
                         "folder of a run with the same --warmup/--steps")
    args = ap.parse_args(argv)

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.warmup, args.steps))
        return
    if args.summarize_counters:
        print(json.dumps(summarize_counters(*args.summarize_counters), indent=1))
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the WKV path here runs on a single device "
              "(--gpus %d, WORLD_SIZE %d requested); run with --gpus 1" % (args.gpus, world),
              file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    sys.path.insert(0, HERE)
    import numpy as np  # noqa: F401
    import torch
    import rwkv_linear_attention_forward_amd as wkv
    import wkv_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    x = wkv_inputs.generate("l3b", with_dy=True)
    r = bench_step(wkv, torch, dev, x, args.steps, args.warmup)
    B, T, C = r["B"], r["T"], r["C"]
    n = B * T * C
    ms_per_step = r["span_ms"] / args.steps
    fwd = statistics.mean(r["fwd_ms"])
    bwd = statistics.mean(r["bwd_ms"])
    op = "backward" if bwd >= fwd else "forward"
    dur_ms = bwd if op == "backward" else fwd
    alg = BYTES_PER_ELEM[op] * n
    achieved = alg / (dur_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": n / (ms_per_step * 1e-3), "unit": "elem/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "3B-class layer WKV forward+backward", "B": B, "T": T, "C": C,
                   "dist": "k,v,dy ~ N(0,1); w = exp(U(-8,2)); u ~ U(-1,1)",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": KERNELS[op], "achieved": achieved,
                     "peak": PEAK_GBPS, "unit": "GB/s", "frac": achieved / PEAK_GBPS,
                     "traffic": counter_traffic(op), "algorithmic_bytes": alg,
                     "mean_launch_us": dur_ms * 1e3},
        "step_gbps": 32 * n / (ms_per_step * 1e-3) / 1e9,
        "kernels_us": {"forward_mean": fwd * 1e3, "forward_min": min(r["fwd_ms"]) * 1e3,
                       "backward_mean": bwd * 1e3, "backward_min": min(r["bwd_ms"]) * 1e3},
        "forward_frac_of_peak": 12 * n / (fwd * 1e-3) / 1e9 / PEAK_GBPS,
        "outputs_finite": r["finite"],
    }
    if args.with_copy:
        out["copy_1gib"] = bench_copy(torch, dev)
    if not args.no_decode:
        out["decode"] = bench_decode(wkv, torch, dev)
        out["decode"]["bf16"] = bench_decode(wkv, torch, dev, dtype=torch.bfloat16)
    if not args.no_state:
        out["forward_state"] = bench_forward_state(wkv, torch, dev, x)
    if not args.no_gated:
        out["gated"] = bench_gated(wkv, torch, dev, x)
    if not args.no_bf16:
        out["bf16"] = bench_bf16(wkv, torch, dev, x)
    if not args.no_shift:
        out["token_shift"] = bench_shift(wkv, torch, dev)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(x)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
