#!/usr/bin/env python3
"""Throughput of the conv2d input-gradient HIP path on one MI355X (or, with
--op forward, of the forward convolution on the same kernels, or with
--op grad_weight, of the weight gradient; with --op rms_norm_matmul, of the
RMSNorm-fused matrix product of the second page; with --op mha_grad_v, of
the attention dV of the third page).

One step = one conv2d_grad_input call over the whole workload (all batch
items, all stride classes), inputs already resident in HBM.  Before the
warm-up the step runs untimed for 40 ms of GPU time (--clock-warmup-ms), so
that the tuning and the timed steps see the steady shader clock, not its
ramp, and the kernel variant is chosen by measurement (conv2d_tune), outside
the timed region.  Prints one JSON
line with useful TFLOP/s (2*N*Co*out_h*out_w*Ci*kH*kW per second), the
roofline of the kernel (timed with HIP events on the stream it runs on) and
the CPU oracle timed on the host cores on the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--f16 | --fp32] [--no-cpu] [--no-tune] [--clock-warmup-ms MS]
                    [--op grad_input|forward|grad_weight|rms_norm_matmul|mha_grad_v]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "conv2d grad-input useful TFLOP/s per MI355X and % of MFMA peak (fp32, f16)"
METRIC_FORWARD = "conv2d forward useful TFLOP/s per MI355X and % of MFMA peak (fp32, f16)"
METRIC_GRAD_WEIGHT = "conv2d grad-weight useful TFLOP/s per MI355X and % of MFMA peak (fp32)"
METRIC_RMS = "RMSNorm-fused matmul useful TFLOP/s per MI355X and % of MFMA peak (fp32)"
METRIC_MHA = "attention dV useful TFLOP/s per MI355X and % of MFMA peak (fp32)"
# What pct_of_mfma_peak divides: `value` (useful flops over the wall clock of
# the timed steps, launch gaps included) by the dtype's peak.  roofline.frac
# divides useful flops over the GPU time per call of the same steps (one HIP
# event pair around them on the kernel's stream) by the peak.
PCT_BASIS = "value (wall clock of the timed steps) / dtype peak"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6}
PEAK_HBM_GBS = 8000.0
_CSRC = "conv2d_backward_implicit_amd/csrc/"
# the sources each entry point's kernels and launch set-up are built from
KERNEL_SOURCES = {
    "grad_input": [_CSRC + f for f in ("kernels.hip", "tile_index.hpp", "plan.hpp", "plan.cpp",
                                        "pointwise_gemm.hip", "pointwise.hpp")],
    "forward": [_CSRC + f for f in ("kernels.hip", "tile_index.hpp", "plan.hpp", "plan.cpp",
                                     "forward_gemm.hip", "pointwise_gemm.hip", "pointwise.hpp")],
    "grad_weight": [_CSRC + f for f in ("grad_weight.hip", "tile_index.hpp", "plan.hpp")],
    "rms_norm_matmul": [_CSRC + "rms_matmul.hip"],
    "mha_grad_v": [_CSRC + "mha_grad_v.hip"],
}


def _code_only(text: str) -> str:
    """C/C++ source with comments and blank lines removed (string literals in
    these sources hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def source_digest(op: str = "grad_input") -> str:
    """Digest of the code (not the comments) of one entry point's kernel
    sources: a counter summary taken on other code is stale."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[op]:
        with open(os.path.join(ROOT, rel)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel_tag: str, workload: str, op: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (kernel_tag, workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"^source_digest:\s*(\S+)", text, re.M)
    m_val = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_sha or not m_val or m_sha.group(1) != source_digest(op):
        return None
    return float(m_val.group(1))


def cpu_baseline(shape, go, w, op="grad_input"):
    """The oracle as it stands, on the whole workload, on this host's cores
    (``go`` is x for the forward convolution; ``w`` is x for the weight
    gradient)."""
    import numpy as np
    import oracle

    go64 = np.ascontiguousarray(go, dtype=np.float64)
    w64 = np.ascontiguousarray(w, dtype=np.float64)
    orc = oracle.default()
    t0 = time.perf_counter()
    if op == "forward":
        orc.conv2d_forward(go64, w64, shape.out_h, shape.out_w, shape.stride,
                           shape.padding_h, shape.padding_w)
    elif op == "grad_weight":
        orc.grad_weight(go64, w64, shape.kernel_h, shape.kernel_w, shape.stride,
                        shape.padding_h, shape.padding_w)
    else:
        orc.grad_input_gather(go64, w64, shape.in_h, shape.in_w, shape.stride,
                              shape.padding_h, shape.padding_w)
    dt = time.perf_counter() - t0
    return {"value": shape.useful_flops / dt / 1e12, "unit": "TFLOP/s",
            "cores": orc.num_threads(), "kind": "oracle",
            "sample": "whole workload (%d images), one pass, %.2f s" % (shape.batch, dt)}


def copy_calibration(mib: int, steps: int) -> int:
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch
    (KiB) against the true bytes gives the scale for the byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4,
                      "dispatches": steps}), flush=True)
    return 0


def clock_warmup(step, stream, ms: float):
    """Run `step` untimed, in batches of 10, until `ms` milliseconds of GPU
    time have passed on `stream` (at most 5000 steps).  MI355X raises its
    shader clock over the first ~15 ms of sustained matrix work, so a short
    warmup leaves the timed steps partly on the ramp; a training loop runs
    at the steady clock.  The first call (which plans the shape on the host)
    runs before the timed batches.  Returns (steps run, GPU ms)."""
    import torch
    if ms <= 0:
        return 0, 0.0
    step()                    # the first call plans the shape on the host
    torch.cuda.synchronize()
    done, total = 1, 0.0
    while total < ms and done < 5000:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            step()
        e1.record(stream)
        e1.synchronize()
        total += e0.elapsed_time(e1)
        done += 10
    return done, total


def timed_region(step, stream, steps: int):
    """The timed region: `steps` calls of `step` back to back, bracketed by a
    synchronize on each side (wall clock) and by one HIP event pair on
    `stream` (GPU time per call, launch gaps included).  Nothing else is
    recorded between the calls: a timestamp event pair around every call
    slows the calls themselves (on the strided layer 155.0 µs per call with
    a pair per call against 152.3 µs with one pair around 50 calls).
    Returns (wall seconds, GPU seconds per call)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) / steps / 1e3


def per_call_ms(step, stream, calls: int):
    """After the timed region: `calls` calls, each bracketed by its own event
    pair, for the spread of one call's time (sorted, ms)."""
    import torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(calls)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(calls)]
    torch.cuda.synchronize()
    for i in range(calls):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    return sorted(s_.elapsed_time(e_) for s_, e_ in zip(starts, ends))


def cpu_baseline_rms(shape, x, g, w, rows):
    """The oracle on a bounded sample of the workload's rows (every column of
    each), scaled to useful TFLOP/s of those rows."""
    import numpy as np
    import oracle

    orc = oracle.default()
    sel = np.arange(rows, dtype=np.int64) * (shape.m // rows)
    t0 = time.perf_counter()
    orc.rms_norm_matmul(x, g, w, shape.eps, rows=sel)
    dt = time.perf_counter() - t0
    return {"value": 2.0 * rows * shape.k * shape.n / dt / 1e12, "unit": "TFLOP/s",
            "cores": orc.num_threads(), "kind": "oracle",
            "sample": "%d of %d rows (every %d-th), all %d columns, one pass, %.2f s"
                      % (rows, shape.m, shape.m // rows, shape.n, dt)}


def bench_rms(args) -> int:
    """One step = one rms_norm_matmul call over the whole workload."""
    import torch
    import conv2d_backward_implicit_amd as c2b
    from conv2d_backward_implicit_amd.workloads import (RMS_CONFIGS, RMS_HEADLINE, draw_rms,
                                                        rms_by_name)

    if args.f16:
        print("the RMSNorm-fused matmul has an fp32 path only", file=sys.stderr)
        return 2
    shape = rms_by_name(args.workload) if args.workload else RMS_CONFIGS[RMS_HEADLINE]
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    x, g, w = draw_rms(shape, RMS_CONFIGS.index(shape))
    tx, tg, tw = (torch.from_numpy(a).to(dev) for a in (x, g, w))
    out = torch.empty((shape.m, shape.n), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        c2b.rms_norm_matmul_into(out, tx, tg, tw, shape.eps, stream=stream)

    cw_steps, cw_ms = clock_warmup(step, stream, args.clock_warmup_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wall, ev_avg_s = timed_region(step, stream, args.steps)
    ev_ms = per_call_ms(step, stream, min(10, args.steps))
    value = shape.useful_flops * args.steps / wall / 1e12
    achieved = shape.useful_flops / ev_avg_s / 1e12
    peak = PEAK_TFLOPS["f32"]
    out_json = {
        "metric": METRIC_RMS, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "clock_warmup": {"steps": cw_steps, "gpu_ms": round(cw_ms, 1)},
        "ms_per_step": round(wall / args.steps * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": shape.name, "m": shape.m, "k": shape.k, "n": shape.n,
                   "eps": shape.eps, "op": args.op},
        "pct_of_mfma_peak": round(100.0 * value / peak, 2),
        "pct_of_mfma_peak_basis": PCT_BASIS,
        "kernel_avg_us": round(ev_avg_s * 1e6, 3),
        "kernel_median_us": round(ev_ms[len(ev_ms) // 2] * 1e3, 3),
        "compulsory_hbm_GBps": round(shape.compulsory_bytes / ev_avg_s / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic("rms_norm_matmul_f32", shape.name, args.op)},
        "source_digest": source_digest(args.op),
    }
    # a library fp32 product of the same shape (torch's, after an unfused
    # RMSNorm), for context: not the oracle, not the target
    xn = torch.nn.functional.rms_norm(tx, (shape.k,), weight=tg, eps=shape.eps)
    torch.matmul(xn, tw)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        torch.matmul(torch.nn.functional.rms_norm(tx, (shape.k,), weight=tg, eps=shape.eps), tw)
    e1.record(stream)
    torch.cuda.synchronize()
    lib_s = e0.elapsed_time(e1) / 5 / 1e3
    out_json["library_unfused_us"] = round(lib_s * 1e6, 3)
    if not args.no_cpu:
        out_json["cpu_baseline"] = cpu_baseline_rms(shape, x, g, w, min(shape.m, 512))
    print(json.dumps(out_json), flush=True)
    return 0


def mha_lse_torch(q, k, kv_heads, window, causal):
    """The forward's row statistics (max, log sum exp) of the scaled scores
    under the mask, by plain torch on the device: benchmark input, not a
    reference."""
    import torch
    q_seq, heads, d = q.shape
    kv_seq = k.shape[0]
    grp = heads // kv_heads
    pos = torch.arange(q_seq, device=q.device)[:, None]
    t = torch.arange(kv_seq, device=q.device)[None, :]
    vis = torch.ones(q_seq, kv_seq, dtype=torch.bool, device=q.device)
    if causal:
        vis &= t <= pos
    if window > 0:
        vis &= pos < t + window
    lse = torch.zeros(q_seq, heads, 2, device=q.device)
    for h in range(heads):
        sc = (q[:, h, :] @ k[:, h // grp, :].T.contiguous()) / float(d) ** 0.5
        sc = sc.masked_fill(~vis, float("-inf"))
        mx = sc.max(dim=1).values
        mx = torch.where(torch.isfinite(mx), mx, torch.zeros_like(mx))
        lse[:, h, 0] = mx
        lse[:, h, 1] = torch.log(torch.exp(sc - mx[:, None]).sum(dim=1).clamp_min(1e-30))
    return lse


def bench_mha(args) -> int:
    """One step = one mha_grad_v call over the whole sequence and all heads."""
    import numpy as np
    import torch
    import conv2d_backward_implicit_amd as c2b
    from conv2d_backward_implicit_amd.workloads import (MHA_CONFIGS, MHA_HEADLINE, MhaShape,
                                                        draw_mha, mha_by_name)

    if args.f16:
        print("the attention dV kernel has an fp32 path only", file=sys.stderr)
        return 2
    shape = mha_by_name(args.workload) if args.workload else MHA_CONFIGS[MHA_HEADLINE]
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    q, k, g = draw_mha(shape, MHA_CONFIGS.index(shape))
    tq, tk, tg = (torch.from_numpy(a).to(dev) for a in (q, k, g))
    tl = mha_lse_torch(tq, tk, shape.kv_heads, shape.window, shape.causal)
    dv = torch.empty(k.shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        c2b.mha_grad_v_into(dv, tg, tq, tk, tl, shape.window, shape.causal, stream=stream)

    cw_steps, cw_ms = clock_warmup(step, stream, args.clock_warmup_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wall, ev_avg_s = timed_region(step, stream, args.steps)
    ev_ms = per_call_ms(step, stream, min(10, args.steps))
    value = shape.useful_flops * args.steps / wall / 1e12
    achieved = shape.useful_flops / ev_avg_s / 1e12
    peak = PEAK_TFLOPS["f32"]
    out = {
        "metric": METRIC_MHA, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "clock_warmup": {"steps": cw_steps, "gpu_ms": round(cw_ms, 1)},
        "ms_per_step": round(wall / args.steps * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": shape.name, "q_seq": shape.q_seq, "kv_seq": shape.kv_seq,
                   "heads": shape.heads, "kv_heads": shape.kv_heads,
                   "head_dim": shape.head_dim, "window": shape.window,
                   "causal": shape.causal, "op": args.op},
        "pct_of_mfma_peak": round(100.0 * value / peak, 2),
        "pct_of_mfma_peak_basis": PCT_BASIS,
        "kernel_avg_us": round(ev_avg_s * 1e6, 3),
        "kernel_median_us": round(ev_ms[len(ev_ms) // 2] * 1e3, 3),
        "compulsory_hbm_GBps": round(shape.compulsory_bytes / ev_avg_s / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic("mha_grad_v_f32", shape.name, args.op)},
        "source_digest": source_digest(args.op),
    }
    if not args.no_cpu:
        import oracle
        orc = oracle.default()
        sub = MhaShape("prefix", min(shape.q_seq, 512), min(shape.kv_seq, 512), shape.heads,
                       shape.kv_heads, shape.head_dim, shape.window, shape.causal)
        qs, ks, gs = q[:sub.q_seq], k[:sub.kv_seq], g[:sub.q_seq]
        lse = orc.attention_lse(qs, ks, sub.kv_heads, sub.window, sub.causal)
        t1 = time.perf_counter()
        orc.mha_grad_v(gs, qs, ks, lse, sub.window, sub.causal)
        dt = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": sub.useful_flops / dt / 1e12, "unit": "TFLOP/s",
                               "cores": orc.num_threads(), "kind": "oracle",
                               "sample": "the first %d positions and keys of the sequence, "
                                         "all heads, one pass, %.2f s" % (sub.q_seq, dt)}
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--clock-warmup-ms", type=float, default=40.0,
                    help="untimed steps before the warmup steps until this much GPU time "
                         "has passed, so that the timed steps run at the steady shader "
                         "clock (0: none)")
    ap.add_argument("--workload", default=None, help="workload name (default: headline)")
    g = ap.add_mutually_exclusive_group()
    g.add_argument("--f16", action="store_true", help="f16-staged path")
    g.add_argument("--fp32", action="store_true", help="fp32 path")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-tune", action="store_true",
                    help="use the planner's model choice instead of tuning the variant")
    ap.add_argument("--op", choices=("grad_input", "forward", "grad_weight", "rms_norm_matmul",
                                     "mha_grad_v"),
                    default="grad_input",
                    help="the operation timed (default: the input gradient)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead: run --steps plain device-to-device copies of MIB "
                         "MiB (reference kernel for HBM byte counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration, args.steps)

    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each GPU would run its own batch shard with no exchange); "
              "run with --gpus 1", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    if args.op == "rms_norm_matmul":
        return bench_rms(args)
    if args.op == "mha_grad_v":
        return bench_mha(args)

    import numpy as np
    import torch

    import conv2d_backward_implicit_amd as c2b
    from conv2d_backward_implicit_amd.workloads import (CONFIGS, HEADLINE, by_name, draw,
                                                        draw_forward)

    shape = by_name(args.workload) if args.workload else CONFIGS[HEADLINE]
    f16 = shape.f16_staged if not (args.f16 or args.fp32) else args.f16
    if args.op == "grad_weight":
        if args.f16:
            print("the weight gradient has an fp32 path only", file=sys.stderr)
            return 2
        f16 = False
    dtype = "f16" if f16 else "f32"
    seed = CONFIGS.index(shape)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    fwd = args.op == "forward"
    gwt = args.op == "grad_weight"
    p = c2b.make_params(shape.batch, shape.in_channels, shape.in_h, shape.in_w,
                        shape.out_channels, shape.kernel_h, shape.kernel_w, shape.stride,
                        shape.padding_h, shape.padding_w, shape.out_h, shape.out_w)
    stream = torch.cuda.current_stream()
    if gwt:
        # weight gradient: grad_out and x -> grad_weight (go, w and gi below
        # hold grad_out, x and grad_weight); the workspace is allocated once,
        # outside the timed region
        go, _ = draw(shape, seed)
        w, _ = draw_forward(shape, seed + 100)
        tgo = torch.from_numpy(go).to(dev)
        tw = torch.from_numpy(w).to(dev)
        gi = torch.empty(shape.w_shape, dtype=torch.float32, device=dev)
        need = c2b.grad_weight_workspace_size(p)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        plan = {"workspace_bytes": need, "variant": -1, "tuned": False}

        def step():
            c2b.grad_weight_into(gi, tgo, tw, p, workspace=ws, stream=stream)
    else:
        # input gradient: grad_out -> grad_input; forward: x -> y (go and gi
        # below hold x and y)
        go, w = draw_forward(shape, seed) if fwd else draw(shape, seed)
        tgo = torch.from_numpy(go).to(dev)
        tw = torch.from_numpy(w).to(dev)
        gi = torch.empty(shape.go_shape if fwd else shape.gi_shape, dtype=torch.float32,
                         device=dev)
        plan = c2b.describe_forward_plan(p, f16) if fwd else c2b.describe_plan(p, f16)

        def step():
            if fwd:
                c2b.forward_into(gi, tgo, tw, p, f16=f16, stream=stream)
            else:
                c2b.grad_input_into(gi, tgo, tw, p, f16=f16, stream=stream)

        # the clock warm-up first, so that the tuning below times its
        # candidates at the steady clock
        cw_steps, cw_ms = clock_warmup(step, stream, args.clock_warmup_ms)
        # measured variant choice for this shape, once, outside the timed
        # region (conv2d_tune; the default entry point then uses the tuned plan)
        if not args.no_tune:
            variant = (c2b.tune_forward(gi, tgo, tw, p, f16=f16, stream=stream) if fwd else
                       c2b.tune(gi, tgo, tw, p, f16=f16, stream=stream))
        else:
            variant = (c2b.planned_forward_variant(p, f16) if fwd else
                       c2b.planned_variant(p, f16))
        if variant >= 0:   # the plan the timed calls run
            plan = (c2b.describe_forward_plan_variant(p, variant) if fwd else
                    c2b.describe_plan_variant(p, variant))
        plan["variant"] = variant
        plan["tuned"] = not args.no_tune
        if fwd and not f16 and 1 <= shape.in_channels < 16:
            # conv2d_forward takes the im2col GEMM over (ci, kh, kw) for these
            # shapes; the variant above belongs to the other kernel family
            plan = {"path": "forward im2col GEMM (fewer than 16 input channels)",
                    "variant": -1, "tuned": False}

    if gwt:
        cw_steps, cw_ms = clock_warmup(step, stream, args.clock_warmup_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps back to back on the kernel's stream, one HIP
    # event pair around them; then the spread of single calls
    wall, ev_avg_s = timed_region(step, stream, args.steps)
    ev_ms = per_call_ms(step, stream, min(10, args.steps))

    # after the timed region: the same step with the caches flushed before
    # each call (a 512 MiB write, outside the events), since the 256 MiB
    # Infinity Cache can hold every working set of these workloads
    flush = torch.empty(128 << 20, dtype=torch.float32, device=dev)
    nfl = min(10, args.steps)
    fstarts = [torch.cuda.Event(enable_timing=True) for _ in range(nfl)]
    fends = [torch.cuda.Event(enable_timing=True) for _ in range(nfl)]
    for i in range(nfl):
        flush.fill_(float(i))
        fstarts[i].record(stream)
        step()
        fends[i].record(stream)
    torch.cuda.synchronize()
    fl_ms = sorted(s_.elapsed_time(e_) for s_, e_ in zip(fstarts, fends))
    del flush
    ev_sorted = ev_ms

    value = shape.useful_flops * args.steps / wall / 1e12
    achieved = shape.useful_flops / ev_avg_s / 1e12
    kernel_tag = ("forward_%s" if fwd else "grad_weight_%s" if gwt else "grad_input_%s") % dtype
    traffic = measured_traffic(kernel_tag, shape.name, args.op)
    # bound: compare the workload's arithmetic intensity (useful flops per
    # compulsory byte) with the ridge point of the path's matrix peak
    intensity = shape.useful_flops / shape.compulsory_bytes
    ridge = PEAK_TFLOPS[dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    if intensity >= ridge:
        roofline = {"bound": "mfma", "achieved": round(achieved, 3),
                    "peak": PEAK_TFLOPS[dtype], "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_TFLOPS[dtype], 4), "traffic": traffic}
    else:
        gbs = shape.compulsory_bytes / ev_avg_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                    "traffic": traffic}
    out = {
        "metric": METRIC_FORWARD if fwd else METRIC_GRAD_WEIGHT if gwt else METRIC,
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "clock_warmup": {"steps": cw_steps, "gpu_ms": round(cw_ms, 1)},
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic",
        "config": {"workload": shape.name, "batch": shape.batch,
                   "in_channels": shape.in_channels, "out_channels": shape.out_channels,
                   "in_hw": [shape.in_h, shape.in_w], "kernel": [shape.kernel_h, shape.kernel_w],
                   "stride": shape.stride, "padding": [shape.padding_h, shape.padding_w],
                   "out_hw": [shape.out_h, shape.out_w], "path": dtype,
                   "op": args.op},
        "pct_of_mfma_peak": round(100.0 * value / PEAK_TFLOPS[dtype], 2),
        "pct_of_mfma_peak_basis": PCT_BASIS,
        "kernel_avg_us": round(ev_avg_s * 1e6, 3),
        "kernel_median_us": round(ev_sorted[len(ev_sorted) // 2] * 1e3, 3),
        "kernel_min_us": round(ev_sorted[0] * 1e3, 3),
        "flushed_kernel_median_us": round(fl_ms[len(fl_ms) // 2] * 1e3, 3),
        "compulsory_hbm_GBps": round(shape.compulsory_bytes / ev_avg_s / 1e9, 1),
        "plan": plan,
        "roofline": roofline,
        "source_digest": source_digest(args.op),
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(shape, go, w, args.op)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
