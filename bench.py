#!/usr/bin/env python3
"""Benchmark of the per-token JSD hot path on one MI355X.

One step is the whole JSD forward and backward over one batch, with inputs
resident in HBM and outputs and workspace preallocated: the forward (paired
statistics, merge and divergence) and the closed-form backward with gradients to
both inputs, for a per-token upstream gradient known before the step.  It runs as
one call (vjsd_forward_backward: one launch, each workgroup a row's forward and
then its gradients); the same outputs as two calls (vjsd_forward, then vjsd_bwd)
are timed beside it.  The workload is N=8192 tokens over a V=151936 vocabulary in
bf16 with a per-column Zipf bias (the pages' Qwen2.5-sized vocabulary, B4 x ISL2048
tokens); beta cycles through 0.1, 0.5, 0.9 from step to step.

Printed: one JSON line with tokens/s, ms per step, the roofline of the dominant
kernel (the one-call kernel), measured with HIP events on the stream the kernels
run on, the fp64 CPU oracle's rate on a bounded sample of the same rows, and
per-kernel and sibling-op timings (forward / reverse KL, entropy, top-k
log-probabilities, teacher top-k forward KL, cross-entropy at N=16384, V=128256 in
bf16 and fp16; the beta = 0 / 1 JSD
branches; the distillation-loss form at temperature 2 with a token mean, all tokens
and 3% kept; the one-pass forward at one tensor-parallel rank's shard width).  The HBM traffic figure comes from committed rocprofv3 counters and
is reported only while the kernel sources match the ones profiled.

    python bench.py [--gpus 1] [--steps 30] [--warmup 5]
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

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
# Transcendental results per second: 1024 SIMDs x 2.4 GHz x 8 lanes per cycle.  The
# 157.3 TFLOP/s FP32 vector peak is 32 FMA lanes per SIMD per cycle; v_exp_f32 and
# v_log_f32 issue at a quarter of that rate (a wave64 instruction every 8 cycles,
# measured on MI355X against 2.2 cycles for v_add_f32 / v_fma_f32).
PEAK_TRANS_PER_S = 1024 * 2.4e9 * 8
METRIC = "JSD fwd+bwd tokens/s and HBM GB/s (% peak), N=8192 V=151936 bf16, 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
CSRC = os.path.join(ROOT, "vocab_sharded_softmax_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sources_digest() -> str:
    """Digest of every kernel source, comments and layout left out (the kernel sources
    hold no comment markers inside string literals): committed counters are used only
    while it matches the digest recorded with them."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(CSRC, name), encoding="utf-8") as f:
                code = f.read()
            code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
            code = re.sub(r"//[^\n]*", " ", code)
            h.update(name.encode() + b"\0" + " ".join(code.split()).encode())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-siblings", action="store_true")
    p.add_argument("--no-linear", action="store_true", help="skip the fused-linear row")
    p.add_argument("--linear-only", action="store_true",
                   help="only the fused-linear row, printed as its own JSON line (for profiling)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="wall-clock budget of the oracle sample")
    p.add_argument("--no-extras", action="store_true",
                   help="time the step only (no per-part, branch, shard-width or sibling rows)")
    p.add_argument("--calib-copy", action="store_true",
                   help="only run a streaming 2 GiB device copy (counter calibration for rocprofv3)")
    p.add_argument("--counter-set", action="store_true",
                   help="only run the forward and backward of each counted workload (rocprofv3 --pmc)")
    return p.parse_args()


class Timer:
    """HIP events on torch's current stream, which is the stream the library's
    kernels are enqueued on."""

    def __init__(self, torch):
        self.torch = torch
        self.spans = {}

    def mark(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def add(self, name, a, b):
        self.spans.setdefault(name, []).append((a, b))

    def ms(self, name):
        v = [a.elapsed_time(b) for a, b in self.spans.get(name, [])]
        return sum(v) / len(v) if v else float("nan")

    def spread(self, name):
        v = sorted(a.elapsed_time(b) for a, b in self.spans.get(name, []))
        if not v:
            return None
        mid = len(v) // 2
        med = v[mid] if len(v) % 2 else 0.5 * (v[mid - 1] + v[mid])
        return {"median": round(med, 4), "min": round(v[0], 4), "max": round(v[-1], 4)}


def calib_copy(torch):
    """Three streaming copies of 2 GiB (k_probe_copy): each reads and writes exactly n
    bytes, so the byte counters of a profiled run divided by n give their scale."""
    import vocab_sharded_softmax_amd as vj

    n = 1 << 31  # bytes
    src = torch.empty(n // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        vj.vjsd_membw_probe(src, dst, 1)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n, "launches": 3, "kernel": "k_probe_copy"}))


def ceilings(torch, vj, x, y, out, reps=5):
    """Measured streaming ceilings on this GPU: a read of x and y (two launches) and
    a copy of x into out, with the library's probe kernels."""
    nb = x.numel() * x.element_size()
    res = {}
    for name, fn, moved in (("read", lambda: (vj.vjsd_membw_probe(x, out, 0),
                                              vj.vjsd_membw_probe(y, out, 0)), 2 * nb),
                            ("copy", lambda: vj.vjsd_membw_probe(x, out, 1), 2 * nb)):
        fn()
        tm = Timer(torch)
        for _ in range(reps):
            a = tm.mark()
            fn()
            tm.add("x", a, tm.mark())
        torch.cuda.synchronize()
        res[f"{name}_gbps"] = round(moved / (tm.ms("x") * 1e-3) / 1e9, 1)
    res["bytes_per_launch"] = nb
    return res


def clock_state():
    """Current shader and memory clock levels from sysfs, where readable."""
    import glob

    out = {}
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_[sm]clk")):
        try:
            with open(path) as f:
                cur = [ln.strip() for ln in f if ln.strip().endswith("*")]
        except OSError:
            continue
        key = path.split("/")[-3] + "_" + path.rsplit("_", 1)[-1]
        if cur:
            out[key] = cur[0]
    return out or None


def cpu_baseline(torch, s, t, gout, budget_s):
    """The fp64 oracle (as it stands) on a bounded sample of the timed rows."""
    import numpy as np

    import oracle

    cores = oracle.num_threads()
    chunk = 64
    rows_done, elapsed, r0 = 0, 0.0, 0
    N = s.shape[0]
    while elapsed < budget_s and r0 < N:
        rows = list(range(r0, min(N, r0 + chunk)))
        sc, tc = s[rows].cpu(), t[rows].cpu()
        g = gout[rows].cpu().double().numpy()
        t0 = time.perf_counter()
        oracle.jsd(sc, tc, 0.5, gout=g)
        elapsed += time.perf_counter() - t0
        rows_done += len(rows)
        r0 += chunk
    return {"value": rows_done / elapsed, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"JSD beta=0.5 fwd+bwd (loss and both gradients, fp64) of the first "
                      f"{rows_done} of {N} rows of the same workload, {elapsed:.1f} s"}


_COUNTERS = None


def counters(workload):
    """The committed rocprofv3 counters of a workload's forward and backward (bytes
    fetched and written per step, scaled by the copy calibration; VALU and
    transcendental instructions), or None when the kernel sources changed since they
    were taken."""
    global _COUNTERS
    if _COUNTERS is None:
        _COUNTERS = {}
        if os.path.exists(TRAFFIC_FILE):
            with open(TRAFFIC_FILE) as f:
                rec = json.load(f)
            if rec.get("sources_sha") == sources_digest():
                _COUNTERS = rec.get("workloads", {})
    return _COUNTERS.get(workload)


def traffic_fields(workload, parts, ms, fallback_bytes, fallback_basis, pages_bytes,
                   part_ms=None):
    """HBM rate and fraction of one route's step (parts: ("fwd", "bwd") for the two
    calls, ("fb",) for the one call) on the bytes its kernels move: the counters'
    fetch + write bytes when they match the sources ("bytes_basis": "counters"), else
    fallback_bytes, a lower bound of the route's traffic ("compulsory": one forward and
    one backward read of the inputs and the gradient writes, for the two calls;
    "minimum": one read and the gradient writes, for the one call).  The pages' count
    (three input passes plus the gradient writes) is reported beside as bytes only: held
    steps and register-held rows let it exceed what the kernels fetch, so no fraction is
    quoted on it.
    With counters, the transcendental utilisation of each part: its transcendental
    results per second (time part_ms[part], else ms) against PEAK_TRANS_PER_S."""
    c = counters(workload)
    if c is not None and not all(p in c for p in parts):
        c = None
    if c is not None:
        nbytes, basis = sum(c[p]["bytes"] for p in parts), "counters"
    else:
        nbytes, basis = fallback_bytes, fallback_basis
    gbps = nbytes / (ms * 1e-3) / 1e9
    out = {"bytes_per_step": nbytes, "bytes_basis": basis, "hbm_gbps": round(gbps, 1),
           "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4), "pages_equivalent_bytes": pages_bytes}
    if c is not None:
        pm = part_ms or {}
        out["counter_bytes"] = {p: c[p]["bytes"] for p in parts}
        out["trans_util"] = {
            p: round(c[p]["trans_lane_insts"] / (pm.get(p, ms) * 1e-3) / PEAK_TRANS_PER_S, 4)
            for p in parts}
        out["valu_busy_pct"] = {p: c[p].get("valu_busy_pct") for p in parts}
    return out


# The workloads whose forward and backward the committed counters cover, in the order
# `--counter-set` runs them: name -> (draw arguments, beta, shard widths, student only).
COUNTER_WORKLOADS = {
    "full_vocab": (("full_vocab",), {}, 0.5, None, False),
    "tp8_shard": (("tp8_shard",), {}, 0.5, None, False),
    "tp8_shard_teacher_detached": (("tp8_shard",), {}, 0.5, None, True),
    "robust_fp32_4_shards": (("robust",), {}, 0.5, "robust", False),
    "robust_fp32_1_shard": (("robust",), {}, 0.5, None, False),
    "rank_share_75968": (("full_vocab",), {"N": 1024, "V": 75968}, 0.3, None, True),
    "rank_share_37984": (("full_vocab",), {"N": 1024, "V": 37984}, 0.3, None, True),
}


class Workload:
    """Inputs, outputs and workspace of one JSD workload through the C ABI, preallocated:
    fwd() is vjsd_forward, bwd() vjsd_bwd (both gradients, or the student's alone),
    fb() vjsd_forward_backward (the same outputs in one call)."""

    def __init__(self, torch, vj, synth, name, batch=None):
        draw, kw, self.beta, widths, student_only = COUNTER_WORKLOADS[name]
        self.name = name
        b = batch if batch is not None else synth.draw(*draw, device="cuda", **kw)
        if widths == "robust":
            widths = list(synth.WORKLOADS["robust"].widths)
        self.b = b
        N, V = b.s.shape
        self.N, self.V, self.S = N, V, 1 if widths is None else len(widths)
        self.tensor_bytes = N * V * b.s.element_size()
        self.ngrads = 1 if student_only else 2
        self.part = vj.new_part(N, self.S, "cuda")
        self.stats = torch.empty((N, 4), dtype=torch.float64, device="cuda")
        self.kl = torch.empty((N, 2), dtype=torch.float32, device="cuda")
        self.loss = torch.empty((N,), dtype=torch.float32, device="cuda")
        self.gs = torch.empty_like(b.s)
        self.gt = None if student_only else torch.empty_like(b.t)
        self.sh = vj.ShardSet(b.s, b.t, widths=widths)
        self.shg = vj.ShardSet(b.s, b.t, widths=widths, gs=self.gs, gt=self.gt)
        self.vj = vj

    def fwd(self):
        self.vj.vjsd_forward(self.sh, self.beta, self.part, self.stats, self.kl, self.loss)

    def bwd(self):
        self.vj.vjsd_bwd(self.shg, self.stats, self.kl, self.beta, self.b.gout, self.part)

    def fb(self):
        self.vj.vjsd_forward_backward(self.shg, self.beta, self.b.gout, self.part, self.stats,
                                      self.kl, self.loss)

    def compulsory_bytes(self):
        """One forward read and one backward read of both inputs, and the gradients."""
        return (4 + self.ngrads) * self.tensor_bytes

    def minimum_bytes(self):
        """One read of both inputs and the gradients: the least any route moves."""
        return (2 + self.ngrads) * self.tensor_bytes

    def pages_bytes(self):
        """The pages' count: three input passes over both inputs, and the gradients."""
        return (6 + self.ngrads) * self.tensor_bytes


def counter_set(torch, vj, synth, reps=3):
    """Each of COUNTER_WORKLOADS in turn, for rocprofv3 --pmc runs: a one-page read with
    the bandwidth probe (a marker dispatch that opens the workload's dispatches), then
    1 + reps steps of the forward and the backward as two calls; another marker, then
    1 + reps steps of the one call."""
    marker_src = torch.zeros(1024, dtype=torch.float32, device="cuda")
    marker_dst = torch.zeros(1024, dtype=torch.float32, device="cuda")
    for name in COUNTER_WORKLOADS:
        w = Workload(torch, vj, synth, name)
        torch.cuda.synchronize()
        vj.vjsd_membw_probe(marker_src, marker_dst, 0)
        for _ in range(1 + reps):
            w.fwd()
            w.bwd()
        vj.vjsd_membw_probe(marker_src, marker_dst, 0)
        for _ in range(1 + reps):
            w.fb()
        torch.cuda.synchronize()
        log(f"counter set: {name} ({1 + reps} steps)")
        del w
        torch.cuda.empty_cache()
    print(json.dumps({"counter_set": list(COUNTER_WORKLOADS), "steps": 1 + reps}))


def main():
    args = parse()
    if args.linear_only:
        import torch
        import synth
        import vocab_sharded_softmax_amd as vj
        print(json.dumps(fused_linear_row(torch, vj, synth)), flush=True)
        return
    if args.gpus != 1:
        log(f"bench.py measures one GPU: the op runs on one GPU's vocabulary shards with an "
            f"on-device merge, and no multi-GPU path exists (asked for --gpus {args.gpus}).")
        sys.exit(2)
    import torch

    if args.calib_copy:
        calib_copy(torch)
        return
    if args.counter_set:
        import synth
        import vocab_sharded_softmax_amd as vj
        counter_set(torch, vj, synth)
        return

    import synth
    import vocab_sharded_softmax_amd as vj

    w = synth.WORKLOADS["full_vocab"]
    N, V = w.N, w.V
    log(f"drawing {w.name}: N={N} V={V} bf16")
    b = synth.draw("full_vocab", device="cuda")
    s, t, gout = b.s, b.t, b.gout
    el = s.element_size()
    part = vj.new_part(N, 1, "cuda")
    stats = torch.empty((N, 4), dtype=torch.float64, device="cuda")
    kl = torch.empty((N, 2), dtype=torch.float32, device="cuda")
    loss = torch.empty((N,), dtype=torch.float32, device="cuda")
    gs = torch.empty_like(s)
    gt = torch.empty_like(t)
    sh = vj.ShardSet(s, t)
    shg = vj.ShardSet(s, t, gs=gs, gt=gt)
    timer = Timer(torch)

    def step(beta, rec):
        e0 = timer.mark()
        vj.vjsd_forward_backward(shg, beta, gout, part, stats, kl, loss)
        e1 = timer.mark()
        if rec:
            timer.add("step", e0, e1)
            timer.add(f"step_beta{beta}", e0, e1)

    def two_calls(beta, tm):
        e0 = tm.mark()
        vj.vjsd_forward(sh, beta, part, stats, kl, loss)
        e1 = tm.mark()
        vj.vjsd_bwd(shg, stats, kl, beta, gout, part)
        e2 = tm.mark()
        tm.add("forward", e0, e1)
        tm.add("bwd", e1, e2)
        tm.add("step", e0, e2)

    def three_launch_forward(beta, tm):
        e0 = tm.mark()
        vj.vjsd_stats(sh, 3, part)
        e1 = tm.mark()
        vj.vjsd_merge(part, 1, N, 3, stats)
        e2 = tm.mark()
        vj.vjsd_fwd(sh, stats, beta, part, kl, loss)
        e3 = tm.mark()
        tm.add("stats", e0, e1)
        tm.add("merge", e1, e2)
        tm.add("div", e2, e3)
        tm.add("forward", e0, e3)

    betas = list(w.betas)
    for i in range(args.warmup):
        step(betas[i % 3], False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(betas[i % 3], True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    # the same outputs as two calls, for comparison (not the timed step)
    tm2 = Timer(torch)
    for i in range(2):
        two_calls(betas[i % 3], Timer(torch))
    for i in range(max(args.steps, 3)):
        two_calls(betas[i % 3], tm2)
    torch.cuda.synchronize()

    tensor_bytes = N * V * el
    one_ms = timer.ms("step")  # one launch: the one-call kernel's average duration
    # The roofline's bytes per launch: the pages' count of the step (three input passes
    # and both gradients), unless the counters show fewer bytes moved; without current
    # counters, the least any route moves (one read of the inputs, the gradient writes).
    pages_bytes = 8 * tensor_bytes
    cfv = counters("full_vocab")
    measured = (cfv or {}).get("fb", {}).get("bytes")
    if measured is not None:
        roof_bytes = min(pages_bytes, measured)
        roof_basis = "counters" if measured < pages_bytes else "pages"
    else:
        roof_bytes, roof_basis = 4 * tensor_bytes, "minimum"
    achieved = roof_bytes / (one_ms * 1e-3) / 1e9
    two = {k: round(tm2.ms(k), 4) for k in ("forward", "bwd", "step")}
    # betas that no timed step reached (fewer steps than betas) are left out
    per_beta = {str(bt): round(timer.ms(f"step_beta{bt}"), 4) for bt in betas
                if timer.spans.get(f"step_beta{bt}")}
    log(f"step {ms_step:.3f} ms (events {one_ms:.3f}); two calls {two}")

    three = branches = siblings = tp8 = linear = configs = pages_shape = None
    if not args.no_extras:
        # the same forward as three separate launches (statistics, merge, divergence),
        # timed one by one for comparison with the one-launch forward above
        tm3 = Timer(torch)
        for i in range(2):
            three_launch_forward(betas[i % 3], Timer(torch))
        for i in range(10):
            three_launch_forward(betas[i % 3], tm3)
        torch.cuda.synchronize()
        three = {k: round(tm3.ms(k), 4) for k in ("stats", "merge", "div", "forward")}

        # the KL branches of the same engine on the same data
        branches = {}
        for beta in (0.0, 1.0):
            for _ in range(2):
                step(beta, False)
            tm = Timer(torch)
            for _ in range(5):
                a = tm.mark()
                vj.vjsd_forward(sh, beta, part, stats, kl, loss)
                vj.vjsd_bwd(shg, stats, kl, beta, gout, part)
                tm.add("x", a, tm.mark())
            torch.cuda.synchronize()
            branches[f"jsd_beta{beta:g}_fwd_bwd_ms"] = round(tm.ms("x"), 4)

        # the distillation-loss form: temperature 2, T^2, token mean; all tokens kept,
        # then the few-response-tokens shape of a teacher-cache caller (3% kept)
        loss_rows = {}
        out1 = torch.empty(1, dtype=torch.float32, device="cuda")
        g1 = torch.ones(1, dtype=torch.float32, device="cuda")
        gen = torch.Generator(device="cuda").manual_seed(5)
        for name, frac in (("all_tokens", 1.0), ("3pct_tokens", 0.03)):
            keep = (torch.rand(N, generator=gen, device="cuda") < frac).to(torch.uint8)
            # every token kept is no mask at all (the one call applies); a mask runs the
            # forward and backward launches (one launch would end on the kept rows' tail)
            opts = vj.loss_opts(N, 2.0, True, None if frac == 1.0 else keep, "mean")

            def lstep():
                vj.vjsd_loss_forward(sh, 0.5, opts, part, stats, kl, loss, out1)
                vj.vjsd_loss_backward(shg, 0.5, opts, stats, kl, g1, part)

            def lone():
                vj.vjsd_loss_forward_backward(shg, 0.5, opts, g1, part, stats, kl, loss, out1)
            two_ms, one_ms_ = timed_pair(torch, lstep, lone, 10)
            loss_rows[name] = {"kept": int(keep.sum().item()), "fwd_bwd_ms": round(one_ms_, 4),
                               "two_calls_ms": round(two_ms, 4)}
        branches["jsd_loss_T2_mean"] = loss_rows

        # the same loss through the autograd op (all tokens kept): its gradients in the
        # backward (two calls), and in the forward (one call, then a unit-scale no-op)
        auto = {}
        for gif in (False, True):
            xs = s.detach().clone().requires_grad_()
            xt = t.detach().clone().requires_grad_()

            def astep():
                vj.jsd_loss(xs, xt, 0.5, temperature=2.0, scale_t2=True, reduction="mean",
                            grad_in_forward=gif).backward()
                xs.grad = xt.grad = None
            auto["grad_in_forward" if gif else "grad_in_backward"] = round(
                min(timed(torch, astep, 5), timed(torch, astep, 5)), 4)
            del xs, xt
        branches["jsd_loss_T2_mean_autograd_ms"] = auto

    # streaming read and copy ceilings measured on the same buffers
    ceil = ceilings(torch, vj, s, t, gs)
    fwd_ms, bwd_ms = tm2.ms("forward"), tm2.ms("bwd")
    # the two calls' backward (read s, t; write gs, gt) against the copy ceiling
    ceil["bwd_frac_of_copy"] = round(
        4 * tensor_bytes / (bwd_ms * 1e-3) / 1e9 / ceil["copy_gbps"], 4)
    if cfv is not None:
        # the forward's fetched bytes against the read ceiling; the one call's bytes
        # (about 72 % reads) against the copy ceiling
        ceil["fwd_frac_of_read"] = round(
            cfv["fwd"]["bytes"] / (fwd_ms * 1e-3) / 1e9 / ceil["read_gbps"], 4)
        if measured is not None:
            ceil["one_call_frac_of_copy"] = round(
                measured / (one_ms * 1e-3) / 1e9 / ceil["copy_gbps"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample")
        cpu = cpu_baseline(torch, s, t, gout, args.cpu_seconds)
    del gs, gt, shg, sh, s, t, b
    torch.cuda.empty_cache()

    if not args.no_extras:
        siblings = None if args.no_siblings else sibling_rows(torch, vj, synth)
        tp8 = tp8_forward(torch, vj, synth)
        configs = config_rows(torch, vj, synth)
        pages_shape = {"siblings": pages_shape_siblings(torch, vj, synth),
                       "jsd_rank_share": pages_shape_jsd(torch, vj, synth)}
        linear = None if args.no_linear else fused_linear_row(torch, vj, synth)

    out = {
        "metric": METRIC,
        "value": round(N / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "full_vocab N=8192 V=151936 bf16 logits, Zipf column bias",
                   "global_batch": N, "vocab": V, "storage_dtype": "bf16",
                   "betas": betas, "grads": "student and teacher", "shards": 1},
        **traffic_fields("full_vocab", ("fb",), ms_step, 4 * tensor_bytes, "minimum",
                         pages_bytes),
        "roofline": {"kernel": "k_fwdbwd_twice<BF16, both grads>", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": measured,
                     "bytes_per_launch": roof_bytes, "bytes_basis": roof_basis,
                     "pages_bytes_per_launch": pages_bytes, "avg_launch_ms": round(one_ms, 4)},
        "cpu_baseline": cpu,
        "step_ms_spread": timer.spread("step"),
        "kernel_ms": {"one_call": round(one_ms, 4)},
        "two_calls": {"ms": two, "spread": {k: tm2.spread(k) for k in ("forward", "bwd", "step")},
                      "tokens_per_s": round(N / (two["step"] * 1e-3), 1),
                      **traffic_fields("full_vocab", ("fwd", "bwd"), two["step"],
                                       6 * tensor_bytes, "compulsory", pages_bytes,
                                       part_ms={"fwd": fwd_ms, "bwd": bwd_ms})},
        "ceiling": ceil,
        "clocks": clock_state(),
        "forward_parts_ms": three,
        "tp8_shard": tp8,
        "other_configs": configs,
        "pages_shapes": pages_shape,
        "step_ms_by_beta": per_beta,
        "branches": branches,
        "siblings": siblings,
        "fused_linear": linear,
    }
    print(json.dumps(out), flush=True)


PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def fused_linear_row(torch, vj, synth, reps=3, chunk=1024):
    """The fused-linear loss (hidden states and LM heads -> JSD loss, mean over tokens,
    gradients of the student's hidden states and head) on the linear workload: N=8192,
    V=151936, Ds=Dt=3584 bf16, `chunk` tokens per logit block (the library's default
    plan), with its workspace against what the unfused route holds."""
    log("fused linear")
    b = synth.draw_linear("cuda")
    N, V, Ds = b.hs.shape[0], b.ws.shape[0], b.hs.shape[1]
    Dt = b.ht.shape[1]
    st, te = vj.lin_head(b.hs, b.ws, "student"), vj.lin_head(b.ht, b.wt, "teacher")
    wsb = vj.vljsd_workspace_bytes(N, V, Ds, chunk, 0)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty(1, dtype=torch.float32, device="cuda")
    gh, gw = torch.empty_like(b.hs), torch.empty_like(b.ws)
    opts = vj.loss_opts(N, 1.0, False, None, "mean")
    fn = lambda: vj.vljsd(st, te, N, V, 0.5, opts, chunk, ws, out, gh, gw)
    fn()
    tm = Timer(torch)
    for _ in range(reps):
        a = tm.mark()
        fn()
        tm.add("x", a, tm.mark())
    torch.cuda.synchronize()
    ms = tm.ms("x")
    # the four products: student and teacher logits, hidden and head gradients
    flops = 2 * N * V * (Ds + Dt + 2 * Ds)
    tf = flops / (ms * 1e-3) / 1e12
    res = {"workload": f"linear N={N} V={V} Ds={Ds} Dt={Dt} bf16, chunk {chunk}, beta 0.5, mean",
           "fwd_bwd_ms": round(ms, 4), "tokens_per_s": round(N / (ms * 1e-3), 1),
           "spread": tm.spread("x"),
           "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                        "flops_per_call": flops},
           "workspace_bytes": wsb,
           # what the unfused route holds at once: bf16 logits of both sides and the
           # student's logit gradient, [N, V] each
           "unfused_bytes": 3 * N * V * 2,
           "workspace_frac_of_unfused": round(wsb / (3 * N * V * 2), 4)}
    del ws, gh, gw, b
    torch.cuda.empty_cache()
    return res


def tp8_forward(torch, vj, synth, reps=10):
    """JSD at one tensor-parallel rank's vocabulary shard (N=8192, V=16032 bf16, one
    shard, beta=0.5, both gradients) through the C ABI: the one-pass forward (a row per
    workgroup, held in registers) against the same forward as three launches, the one
    call (forward and backward of a register-held row: one read of the inputs), the
    two calls, and their traffic."""
    w = Workload(torch, vj, synth, "tp8_shard")
    three = lambda: (vj.vjsd_stats(w.sh, 3, w.part), vj.vjsd_merge(w.part, 1, w.N, 3, w.stats),
                     vj.vjsd_fwd(w.sh, w.stats, 0.5, w.part, w.kl, w.loss))
    res = {"one_pass_forward_ms": round(timed(torch, w.fwd, reps), 4),
           "three_launch_forward_ms": round(timed(torch, three, reps), 4)}
    row = workload_row(torch, w, reps)
    res.update({k: row[k] for k in row if k not in ("N", "V", "shards", "fwd_ms")})
    del w
    torch.cuda.empty_cache()
    return res


def timed(torch, fn, reps=10):
    """Mean HIP-event time of fn after two untimed calls."""
    fn()
    fn()
    tm = Timer(torch)
    for _ in range(reps):
        a = tm.mark()
        fn()
        tm.add("x", a, tm.mark())
    torch.cuda.synchronize()
    return tm.ms("x")


def timed_pair(torch, fa, fb, reps=10):
    """Two routes of one computation timed in alternation (a, b, a, b; timed each
    time), each its faster round: neither pays for coming first."""
    ta, tb = [], []
    for _ in range(2):
        ta.append(timed(torch, fa, reps))
        tb.append(timed(torch, fb, reps))
    return min(ta), min(tb)


def workload_row(torch, w, reps=10):
    """The one-call forward and backward of a Workload, with its traffic fields, and the
    same outputs as two calls (forward, backward and their sum) beside it."""
    f_ms = timed(torch, w.fwd, reps)
    b_ms = timed(torch, w.bwd, reps)
    two, one = timed_pair(torch, lambda: (w.fwd(), w.bwd()), w.fb, reps)
    return {"N": w.N, "V": w.V, "shards": w.S, "fwd_bwd_ms": round(one, 4),
            "tokens_per_s": round(w.N / (one * 1e-3), 1),
            **traffic_fields(w.name, ("fb",), one, w.minimum_bytes(), "minimum",
                             w.pages_bytes()),
            "two_calls": {"fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
                          "fwd_bwd_ms": round(two, 4),
                          "tokens_per_s": round(w.N / (two * 1e-3), 1),
                          **traffic_fields(w.name, ("fwd", "bwd"), two, w.compulsory_bytes(),
                                           "compulsory", w.pages_bytes(),
                                           part_ms={"fwd": f_ms, "bwd": b_ms})}}


def config_rows(torch, vj, synth, reps=10):
    """The other configurations of the path, each fwd+bwd through the C ABI with both
    gradients unless stated: the tiny fp32 case (launch-latency bound, no roofline
    meaning), one tensor-parallel rank's width with the teacher detached (student
    gradient only), and the robustness mix (fp32, four column-slice shards of widths
    60000/0/40000/28256 merged on the device, masked columns and rows, offset rows)
    beside the same data as one shard."""
    rows = {}
    b = synth.draw("tiny", device="cuda")
    w = Workload(torch, vj, synth, "full_vocab", batch=b)  # the full_vocab route, tiny data
    w.name = "tiny_fp32"
    r = workload_row(torch, w, reps)
    rows["tiny_fp32"] = {k: r[k] for k in ("N", "V", "fwd_bwd_ms", "tokens_per_s")}
    rows["tiny_fp32"]["two_calls_fwd_bwd_ms"] = r["two_calls"]["fwd_bwd_ms"]
    for name in ("tp8_shard_teacher_detached", "robust_fp32_4_shards", "robust_fp32_1_shard"):
        w = Workload(torch, vj, synth, name)
        rows[name] = workload_row(torch, w, reps)
        del w
        torch.cuda.empty_cache()
    return rows


# The sibling ops' fwd+bwd time and peak memory the pages print for one Intel Arc Pro
# B70 at T=8192, V_local=16032, bf16 ([OPS-PR, Memory]: naive PyTorch -> the eager
# vocabulary-parallel ops), quoted as context beside ours at the same shape.
PAGES_B70_SIBLINGS = {
    "logprobs": {"naive_ms": 7.5, "eager_ms": 21.4, "naive_mib": 1506, "eager_mib": 443},
    "entropy": {"naive_ms": 30.7, "eager_ms": 41.5, "naive_mib": 3012, "eager_mib": 586},
    "reverse_kl": {"naive_ms": 37.2, "eager_ms": 70.2, "naive_mib": 3012, "eager_mib": 698},
    "forward_kl": {"naive_ms": 24.8, "eager_ms": 64.3, "naive_mib": 2510, "eager_mib": 634},
}


def pages_shape_siblings(torch, vj, synth, reps=10):
    """The autograd ops at the shape of the pages' memory table (T=8192, V=16032 bf16,
    one id per token, teacher detached): fwd+bwd ms and the peak device memory of the
    forward and backward beyond the inputs (the student gradient included)."""
    b = synth.draw("tp8_shard", device="cuda")
    N, V = b.s.shape
    gen = torch.Generator(device="cuda").manual_seed(11)
    ids = torch.randint(0, V, (N,), generator=gen, device="cuda")
    t = b.t
    ops = {
        "logprobs": lambda x: vj.logprobs(x, ids),
        "entropy": lambda x: vj.entropy(x),
        "reverse_kl": lambda x: vj.kl_div(x, t, reverse=True),
        "forward_kl": lambda x: vj.kl_div(x, t),
    }
    rows = {}
    for name, fn in ops.items():
        x = b.s.detach().clone().requires_grad_()

        def once():
            fn(x).sum().backward()
            x.grad = None
        once()
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        once()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        tm = Timer(torch)
        for _ in range(reps):
            a = tm.mark()
            once()
            tm.add("x", a, tm.mark())
        torch.cuda.synchronize()
        rows[name] = {"fwd_bwd_ms": round(tm.ms("x"), 4), "peak_mib": round(peak / 2**20, 1),
                      "pages_b70": PAGES_B70_SIBLINGS[name]}
        del x
    return {"shape": f"T={N} V={V} bf16, teacher detached", "ops": rows}


# The pages' JSD fwd+bwd per TP rank at N=1024, global V=151936, bf16, beta=0.3, frozen
# teacher ([JSD-PR, Validation]: median ms with collectives, peak GiB per rank), quoted
# as context beside one rank's share computed here with no exchange.
PAGES_JSD_RANKS = {
    75968: {"tp": 2, "b70_triton_ms": 3.08, "l20_triton_ms": 1.95, "peak_gib_per_rank": 0.435},
    37984: {"tp": 4, "b70_triton_ms": 3.41, "l20_triton_ms": 1.57, "peak_gib_per_rank": 0.217},
}


def pages_shape_jsd(torch, vj, synth, reps=10):
    """One tensor-parallel rank's share of the pages' JSD benchmark: N=1024 and V_local =
    151936 / TP, beta 0.3, student gradient only.  Through the C ABI with preallocated
    buffers (kernel time, with the step's traffic), and through the autograd jsd op
    (which adds the framework's allocations and launches: context for the pages'
    op-level medians), with the op's peak device memory beyond the inputs."""
    rows = {}
    for V, ref in PAGES_JSD_RANKS.items():
        w = Workload(torch, vj, synth, f"rank_share_{V}")
        row = workload_row(torch, w, reps)
        b = w.b
        del w
        t = b.t.detach()
        x = b.s.detach().clone().requires_grad_()

        def once():
            vj.jsd(x, t, 0.3).sum().backward()
            x.grad = None
        once()
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        once()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        tm = Timer(torch)
        for _ in range(reps):
            a = tm.mark()
            once()
            tm.add("x", a, tm.mark())
        torch.cuda.synchronize()
        row.update({"autograd_fwd_bwd_ms": round(tm.ms("x"), 4),
                    "peak_gib_beyond_inputs": round(peak / 2**30, 3), "pages": ref})
        rows[f"V_local={V}"] = row
        del x, b
        torch.cuda.empty_cache()
    return rows


def sibling_rows(torch, vj, synth, reps=3):
    """Forward+backward of the sibling ops at N=16384, V=128256 (teacher detached)."""
    res = {}
    for dtype in (torch.bfloat16, torch.float16):
        name = "bf16" if dtype == torch.bfloat16 else "fp16"
        log(f"siblings {name}")
        b = synth.draw("siblings", device="cuda", dtype=dtype)
        N, V = b.s.shape
        K = b.ids.shape[1]
        tb = N * V * b.s.element_size()
        part = vj.new_part(N, 1, "cuda")
        stats = torch.empty((N, 4), dtype=torch.float64, device="cuda")
        kl = torch.empty((N, 2), dtype=torch.float32, device="cuda")
        loss = torch.empty((N,), dtype=torch.float32, device="cuda")
        out = torch.empty((N, K), dtype=torch.float32, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        gs = torch.empty_like(b.s)
        sh = vj.ShardSet(b.s, b.t)
        shg = vj.ShardSet(b.s, b.t, gs=gs)
        sx = vj.ShardSet(b.s)
        sxg = vj.ShardSet(b.s, gs=gs)
        # the teacher's top-K ids and log-probabilities, as a rollout would hand them over
        tk_lp, tk_ids = torch.log_softmax(b.t.float(), dim=-1).topk(K, dim=-1)
        tk_lp, tk_ids = tk_lp.contiguous(), tk_ids.contiguous()
        ce_lab = b.ids[:, 0].contiguous()  # one label per token, 10% ignore_index
        ce_out = torch.empty(1, dtype=torch.float32, device="cuda")
        one = torch.ones(1, dtype=torch.float32, device="cuda")
        ops = {
            "fwd_kl": (lambda: (vj.vkl_fwd(sh, False, part, stats, kl, loss),
                                vj.vkl_bwd(shg, False, stats, kl, b.gout, part)), 5 * tb),
            "rev_kl": (lambda: (vj.vkl_fwd(sh, True, part, stats, kl, loss),
                                vj.vkl_bwd(shg, True, stats, kl, b.gout, part)), 5 * tb),
            "entropy": (lambda: (vj.ventropy_fwd(sx, part, stats, loss),
                                 vj.ventropy_bwd(sxg, stats, loss, b.gout, part)), 3 * tb),
            "logprobs_top20": (lambda: (vj.vlogprobs_fwd(sx, V, b.ids, -100, part, stats, out, err),
                                        vj.vlogprobs_bwd(sxg, V, stats, b.ids, -100, b.gids, part)),
                               3 * tb),
            "topk_fwd_kl_top20": (lambda: (vj.vtopk_kl_fwd(sx, V, tk_ids, tk_lp, -100, part, stats,
                                                           loss, err),
                                           vj.vtopk_kl_bwd(sxg, V, stats, tk_ids, tk_lp, -100,
                                                           b.gout, part)), 3 * tb),
            "cross_entropy_mean": (lambda: (vj.vce_fwd(sx, V, ce_lab, -100, "mean", part, stats,
                                                       loss, ce_out, err),
                                            vj.vce_bwd(sxg, V, stats, ce_lab, -100, "mean", one,
                                                       part)), 3 * tb),
        }
        for op, (fn, nbytes) in ops.items():
            fn()
            tm = Timer(torch)
            for _ in range(reps):
                a = tm.mark()
                fn()
                tm.add("x", a, tm.mark())
            torch.cuda.synchronize()
            ms = tm.ms("x")
            res[f"{op}_{name}"] = {"fwd_bwd_ms": round(ms, 4),
                                   "tokens_per_s": round(N / (ms * 1e-3), 1),
                                   "bytes_per_step": nbytes, "bytes_basis": "compulsory",
                                   "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
        del b, gs, sh, shg, sx, sxg, tk_lp, tk_ids, ce_lab
        torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
