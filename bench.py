#!/usr/bin/env python3
"""Benchmark: shape-specialised bf16 projections on one MI355X.

One step = one decode pass of the 27B-like decoder layer at M = 1 -- the largest
single-GPU workload: QKV 5120->10240, out 8192->5120, gate/up 5120->34816, down
17408->5120, weights bf16 ~N(0, 0.01) with 1 % outliers x10, activations bf16
~N(0, 1), Y bf16 -- four proj_run calls through the C ABI on tuned plans.
Weights are resident in HBM before timing and rotate over copies of at least
2 GiB in total, so no step finds them in the 256 MB last-level cache: a decode
step re-reads every weight ("#001 un compilateur pour moteur de LLM", section
"Ce que coute un token").

Reported (one JSON line on stdout; progress on stderr):
  value        decode HBM GB/s of the step = its algorithmic bytes (W once, X
               once, Y once per projection) / step time, over exactly --steps
               timed steps after a device warm-up and --warmup untimed steps
  roofline     the step's dominant kernel (the gate/up GEMV): algorithmic bytes
               per launch / mean launch time (HIP events on the launch stream,
               back-to-back launches with rotating weights), against 8 TB/s;
               traffic from the committed rocprofv3 counter runs
  per_shape    every M = 1 projection of the step alone: GB/s (mean over
               back-to-back launches) and median / p10 / p90 of single
               launches (an event pair each); launch_bound marks shapes whose
               ideal time at 8 TB/s is under 5 us
  graph        the same step recorded as a HIP graph and replayed
  host_call_us the host time of one proj_run call through the binding
  prefill_27b_m8192  the same layer at M = 8192: TFLOP/s per projection and
               for the layer, against 2.5 PFLOP/s and against
               256 CUs x 4096 flop/clk x the engine clock each kernel ran at,
               read inside a probe copy of it (clock_probe)
               (roofline_prefill: its dominant GEMM)
  decode_08b   the 0.8B-like layer plus its 151936-row head at M = 1 (f32 Y):
               the same figures, and the step replayed as a HIP graph
  prefill_4b   the 4B-like layer at M = 128, 512, 2048 (bf16 Y), rotating weights
  long_prompt  8192 rows through the 4B-like layer in blocks of 1024 (a weight
               copy per block), then the 151936 x 2560 head on the last row
  swiglu_epilogue, rmsnorm_prologue, packed_weights  the fused epilogue /
               prologue and the packed layout against their unfused / row-major
               forms (skipped with --no-extra)
  clocks       sclk and mclk before and after (board level)
  probe        HBM read-probe bandwidth (the pages' measured denominator)
  cpu_baseline the fp64 CPU oracle on the same decode step (bounded sample, all
               host cores up to 16), with a 64-row prefill sample of the M = 8192
               layer scaled to the full layer (labelled extrapolated) and a
               single-core rate
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0     # MI355X dense bf16 MFMA (256 CUs x 4096 flop/clk x 2.4 GHz)
CUS, FLOP_PER_CLK_PER_CU = 256, 4096
ROTATE_BYTES = 2 << 30          # weights rotate over at least this many bytes (8x the 256 MB last-level cache)
WARM_MS = 30.0                  # device time of warm-up before each kernel measurement
DEVICE_WARM_MS = 60.0           # device time of warm-up before the timed decode steps


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def upload(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _stream_handle():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


_WEIGHTS = {}


def weights(cfg, i):
    """synth.weights, drawn once per process (the 27B-like layer takes seconds)."""
    import synth
    key = (cfg.name, i)
    if key not in _WEIGHTS:
        _WEIGHTS[key] = synth.weights(cfg, i)
    return _WEIGHTS[key]


def copies_for(nbytes: int, minimum: int = 2) -> int:
    return max(minimum, -(-ROTATE_BYTES // max(1, nbytes)))


def rotation(W, nbytes=None):
    """W and clones of it, at least ROTATE_BYTES in total."""
    n = copies_for(nbytes or W.numel() * W.element_size())
    return [W] + [W.clone() for _ in range(n - 1)]


# ---------------------------------------------------------------- timing
def events_us(fn, n):
    """Mean device time (us) per call of the enqueue-only closure fn(s), s = 0..n-1:
    one event pair on torch's current stream around all n calls."""
    import torch
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for s in range(n):
        fn(s)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def per_call_us(fn, n):
    """Device time (us) of each of n calls, an event pair around each."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for s in range(n):
        ev[s][0].record(stream)
        fn(s)
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, int(q * (len(v) - 1) + 0.5))]


def dist(v):
    return dict(median=round(statistics.median(v), 3), p10=round(pct(v, 0.1), 3), p90=round(pct(v, 0.9), 3))


def warm(fn, warm_ms: float = WARM_MS):
    """Run fn for at least warm_ms of device time.  After an idle gap the device
    needs ~15 ms of work to reach its steady clocks: a 4B-like gate/up GEMM at
    M = 2048 measured 196-206 us per launch over its first ~80 launches after a
    3 s pause, then 172-175 us for as long as it kept running."""
    est = events_us(fn, 2)
    k = int(warm_ms * 1e3 / max(est, 1.0)) + 1
    return events_us(fn, k) * k / 1e3


def steady(fn, n, rounds: int = 5):
    """Steady-state device time (us) per call: warm-up, then `rounds` rounds of
    n calls, one event pair each; median and p10 / p90 of the rounds."""
    warm(fn)
    r = [events_us(fn, n) for _ in range(rounds)]
    return statistics.median(r), r


# ---------------------------------------------------------------- clocks
def _sysfs(name):
    """The current DPM level's frequency (MHz) from sysfs (the level marked *)."""
    for f in sorted(glob.glob(f"/sys/class/drm/card*/device/{name}")):
        try:
            for line in open(f):
                if line.rstrip().endswith("*"):
                    return int(line.split(":")[1].strip().split("M")[0].rstrip("hzHZ *"))
        except (OSError, ValueError, IndexError):
            continue
    return None


def _hwmon(name):
    for f in sorted(glob.glob(f"/sys/class/drm/card*/device/hwmon/hwmon*/{name}")):
        try:
            return int(open(f).read().strip())
        except (OSError, ValueError):
            continue
    return None


def _gfx_clocks():
    """The graphics clock of each XCD (MHz) as amd-smi reports it (the actual
    clock, unlike the DPM level in sysfs); [] if amd-smi is not there."""
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "--clock"], capture_output=True, text=True, timeout=10)
    except (OSError, subprocess.TimeoutExpired):
        return []
    return [int(v) for v in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", r.stdout)]


def clocks():
    g = _gfx_clocks()
    p = _hwmon("power1_input")
    return dict(sclk_dpm_mhz=_sysfs("pp_dpm_sclk"), mclk_mhz=_sysfs("pp_dpm_mclk"),
                gfx_clk_mhz=round(statistics.mean(g), 1) if g else None,
                power_w=round(p / 1e6, 1) if p else None, temp_c=[(_hwmon(f"temp{i}_input") or 0) / 1e3 for i in (2, 3)])


def mfma_peak_at(mhz):
    return CUS * FLOP_PER_CLK_PER_CU * mhz * 1e6 / 1e12 if mhz else None


# ---------------------------------------------------------------- plans
class Plans:
    """Tuned plans shared by every leg (one per shape, output type and options)."""

    def __init__(self):
        self.d = {}
        self.created = []   # plan creation (emit, compile, validate, tune), outside every timed region

    def get(self, N, K, dtype, **kw):
        from shape_specialised_bf16_amd import Plan
        key = (N, K, dtype, tuple(sorted(kw.items())))
        if key not in self.d:
            t0 = time.time()
            self.d[key] = Plan(N, K, dtype, **kw)
            d = self.d[key].describe()
            log(f"  plan {N}x{K} {dtype} {kw or ''}: {time.time() - t0:.1f} s "
                f"(compile {d['compile_s']:.1f} s in {d['modules']} modules, tune {d['tune_s']:.1f} s)")
            self.created.append(dict(shape=f"{N}x{K}", dtype=dtype, options=dict(kw) or None,
                                     wall_s=round(time.time() - t0, 2), compile_s=round(d["compile_s"], 2),
                                     tune_s=round(d["tune_s"], 2), modules=d["modules"],
                                     code_cache=d.get("code_cache"), tuning_cache=d.get("cache")))
        return self.d[key]

    def close(self):
        for p in self.d.values():
            p.close()
        self.d.clear()


def _check_rows(Y, X, W, rows, dtype, label):
    """Sampled rows of a timed output against the oracle (tolerance of its dtype)."""
    import numpy as np
    import torch

    import oracle
    from oracle import tolerance
    ref = oracle.matmul_rows(X, rows, W)
    got = Y[rows].cpu()
    if dtype == "bf16":
        rep = tolerance.check_bf16(got.view(torch.int16).numpy().view(np.uint16), ref)
    else:
        rep = tolerance.check_f32(got.numpy(), ref)
    if not rep.ok:
        raise SystemExit(f"bench: {label} does not match the oracle: {rep}")


# ---------------------------------------------------------------- decode (M = 1)
def decode_layer(plans, wl: str, dtype: str, steps: int, warmup: int, graph: bool = False):
    """One M = 1 step of workload `wl` (every projection, rotating weight
    copies): the timed steps, per-step and per-shape distributions, the
    dominant kernel's launch time, optionally the step replayed as a HIP graph;
    every output checked against the oracle."""
    import torch

    import oracle
    import synth
    from oracle import tolerance

    cfg = synth.workload(wl)
    projs = cfg.projections
    ysz = 2 if dtype == "bf16" else 4
    pl = [plans.get(p.N, p.K, dtype) for p in projs]
    host = [(synth.activations(cfg, i, 1), weights(cfg, i)) for i in range(len(projs))]
    Xs = [upload(x) for x, _ in host]
    Ws = [upload(w) for _, w in host]
    Ys = [torch.empty((1, p.N), dtype=pl[i].out_dtype, device="cuda") for i, p in enumerate(projs)]
    layer_w = sum(w.numel() * 2 for w in Ws)
    ncp = copies_for(layer_w)
    Wrot = [[w] + [w.clone() for _ in range(ncp - 1)] for w in Ws]
    wptr = [[w.data_ptr() for w in r] for r in Wrot]
    xptr, yptr = [x.data_ptr() for x in Xs], [y.data_ptr() for y in Ys]
    sh = _stream_handle()
    bytes_of = [2 * p.N * p.K + 2 * p.K + ysz * p.N for p in projs]
    step_bytes = sum(bytes_of)

    def step(s, h=sh):
        c = s % ncp
        for i in range(len(projs)):
            pl[i].run_ptr(xptr[i], wptr[i][c], yptr[i], 1, h)

    warm_ms = warm(step, DEVICE_WARM_MS)
    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    # the timed region: exactly `steps` steps, nothing but the proj_run calls
    t_us = events_us(step, steps)
    ms_per_step = t_us / 1e3
    # diagnostics, untimed: per-step distribution, per-shape times
    step_us = per_call_us(step, max(200, steps))
    per = []
    for i, p in enumerate(projs):
        def one(s, i=i):
            pl[i].run_ptr(xptr[i], wptr[i][s % ncp], yptr[i], 1, sh)
        warm(one, 10.0)
        b2b = statistics.median(events_us(one, 200) for _ in range(3))
        single = per_call_us(one, 300)
        ideal = bytes_of[i] / HBM_PEAK_GBS / 1e3      # us at 8 TB/s
        per.append(dict(proj=p.name, N=p.N, K=p.K, kernel=pl[i].choice(1), bytes=bytes_of[i],
                        ideal_us=round(ideal, 2), launch_bound=ideal < 5.0,
                        mean_launch_us=round(b2b, 3), GBps=round(bytes_of[i] / b2b / 1e3, 1),
                        pct_peak=round(100 * bytes_of[i] / b2b / 1e3 / HBM_PEAK_GBS, 1),
                        single_launch_us=dist(single),
                        single_launch_GBps_median=round(bytes_of[i] / statistics.median(single) / 1e3, 1)))
    # host cost of one proj_run call through the Python binding (argument
    # checks, bucket lookup, the enqueue of its kernel): 200 calls, not waited for
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(200):
        pl[0].run_ptr(xptr[0], wptr[0][0], yptr[0], 1, sh)
    host_us = (time.perf_counter() - t0) * 1e6 / 200
    torch.cuda.synchronize()
    out = dict(step_us=t_us, step_bytes=step_bytes, weight_copies_rotated=ncp, device_warmup_ms=round(warm_ms, 1),
               step_dist_us=dist(step_us), per_shape=per, host_call_us=round(host_us, 2))
    if graph:
        # the same steps recorded by stream capture as one HIP graph per
        # rotation of the weight copies, replayed
        gs = torch.cuda.Stream()
        gh = ctypes.c_void_p(gs.cuda_stream)
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.stream(gs):
            with torch.cuda.graph(g, stream=gs):
                for c in range(ncp):
                    step(c, gh)
        torch.cuda.synchronize()
        warm(lambda s: g.replay(), 10.0)
        n_rep = max(1, 400 // ncp)
        eager = statistics.median(events_us(step, n_rep * ncp) for _ in range(3))
        replay = statistics.median(events_us(lambda s: g.replay(), n_rep) for _ in range(3)) / ncp
        for Y in Ys:
            Y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, ((X, W), Y) in enumerate(zip(host, Ys)):
            _check_rows(Y, X, W, [0], dtype, f"graph replay {projs[i].name}")
        out["graph"] = dict(eager_step_us=round(eager, 3), replayed_step_us=round(replay, 3),
                            eager_GBps=round(step_bytes / eager / 1e3, 1),
                            replayed_GBps=round(step_bytes / replay / 1e3, 1),
                            launch=f"one HIP graph recording {ncp} steps (a rotation of the weight copies)")
        del g
    # the timed path's own outputs, every element, against the oracle
    step(0)
    torch.cuda.synchronize()
    for i, ((X, W), Y) in enumerate(zip(host, Ys)):
        ref = oracle.matmul(X, W, threads=min(16, os.cpu_count() or 1))
        import numpy as np
        got = Y.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else Y.cpu().numpy()
        rep = tolerance.check_bf16(got, ref) if dtype == "bf16" else tolerance.check_f32(got, ref)
        if not rep.ok:
            raise SystemExit(f"bench: {wl} {projs[i].name} does not match the oracle: {rep}")
    out["host"] = host
    del Wrot
    return out


# ---------------------------------------------------------------- prefill
def kernel_clock(N, K, name, X, Wrot, Y, M):
    """The engine clock the tuned GEMM `name` runs at under its own load, read
    inside a probe copy of it (shape_specialised_bf16_amd.clock_probe); None for
    candidates the probe does not cover (split-K, split tail) or if it fails."""
    import subprocess

    from shape_specialised_bf16_amd import clock_probe
    try:
        r = clock_probe.measure(N, K, "bf16", name, X, Wrot, Y, M, launches=20, warm_s=0.1)
    except (RuntimeError, ValueError, OSError, subprocess.SubprocessError) as e:
        log(f"  clock probe of {name} at M={M}: {e}")
        return None
    if r:
        log(f"  clock probe {name} {N}x{K} M={M}: {r['mhz_weighted']} MHz (workgroups p10 {r['mhz_p10']}, "
            f"p90 {r['mhz_p90']}); probe copy {r['probe_tflops']} TFLOP/s")
    return r


def prefill_layer(plans, wl: str, Ms, rounds: int = 5, clock_from: int = 512):
    """Each projection of workload `wl` at each M (bf16 Y, weights rotating over
    >= 2 GiB of copies: a prompt block meets every weight after the other
    layers' weights have gone through the cache), steady state, sampled rows
    checked against the oracle.  From M = `clock_from` rows (MFMA-bound) also
    the engine clock each projection's kernel runs at and its fraction of the
    dense peak at that clock."""
    import torch

    import synth

    cfg = synth.workload(wl)
    out = {}
    sh = _stream_handle()
    for M in Ms:
        per, flops = [], 0.0
        for i, p in enumerate(cfg.projections):
            plan = plans.get(p.N, p.K, "bf16")
            wh, xh = weights(cfg, i), synth.activations(cfg, i, M)
            Wrot = rotation(upload(wh))
            X = upload(xh)
            Y = torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda")
            ncp = len(Wrot)
            wps, xp, yp = [w.data_ptr() for w in Wrot], X.data_ptr(), Y.data_ptr()
            n = max(ncp, min(200, int(20000 / max(1.0, 2.0 * M * p.N * p.K / 1e12 * 1e6 / 1000))))
            med, rs = steady(lambda s: plan.run_ptr(xp, wps[s % ncp], yp, M, sh), n, rounds)
            _check_rows(Y, xh, wh, sorted({0, M // 2, M - 1}), "bf16", f"{wl} {p.name} M={M}")
            f = 2.0 * M * p.N * p.K
            flops += f
            per.append(dict(proj=p.name, N=p.N, K=p.K, kernel=plan.choice(M), us=round(med, 2),
                            tflops=round(f / med / 1e6, 1), pct_peak=round(100 * f / med / 1e6 / MFMA_BF16_PEAK_TFS, 1),
                            rounds_us=dict(p10=round(pct(rs, 0.1), 2), p90=round(pct(rs, 0.9), 2)),
                            weight_copies_rotated=ncp))
            if M >= clock_from:
                kc = kernel_clock(p.N, p.K, plan.choice(M), X, Wrot, Y, M)
                if kc:
                    pk = mfma_peak_at(kc["mhz_weighted"])
                    per[-1]["kernel_clock"] = {k: kc[k] for k in ("mhz_weighted", "mhz_p10", "mhz_p90", "probe_tflops")}
                    per[-1]["peak_at_kernel_clock"] = round(pk, 1)
                    per[-1]["frac_at_kernel_clock"] = round(f / med / 1e6 / pk, 4)
            del Wrot, X, Y
        tot = sum(x["us"] for x in per)
        dom = max(per, key=lambda x: x["us"])
        out[f"M{M}"] = dict(value=round(flops / tot / 1e6, 1), unit="TFLOP/s", layer_us=round(tot, 2),
                            pct_peak=round(100 * flops / tot / 1e6 / MFMA_BF16_PEAK_TFS, 1), projections=per,
                            dominant=dict(kernel=dom["kernel"], shape=f"{dom['N']}x{dom['K']}", us=dom["us"],
                                          tflops=dom["tflops"]))
        if "peak_at_kernel_clock" in dom:
            out[f"M{M}"]["dominant"].update(kernel_clock=dom["kernel_clock"], peak_at_kernel_clock=dom["peak_at_kernel_clock"],
                                            frac_at_kernel_clock=dom["frac_at_kernel_clock"])
        if all("peak_at_kernel_clock" in x for x in per):
            # the layer's flops over what the dense peak at each kernel's own clock would do in the same time
            cap = sum(x["peak_at_kernel_clock"] * 1e6 * x["us"] for x in per)
            out[f"M{M}"]["pct_peak_at_kernel_clocks"] = round(100 * flops / cap, 1)
        log(f"  {wl} M={M}: {out[f'M{M}']['value']} TFLOP/s over the layer ({tot:.1f} us); "
            + ", ".join(f"{x['proj']} {x['tflops']}" for x in per))
        torch.cuda.empty_cache()
    return out


def roofline_prefill(leg, M):
    """Roofline of a prefill leg's dominant kernel at M: MFMA-bound above the
    ridge point (2.5 PFLOP/s / 8 TB/s = 312.5 flop/B), HBM-bound below."""
    dom = leg[f"M{M}"]["dominant"]
    N, K = map(int, dom["shape"].split("x"))
    nbytes = 2 * (M * K + N * K + M * N)
    fl = 2.0 * M * N * K
    ridge = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if fl / nbytes < ridge:
        gbs = nbytes / dom["us"] / 1e3
        r = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4),
                 tflops=dom["tflops"])
    else:
        r = dict(bound="mfma", achieved=dom["tflops"], peak=MFMA_BF16_PEAK_TFS, unit="TFLOP/s",
                 frac=round(dom["tflops"] / MFMA_BF16_PEAK_TFS, 4))
        if "peak_at_kernel_clock" in dom:
            # the dense peak at the clock this kernel ran at (read inside it)
            r.update(kernel_clock_mhz=dom["kernel_clock"]["mhz_weighted"], peak_at_kernel_clock=dom["peak_at_kernel_clock"],
                     frac_at_kernel_clock=dom["frac_at_kernel_clock"])
    r.update(kernel=dom["kernel"], shape=dom["shape"], M=M, mean_launch_us=dom["us"], algorithmic_bytes=nbytes,
             flop_per_byte=round(fl / nbytes, 1), traffic=traffic_for(f"{dom['kernel']}@{dom['shape']}m{M}"))
    cnt = counters_for(f"{dom['kernel']}@{dom['shape']}m{M}")
    if cnt and r["bound"] == "mfma":
        r.update(counters=cnt)   # the committed counter run of this kernel (profiles/counters.json)
    return r


def long_prompt(plans, rounds: int = 5):
    """The caller-side prompt-block driver: 8192 rows through each 4B-like
    projection as 8 blocks of 1024 (block-major: every projection of block b,
    then block b+1; block b reads weight copy b), then the 151936 x 2560 head on
    the last row only."""
    import torch

    import synth

    cfg = synth.workload("long_prompt_4b_8192x1024")
    rows, block = cfg.extra["prompt_rows"], cfg.extra["block"]
    nb = rows // block
    layer = [p for p in cfg.projections if p.name != "head"]
    head = [p for p in cfg.projections if p.name == "head"][0]
    hi = cfg.projections.index(head)
    pl = [plans.get(p.N, p.K, "bf16") for p in layer]
    hplan = plans.get(head.N, head.K, "f32")
    host = [(synth.activations(cfg, i, rows), weights(cfg, i)) for i in range(len(layer))]
    Xs = [upload(x) for x, _ in host]
    layer_bytes = sum(2 * p.N * p.K for p in layer)
    ncp = max(nb, copies_for(layer_bytes))
    Wrot = [[W] + [W.clone() for _ in range(ncp - 1)] for W in (upload(w) for _, w in host)]
    Ys = [torch.empty((rows, p.N), dtype=torch.bfloat16, device="cuda") for p in layer]
    hx, hw = synth.activations(cfg, hi, 1), weights(cfg, hi)
    HX, HW = upload(hx), upload(hw)
    logits = torch.empty((1, head.N), dtype=torch.float32, device="cuda")
    sh = _stream_handle()
    wps = [[w.data_ptr() for w in r] for r in Wrot]

    def prompt(s):
        for b in range(nb):
            c = (s * nb + b) % ncp
            for i, p in enumerate(layer):
                pl[i].run_ptr(Xs[i].data_ptr() + b * block * p.K * 2, wps[i][c], Ys[i].data_ptr() + b * block * p.N * 2,
                              block, sh)
        hplan.run_ptr(HX.data_ptr(), HW.data_ptr(), logits.data_ptr(), 1, sh)

    med, rs = steady(prompt, 2, rounds)
    for i, p in enumerate(layer):
        _check_rows(Ys[i], *host[i], [0, block - 1, block, rows - 1], "bf16", f"long prompt {p.name}")
    _check_rows(logits, hx, hw, [0], "f32", "long prompt head")
    flops = 2.0 * rows * sum(p.N * p.K for p in layer) + 2.0 * head.N * head.K
    out = dict(workload=f"long_prompt_4b: {rows} rows as {nb} blocks of {block} through QKV 2560->5120, out "
                        "4096->2560, gate/up 2560->18432, down 9216->2560 (bf16 Y), then the head 2560->151936 on the "
                        "last row (f32 Y)",
               value=round(flops / med / 1e6, 1), unit="TFLOP/s", prompt_us=round(med, 1),
               rounds_us=dict(p10=round(pct(rs, 0.1), 1), p90=round(pct(rs, 0.9), 1)),
               pct_peak=round(100 * flops / med / 1e6 / MFMA_BF16_PEAK_TFS, 1), weight_copies_rotated=ncp,
               kernels={p.name: pl[i].choice(block) for i, p in enumerate(layer)} | {"head": hplan.choice(1)})
    log(f"  long prompt: {out['value']} TFLOP/s ({med:.0f} us per 8192-row prompt)")
    del Wrot
    return out


# ---------------------------------------------------------------- fusions and layout
def swiglu_leg(plans, steps: int = 500):
    """The SwiGLU epilogue folded into the gate_up projection against the
    unfused path (the plain plan, then proj_swiglu on its N-column output):
    the 0.8B-like gate/up at M = 1 (f32) and the 4B-like gate/up at M = 2048
    (bf16), both on rotating weight copies."""
    import numpy as np
    import torch

    import oracle
    import shape_specialised_bf16_amd as ssb
    import synth
    from oracle import tolerance

    sh = _stream_handle()
    out = {}
    for key, wl, M, dt in (("decode_gate_up_08b_m1", "decode_0.8b_layer_m1", 1, "f32"),
                           ("prefill_gate_up_4b_m2048", "prefill_4b_layer", 2048, "bf16")):
        cfg = synth.workload(wl)
        pi = [p.name for p in cfg.projections].index("gate_up")
        p = cfg.projections[pi]
        fused = plans.get(p.N, p.K, dt, epilogue="swiglu")
        plain = plans.get(p.N, p.K, dt)
        Wh, Xh = weights(cfg, pi), synth.activations(cfg, pi, M)
        Wrot, X = rotation(upload(Wh)), upload(Xh)
        ncp = len(Wrot)
        odt = torch.bfloat16 if dt == "bf16" else torch.float32
        Gb = torch.empty((M, p.N), dtype=odt, device="cuda")
        Hu = torch.empty((M, p.N // 2), dtype=odt, device="cuda")
        Hf = torch.empty((M, p.N // 2), dtype=odt, device="cuda")
        xp, wps, gp, hup, hfp = X.data_ptr(), [w.data_ptr() for w in Wrot], Gb.data_ptr(), Hu.data_ptr(), Hf.data_ptr()
        swiglu_c, code = ssb._lib.proj_swiglu, (1 if dt == "bf16" else 0)

        def unfused(s):
            plain.run_ptr(xp, wps[s % ncp], gp, M, sh)
            swiglu_c(gp, hup, M, p.N, code, sh)

        def fused_(s):
            fused.run_ptr(xp, wps[s % ncp], hfp, M, sh)

        n = steps if M == 1 else 2 * ncp
        res = {name: steady(fn, n)[0] for name, fn in (("unfused", unfused), ("fused", fused_))}
        rows = [0] if M == 1 else [0, 1023, M - 1]
        ref = oracle.matmul_rows(Xh, rows, Wh)
        half = p.N // 2
        got = Hf[rows].float().cpu().numpy().astype(np.float64) if dt == "f32" else \
            oracle.bf16_bits_to_f64(Hf[rows].view(torch.int16).cpu().numpy().view(np.uint16))
        rep = tolerance.check_swiglu(got, ref[:, :half], ref[:, half:], dt)
        if not rep.ok:
            raise SystemExit(f"bench: fused SwiGLU {key} does not match the oracle: {rep}")
        o = dict(shape=f"{p.N}x{p.K}", M=M, dtype=dt, swiglu_plan_us=round(res["fused"], 3),
                 swiglu_plan_kernel=fused.choice(M), plain_plus_activation_us=round(res["unfused"], 3),
                 plain_kernel=plain.choice(M), speedup=round(res["unfused"] / res["fused"], 3),
                 weight_copies_rotated=ncp)
        out[key] = o
        log(f"  SwiGLU {key}: plan {res['fused']:.2f} us ({fused.choice(M)}), plain + activation {res['unfused']:.2f} us")
        del Wrot
    return out


def rmsnorm_leg(plans, steps: int = 500):
    """The RMSNorm prologue folded into decode projections (M = 1) against the
    separate path (proj_rmsnorm, then the plain plan), rotating weight copies."""
    import numpy as np
    import torch

    import oracle
    import shape_specialised_bf16_amd as ssb
    import synth
    from oracle import tolerance

    eps = 1e-6
    sh = _stream_handle()
    out = {}
    for key, wl, pname, dt in (("decode_qkv_08b_m1", "decode_0.8b_layer_m1", "qkv", "f32"),
                               ("decode_qkv_27b_m1", "layer_27b", "qkv", "bf16")):
        cfg = synth.workload(wl)
        pi = [p.name for p in cfg.projections].index(pname)
        p = cfg.projections[pi]
        normp = plans.get(p.N, p.K, dt, rmsnorm_eps=eps)
        plain = plans.get(p.N, p.K, dt)
        Wh, Xh = weights(cfg, pi), synth.activations(cfg, pi, 1)
        gh = (1.0 + 0.25 * np.random.default_rng(cfg.no * 10 + pi).standard_normal(p.K)).astype(np.float32)
        Wrot, X, g = rotation(upload(Wh)), upload(Xh), torch.from_numpy(gh).cuda()
        ncp = len(Wrot)
        odt = torch.bfloat16 if dt == "bf16" else torch.float32
        Y, Y2 = (torch.empty((1, p.N), dtype=odt, device="cuda") for _ in range(2))
        Xn = torch.empty_like(X)
        xp, gp, xnp, yp, y2p = X.data_ptr(), g.data_ptr(), Xn.data_ptr(), Y.data_ptr(), Y2.data_ptr()
        wps = [w.data_ptr() for w in Wrot]
        norm_c = ssb._lib.proj_rmsnorm

        def separate(s):
            norm_c(xp, gp, xnp, 1, p.K, eps, sh)
            plain.run_ptr(xnp, wps[s % ncp], y2p, 1, sh)

        def tuned(s):
            normp.run_ptr(xp, wps[s % ncp], yp, 1, sh, gp)

        res = {name: steady(fn, steps)[0] for name, fn in (("separate", separate), ("tuned", tuned))}
        ref = oracle.rmsnorm_matmul(Xh, gh, Wh, eps)
        terms = oracle.rmsnorm_matmul(Xh, gh, Wh, eps, absolute=True)
        got = Y.view(torch.int16).cpu().numpy().view(np.uint16) if dt == "bf16" else Y.cpu().numpy()
        rep = tolerance.check_norm_projection(got, ref, terms, dt)
        if not rep.ok:
            raise SystemExit(f"bench: {key} with the norm prologue does not match the oracle: {rep}")
        out[key] = dict(shape=f"{p.N}x{p.K}", dtype=dt, tuned_us=round(res["tuned"], 3),
                        separate_us=round(res["separate"], 3), choice=normp.choice(1), weight_copies_rotated=ncp)
        log(f"  RMSNorm {key}: tuned {res['tuned']:.2f} us ({normp.choice(1)}), separate {res['separate']:.2f} us")
        del Wrot
    return out


def packed_leg(plans, steps: int = 300, rounds: int = 3):
    """Weights in the packed layout (proj_pack_weights once, then
    proj_run_packed) against row-major, each on its own tuned plan: the
    0.8B-like decode step (rotating weights), the 27B-like gate/up at
    M = 8192 and the 4B-like layer at M = 128 and 512, timed in alternation."""
    import torch

    import synth
    from shape_specialised_bf16_amd import pack_weights

    sh = _stream_handle()

    def alternate(fr, fp, n):
        warm(fr)
        tr, tp = [], []
        for _ in range(rounds):
            tr.append(events_us(fr, n))
            tp.append(events_us(fp, n))
        return statistics.median(tr), statistics.median(tp)

    out = {"workload": "packed weights (128-row panels of 128 x 64 blocks) vs row-major, each on its own tuned plan"}
    cfg = synth.workload("decode_0.8b_layer_m1")
    projs = cfg.projections
    pr = [plans.get(p.N, p.K, "f32") for p in projs]
    pk = [plans.get(p.N, p.K, "f32", packed=True) for p in projs]
    Wh = [weights(cfg, i) for i in range(len(projs))]
    Xs = [upload(synth.activations(cfg, i, 1)) for i in range(len(projs))]
    Ws = [upload(w) for w in Wh]
    Wps = [pack_weights(w) for w in Ws]
    Yr = [torch.empty((1, p.N), dtype=torch.float32, device="cuda") for p in projs]
    Yp = [torch.empty((1, p.N), dtype=torch.float32, device="cuda") for p in projs]
    step_bytes = sum(2 * p.N * p.K + 2 * p.K + 4 * p.N for p in projs)
    ncp = copies_for(sum(w.numel() * 2 for w in Ws))
    Wr_rot = [[w] + [w.clone() for _ in range(ncp - 1)] for w in Ws]
    Wp_rot = [[w] + [w.clone() for _ in range(ncp - 1)] for w in Wps]

    def dec(pls, rot, Ys):
        def step(s):
            c = s % ncp
            for i in range(len(projs)):
                pls[i].run_ptr(Xs[i].data_ptr(), rot[i][c].data_ptr(), Ys[i].data_ptr(), 1, sh)
        return step

    ur, up = alternate(dec(pr, Wr_rot, Yr), dec(pk, Wp_rot, Yp), steps)
    for i, p in enumerate(projs):
        if pk[i].choice(1) == pr[i].choice(1) and not torch.equal(Yp[i], Yr[i]):
            raise SystemExit(f"bench: packed {p.name} differs from row-major with the same kernel")
    out["decode_08b_m1"] = dict(unit="GB/s", rows=round(step_bytes / ur / 1e3, 1), packed=round(step_bytes / up / 1e3, 1),
                                packed_over_rows=round(ur / up, 3), weight_copies_rotated=ncp)
    log(f"  packed decode M=1: {out['decode_08b_m1']['packed']} GB/s vs row-major {out['decode_08b_m1']['rows']}")
    del Wr_rot, Wp_rot, Ws, Wps
    cfg27 = synth.workload("layer_27b")
    i = [p.name for p in cfg27.projections].index("gate_up")
    p, M = cfg27.projections[i], 8192
    wh, xh = weights(cfg27, i), synth.activations(cfg27, i, M)
    W, X = upload(wh), upload(xh)
    Wrot = rotation(W)
    Wprot = [pack_weights(w) for w in Wrot]
    n = len(Wrot)
    a, b = plans.get(p.N, p.K, "bf16"), plans.get(p.N, p.K, "bf16", packed=True)
    Ya, Yb = (torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    tr, tp = alternate(lambda s: a.run_ptr(X.data_ptr(), Wrot[s % n].data_ptr(), Ya.data_ptr(), M, sh),
                       lambda s: b.run_ptr(X.data_ptr(), Wprot[s % n].data_ptr(), Yb.data_ptr(), M, sh), n)
    _check_rows(Yb, xh, wh, [0, M // 2, M - 1], "bf16", f"packed {p.name} M={M}")
    f = 2.0 * M * p.N * p.K
    out["gate_up_27b_m8192"] = dict(unit="TFLOP/s", rows=round(f / tr / 1e6, 1), packed=round(f / tp / 1e6, 1),
                                    packed_over_rows=round(tr / tp, 3), kernel_rows=a.choice(M),
                                    kernel_packed=b.choice(M), weight_copies_rotated=n)
    log(f"  packed 27B gate/up M=8192: {out['gate_up_27b_m8192']['packed']} TFLOP/s vs row-major "
        f"{out['gate_up_27b_m8192']['rows']}")
    del Wrot, Wprot, Ya, Yb
    # the 4B-like layer at the row counts where its GEMMs stream W from HBM
    cfg4 = synth.workload("prefill_4b_layer")
    for M in (128, 512):
        tr_sum = tp_sum = flops = 0.0
        kern = {}
        for i, p in enumerate(cfg4.projections):
            wh, xh = weights(cfg4, i), synth.activations(cfg4, i, M)
            W, X = upload(wh), upload(xh)
            Wrot = rotation(W)
            Wprot = [pack_weights(w) for w in Wrot]
            n = len(Wrot)
            a, b = plans.get(p.N, p.K, "bf16"), plans.get(p.N, p.K, "bf16", packed=True)
            Ya, Yb = (torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda") for _ in range(2))
            tr, tp = alternate(lambda s: a.run_ptr(X.data_ptr(), Wrot[s % n].data_ptr(), Ya.data_ptr(), M, sh),
                               lambda s: b.run_ptr(X.data_ptr(), Wprot[s % n].data_ptr(), Yb.data_ptr(), M, sh),
                               max(n, 100))
            _check_rows(Yb, xh, wh, [0, M // 2, M - 1], "bf16", f"packed {p.name} M={M}")
            tr_sum, tp_sum, flops = tr_sum + tr, tp_sum + tp, flops + 2.0 * M * p.N * p.K
            kern[p.name] = dict(rows=a.choice(M), packed=b.choice(M), rows_us=round(tr, 2), packed_us=round(tp, 2))
            del Wrot, Wprot, W, X, Ya, Yb
            torch.cuda.empty_cache()
        out[f"prefill_4b_m{M}"] = dict(unit="TFLOP/s", rows=round(flops / tr_sum / 1e6, 1),
                                       packed=round(flops / tp_sum / 1e6, 1), packed_over_rows=round(tr_sum / tp_sum, 3),
                                       projections=kern)
        log(f"  packed 4B layer M={M}: {out[f'prefill_4b_m{M}']['packed']} TFLOP/s vs row-major "
            f"{out[f'prefill_4b_m{M}']['rows']}")
    return out


# ---------------------------------------------------------------- support
def traffic_for(key: str):
    """HBM bytes per launch from committed rocprofv3 counter runs (FETCH_SIZE and
    WRITE_SIZE, scaled by a copy kernel of known size), if they were taken on
    the current kernel source; else None."""
    from shape_specialised_bf16_amd.profile_summary import kernel_source_sha
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    e = d.get(key)
    if not e or e.get("source_sha") != kernel_source_sha(key.split("@")[0]):
        return None
    return round(e["bytes_per_launch"])


def counters_for(key: str):
    """Engine clock and matrix-unit busy share of a kernel from the committed
    rocprofv3 counter runs (GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES with
    the kernel trace), if they were taken on the current kernel source and the
    kernel ran long enough (>= 100 us) for its counter window to be the
    kernel's own; else None."""
    from shape_specialised_bf16_amd.profile_summary import kernel_source_sha
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        e = json.load(open(path)).get(key)
    except Exception:
        return None
    if not e or e.get("source_sha") != kernel_source_sha(key.split("@")[0]) or e.get("duration_us", 0) < 100:
        return None
    return dict(clock_ghz=round(e["clock_ghz"], 3), mfma_busy_share=round(e["mfma_busy_share"], 3),
                duration_us=round(e["duration_us"], 1))


def probe_bandwidth():
    import torch
    import shape_specialised_bf16_amd as ssb
    buf = torch.empty(1 << 30, dtype=torch.int32, device="cuda")      # 4 GiB
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    best = 0.0
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ssb.probe_read(buf, sink, never=0x12345678)
        e1.record()
        e1.synchronize()
        best = max(best, buf.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    return round(best, 1)


def cpu_baseline(host, step_bytes, budget_s: float = 10.0):
    """The oracle (plain fp64 triple loop, OpenMP over outputs) on the decode
    step, repeated for about `budget_s` seconds of CPU work; one of its
    projections also on a single thread."""
    import oracle
    cores = min(16, os.cpu_count() or 1)
    n, t0 = 0, time.time()
    while True:
        for X, W in host:
            oracle.matmul(X, W, threads=cores)
        n += 1
        if time.time() - t0 >= budget_s:
            break
    dt = (time.time() - t0) / n
    X, W = host[1]
    t1, k = time.time(), 0
    while k == 0 or time.time() - t1 < 2.0:
        oracle.matmul(X, W, threads=1)
        k += 1
    one = (time.time() - t1) / k
    return dict(value=round(step_bytes / dt / 1e9, 3), unit="GB/s", cores=cores, kind="oracle",
                sample=f"{n} full 27B-like decode steps (4 projections at M=1, {step_bytes / 1e6:.1f} MB each), "
                       f"{dt * 1e3:.1f} ms per step",
                single_core=dict(value=round((2 * W.size + 2 * X.size) / one / 1e9, 3), unit="GB/s",
                                 sample=f"{W.shape[0]}x{W.shape[1]} at M=1 on 1 thread, {k} runs, "
                                        f"{one * 1e3:.1f} ms each"))


def cpu_baseline_prefill(rows: int = 64):
    """The oracle on a `rows`-row sample of the 27B-like layer at M = 8192 (every
    projection), scaled to the full layer: the triple loop's cost is linear in
    M, so the rate is the sample's and the full-layer time is extrapolated."""
    import oracle
    import synth
    cfg = synth.workload("layer_27b")
    cores = min(16, os.cpu_count() or 1)
    fl, t = 0.0, 0.0
    for i, p in enumerate(cfg.projections):
        X, W = synth.activations(cfg, i, rows), weights(cfg, i)
        t0 = time.time()
        oracle.matmul(X, W, threads=cores)
        t += time.time() - t0
        fl += 2.0 * rows * p.N * p.K
    full = t * 8192 / rows
    return dict(value=round(fl / t / 1e12, 5), unit="TFLOP/s", cores=cores, kind="oracle", extrapolated=True,
                sample=f"{rows} of 8192 rows of the 27B-like layer (4 projections), {t:.1f} s; full layer "
                       f"extrapolated to {full:.0f} s")


def profile_graph08(steps: int = 60):
    """The 0.8B-like decode step (QKV, out, gate/up, down, head at M = 1, f32 Y,
    rotating weight copies) launched eagerly, then, after a pause, replayed as
    one recorded HIP graph per rotation of the weight copies; for a
    rocprofv3 --kernel-trace of the per-kernel durations and the gaps between
    kernels in either mode (profile_summary steps)."""
    import torch

    import synth

    cfg = synth.workload("decode_0.8b_layer_m1")
    projs = cfg.projections
    plans = Plans()
    pl = [plans.get(p.N, p.K, "f32") for p in projs]
    Xs = [upload(synth.activations(cfg, i, 1)) for i in range(len(projs))]
    Ws = [upload(weights(cfg, i)) for i in range(len(projs))]
    Ys = [torch.empty((1, p.N), dtype=torch.float32, device="cuda") for p in projs]
    ncp = copies_for(sum(w.numel() * 2 for w in Ws))
    Wrot = [[w] + [w.clone() for _ in range(ncp - 1)] for w in Ws]
    sh = _stream_handle()

    def step(s, h=sh):
        for i in range(len(projs)):
            pl[i].run_ptr(Xs[i].data_ptr(), Wrot[i][s % ncp].data_ptr(), Ys[i].data_ptr(), 1, h)

    warm(step, DEVICE_WARM_MS)
    for s in range(steps):
        step(s)
    torch.cuda.synchronize()
    gs = torch.cuda.Stream()
    gh = ctypes.c_void_p(gs.cuda_stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gs):
        with torch.cuda.graph(g, stream=gs):
            for c in range(ncp):
                step(c, gh)
    torch.cuda.synchronize()
    time.sleep(0.05)
    warm(lambda s: g.replay(), DEVICE_WARM_MS)
    for _ in range(max(1, steps // ncp)):
        g.replay()
    torch.cuda.synchronize()
    # the floor: a projection that reads almost nothing (64 x 64 weights), back to back
    tiny = plans.get(64, 64, "f32")
    tx, tw = upload(synth.normal_bf16(99, 0, (1, 64), 1.0)), upload(synth.normal_bf16(99, 1, (64, 64), 0.02))
    ty = torch.empty((1, 64), dtype=torch.float32, device="cuda")
    time.sleep(0.05)
    for _ in range(200):
        tiny.run_ptr(tx.data_ptr(), tw.data_ptr(), ty.data_ptr(), 1, sh)
    torch.cuda.synchronize()
    log(f"profile mode: 0.8B decode step, {steps} eager steps then {max(1, steps // ncp) * ncp} replayed "
        f"({ncp} steps per graph): " + ", ".join(f"{p.name} {pl[i].choice(1)}" for i, p in enumerate(projs))
        + f"; then 200 launches of a 64x64 projection ({tiny.choice(1)})")
    plans.close()


def profile_mode(which: str, M: int, launches: int = 30):
    """Only one dominant kernel at its bench configuration -- decode: the 27B-like
    gate/up GEMV (34816x5120, M=1, bf16 Y) on rotating weight copies; decode08:
    the 0.8B-like head GEMV (151936x1024, M=1, f32 Y); prefill: the 4B-like
    gate/up GEMM (18432x2560, bf16 Y) at M; prefill27: the 27B-like gate/up GEMM
    (34816x5120, bf16 Y) at M -- then a 1 GiB device copy of known size that
    calibrates the FETCH_SIZE / WRITE_SIZE counters; for rocprofv3 counter runs."""
    import torch

    import synth
    from shape_specialised_bf16_amd import Plan

    wl, pname, dt = {"decode": ("layer_27b", "gate_up", "bf16"), "decode08": ("decode_0.8b_layer_m1", "head", "f32"),
                     "prefill": ("prefill_4b_layer", "gate_up", "bf16"),
                     "prefill27": ("layer_27b", "gate_up", "bf16")}[which]
    if which.startswith("decode"):
        M = 1
    cfg = synth.workload(wl)
    pi = [p.name for p in cfg.projections].index(pname)
    p = cfg.projections[pi]
    plan = Plan(p.N, p.K, dt)
    Wrot = rotation(upload(weights(cfg, pi)))
    X = upload(synth.activations(cfg, pi, M))
    Y = torch.empty((M, p.N), dtype=plan.out_dtype, device="cuda")
    for i in range(launches if M == 1 else 10):
        plan.run(X, Wrot[i % len(Wrot)], Y)
    torch.cuda.synchronize()
    a = torch.ones(1 << 29, dtype=torch.int16, device="cuda")      # 1 GiB
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"profile mode: {plan.choice(M)} on {p.N}x{p.K} M={M}, then 3 x 1 GiB copy")


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 4B-like prefill and long-prompt legs")
    ap.add_argument("--no-extra", action="store_true", help="skip the fusion and packed-layout legs")
    ap.add_argument("--prefill-m", type=int, default=2048, help="row count of the GEMM in the profile-prefill modes")
    ap.add_argument("--mode", default="full", choices=["full", "profile-decode", "profile-decode08", "profile-prefill",
                                                       "profile-prefill27", "profile-graph08"],
                    help="profile-*: only that leg's dominant kernel and a calibration copy, for rocprofv3 "
                         "counter runs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (got --gpus {args.gpus}); the projection shards "
              "by output rows across GPUs but no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)
    if args.mode == "profile-graph08":
        profile_graph08()
        return
    if args.mode != "full":
        profile_mode(args.mode.split("-")[1], args.prefill_m)
        return

    import torch

    torch.cuda.set_device(0)
    t_start = time.time()
    log(f"device: {torch.cuda.get_device_name(0)}")
    clk = {"before": clocks()}
    plans = Plans()

    # ---- headline: the 27B-like layer at M = 1
    d = decode_layer(plans, "layer_27b", "bf16", args.steps, args.warmup, graph=True)
    value = d["step_bytes"] / d["step_us"] / 1e3
    dom = max(d["per_shape"], key=lambda x: x["bytes"])
    log(f"decode 27B layer M=1: {d['step_us']:.2f} us/step, {value:.0f} GB/s; "
        + ", ".join(f"{x['proj']} {x['GBps']}" for x in d["per_shape"]))
    result = {
        "metric": "decode GEMV HBM GB/s (% peak); prefill GEMM bf16 TFLOP/s (% MFMA peak)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["step_us"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded bf16 weights ~N(0,0.01) with 1% outliers x10, activations ~N(0,1); no model weights)",
        "pct_peak": round(100 * value / HBM_PEAK_GBS, 1),
        "config": {
            "workload": "layer_27b_m1: QKV 5120->10240, out 8192->5120, gate/up 5120->34816, down 17408->5120 at "
                        "M=1, bf16 Y (the 27B-like layer; its M=8192 prefill under prefill_27b_m8192)",
            "M": 1,
            "bytes_per_step": d["step_bytes"],
            "weight_copies_rotated": d["weight_copies_rotated"],
            "device_warmup_ms": d["device_warmup_ms"],
            "launch": "four proj_run calls per step on torch's current stream",
            "parallelism": "single GPU",
        },
        "step_us": d["step_dist_us"],
        "roofline": {
            "bound": "hbm",
            "kernel": dom["kernel"],
            "shape": f"{dom['N']}x{dom['K']}",
            "achieved": dom["GBps"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dom["GBps"] / HBM_PEAK_GBS, 4),
            "traffic": traffic_for(f"{dom['kernel']}@{dom['N']}x{dom['K']}"),
            "bytes_per_launch": dom["bytes"],
            "mean_launch_us": dom["mean_launch_us"],
            "timing": "HIP events on the launch stream around 200 back-to-back launches on rotating weight "
                      "copies (median of 3 rounds); single_launch_us: an event pair around each of 300 launches",
            "single_launch_us": dom["single_launch_us"],
        },
        "per_shape": d["per_shape"],
        "graph": d["graph"],
        "host_call_us": d["host_call_us"],
    }
    host27 = d.pop("host")
    torch.cuda.empty_cache()

    # ---- the same layer at M = 8192
    pf27 = prefill_layer(plans, "layer_27b", (8192,), rounds=5)
    result["prefill_27b_m8192"] = dict(workload="layer_27b at M=8192, bf16 Y, weights rotating over >= 2 GiB",
                                       **pf27["M8192"])
    result["roofline_prefill"] = roofline_prefill(pf27, 8192)

    # ---- the 0.8B-like layer and head at M = 1, and its graph replay
    d8 = decode_layer(plans, "decode_0.8b_layer_m1", "f32", args.steps, args.warmup, graph=True)
    v8 = d8["step_bytes"] / d8["step_us"] / 1e3
    result["decode_08b"] = dict(workload="decode_0.8b_layer_m1: QKV 1024->2048, out 1024->1024, gate/up 1024->6144, "
                                          "down 3072->1024, head 1024->151936 at M=1, Y f32",
                                value=round(v8, 1), unit="GB/s", pct_peak=round(100 * v8 / HBM_PEAK_GBS, 1),
                                step_us=round(d8["step_us"], 3), step_dist_us=d8["step_dist_us"],
                                bytes_per_step=d8["step_bytes"], weight_copies_rotated=d8["weight_copies_rotated"],
                                per_shape=d8["per_shape"], graph=d8["graph"], host_call_us=d8["host_call_us"])
    hd = max(d8["per_shape"], key=lambda x: x["bytes"])
    result["decode_08b"]["roofline"] = dict(bound="hbm", kernel=hd["kernel"], shape=f"{hd['N']}x{hd['K']}",
                                            achieved=hd["GBps"], peak=HBM_PEAK_GBS, unit="GB/s",
                                            frac=round(hd["GBps"] / HBM_PEAK_GBS, 4),
                                            traffic=traffic_for(f"{hd['kernel']}@{hd['N']}x{hd['K']}"))
    log(f"decode 0.8B layer + head M=1: {d8['step_us']:.2f} us/step, {v8:.0f} GB/s; graph "
        f"{d8['graph']['replayed_step_us']} vs eager {d8['graph']['eager_step_us']} us")
    d8.pop("host")

    # ---- prefill: the 4B-like layer, and the long prompt
    if not args.no_prefill:
        pf4 = prefill_layer(plans, "prefill_4b_layer", (128, 512, 2048), rounds=5)
        result["prefill_4b"] = dict(workload="prefill_4b_layer: QKV 2560->5120, out 4096->2560, gate/up 2560->18432, "
                                             "down 9216->2560, Y bf16, weights rotating over >= 2 GiB", **pf4)
        for M in (128, 512, 2048):
            result["prefill_4b"][f"M{M}"]["roofline"] = roofline_prefill(pf4, M)
        result["long_prompt"] = long_prompt(plans)
    if not args.no_extra:
        result["swiglu_epilogue"] = swiglu_leg(plans)
        result["rmsnorm_prologue"] = rmsnorm_leg(plans)
        result["packed_weights"] = packed_leg(plans)
    torch.cuda.synchronize()
    cr = plans.created
    result["plan_create"] = dict(plans=len(cr), total_s=round(sum(x["wall_s"] for x in cr), 1),
                                 compile_s=round(sum(x["compile_s"] for x in cr), 1),
                                 tune_s=round(sum(x["tune_s"] for x in cr), 1), per_plan=cr)
    plans.close()
    torch.cuda.empty_cache()
    clk["after"] = clocks()
    result["clocks"] = clk
    result["probe"] = {"read_GBps": probe_bandwidth(), "kernel": "proj_probe_read", "bytes": 4 << 30}
    result["pct_probe"] = round(100 * value / result["probe"]["read_GBps"], 1)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(host27, d["step_bytes"])
        result["cpu_baseline_prefill"] = cpu_baseline_prefill()
    else:
        result["cpu_baseline"] = None
    result["bench_wall_s"] = round(time.time() - t_start, 1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
