"""Engine clock under a GEMM's own load, read inside the kernel (measurement only).

A kernel's flop rate is bounded by 256 CUs x 4096 flop per clock x the engine
clock it actually runs at, and under a dense MFMA load that clock sits well
below the 2.4 GHz of the nominal peak.  Board-level readings (amd-smi, the power
sensors) are sampled too seldom to see one kernel of a few hundred microseconds.

This tool compiles a copy of a GEMM candidate of a plan whose workgroups read
the shader-clock counter (s_memtime, engine cycles) and the constant 100 MHz
counter (s_memrealtime) as they start and as they finish, launches that copy on
the grid and operands the plan would use, and reports the clock each workgroup
ran at: its engine cycles over its real time.  The copy is built by the
library's own compile helper (proj_rtc, the plan's compiler options) from the
plan's emitted source, with the candidate's template call unchanged between
the two readings.  The product never launches it: proj_run runs the unmodified
candidate.

Only whole-tile GEMM candidates (no split-K, no split tail) are supported; for
any other candidate `measure` returns None.
"""
from __future__ import annotations

import ctypes
import os
import re
import statistics
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
REALTIME_MHZ = 100.0            # s_memrealtime's constant rate on gfx9 parts
CUS, FLOP_PER_CLK_PER_CU = 256, 4096

_NAME = re.compile(r"^gemm_(\d+)x(\d+)x\d+_st\d+_w(\d+)x(\d+)_sw\d+_g\d+_sk1(_b\d+)?$")
_hip = None
_built: dict = {}


def _hip_lib():
    global _hip
    if _hip is None:
        import torch  # noqa: F401  (torch's HIP runtime first: the library below must be the same one)
        _hip = ctypes.CDLL("libamdhip64.so.7")
    return _hip


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"clock probe: {what} failed with HIP error {rc}")


def probe_source(full_src: str, name: str) -> str:
    """The plan's emitted source cut before its candidate wrappers, plus one
    kernel `clk_probe` that brackets candidate `name`'s template call with the
    two counter readings (per workgroup: start cycles, start real time, end
    cycles, end real time, 4 x u64 at clk[4 * blockIdx.x])."""
    m = re.search(r'extern "C" __global__ __launch_bounds__\((\d+)\) void ' + re.escape(name) +
                  r'\(const u16\* __restrict__ X[^)]*\)\n\{ (gemm_mfma<[^;]*;) \}', full_src)
    if not m:
        raise ValueError(f"clock probe: no wrapper for {name} in the emitted source")
    cut = re.search(r"^// (gemv|gemm)_\w+: ", full_src, re.M)
    if not cut or cut.start() > m.start():
        raise ValueError("clock probe: candidate wrappers not found where expected")
    bounds, call = m.group(1), m.group(2)
    return (full_src[:cut.start()] +
            f'extern "C" __global__ __launch_bounds__({bounds}) void clk_probe(const u16* __restrict__ X, '
            "const u16* __restrict__ W, void* __restrict__ Y, float* __restrict__ ws, const float* __restrict__ gamma, "
            "int M, unsigned long long* __restrict__ clk)\n"
            "{\n"
            "    const unsigned long long c0 = __builtin_amdgcn_s_memtime();\n"
            "    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();\n"
            "    if (threadIdx.x == 0) { clk[4 * blockIdx.x] = c0; clk[4 * blockIdx.x + 1] = r0; }\n"
            "    __builtin_amdgcn_s_waitcnt(0);   // nothing of the probe still in flight when the GEMM starts\n"
            f"    {call}\n"
            "    const unsigned long long c1 = __builtin_amdgcn_s_memtime();\n"
            "    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();\n"
            "    if (threadIdx.x == 0) { clk[4 * blockIdx.x + 2] = c1; clk[4 * blockIdx.x + 3] = r1; }\n"
            "}\n")


def _build(N: int, K: int, dtype: str, name: str, arch: str = "gfx950"):
    key = (N, K, dtype, name, arch)
    if key in _built:
        return _built[key]
    from shape_specialised_bf16_amd import emit_source
    src = probe_source(emit_source(N, K, dtype, arch=arch), name)
    helper = os.path.join(HERE, "proj_rtc")
    if not os.access(helper, os.X_OK):
        raise RuntimeError("clock probe: the proj_rtc helper is not built")
    with tempfile.TemporaryDirectory(prefix="proj-clk-") as d:
        sp, cp = os.path.join(d, "probe.hip"), os.path.join(d, "probe.co")
        with open(sp, "w") as f:
            f.write(src)
        r = subprocess.run([helper, arch, sp, cp], capture_output=True, text=True, timeout=600)
        if r.returncode != 0:
            raise RuntimeError(f"clock probe: compile failed ({r.returncode}): {r.stderr[-2000:]}")
        with open(cp, "rb") as f:
            image = f.read()
    hip = _hip_lib()
    mod, fn = ctypes.c_void_p(), ctypes.c_void_p()
    buf = ctypes.create_string_buffer(image, len(image))
    _check(hip.hipModuleLoadData(ctypes.byref(mod), buf), "hipModuleLoadData")
    _check(hip.hipModuleGetFunction(ctypes.byref(fn), mod, b"clk_probe"), "hipModuleGetFunction")
    _built[key] = (mod, fn, buf)   # the image stays referenced while the module is loaded
    return _built[key]


def geometry(name: str, N: int, M: int):
    """(grid, threads) of a whole-tile GEMM candidate at M rows, or None."""
    m = _NAME.match(name)
    if not m:
        return None
    BM, BN, WM, WN = (int(m.group(i)) for i in (1, 2, 3, 4))
    if N % BN:
        return None
    return ((M + BM - 1) // BM) * (N // BN), 64 * WM * WN


def measure(N: int, K: int, dtype: str, name: str, X, Ws, Y, M: int, launches: int = 40, warm_s: float = 0.3):
    """Launch the probe copy of candidate `name` (plan N x K, output dtype) on
    X [M, K], each W of Ws [N, K] in turn and Y [M, N] (torch device tensors),
    on torch's current stream: first for `warm_s` seconds, then `launches`
    times with an event pair each.  Returns per-workgroup clocks (median, p10,
    p90, and the real-time-weighted mean over all workgroups of all launches),
    the median launch time and the flop rate, or None for an unsupported
    candidate."""
    import time

    import torch

    g = geometry(name, N, M)
    if g is None:
        return None
    grid, threads = g
    if tuple(X.shape) != (M, K) or tuple(Y.shape) != (M, N) or any(tuple(w.shape) != (N, K) for w in Ws):
        raise ValueError("clock probe: operand shapes do not match the plan")
    # bf16 operands may come as bf16 or as their 16-bit patterns (int16), as the binding takes them
    b16 = (torch.bfloat16, torch.int16)
    want = b16 if dtype == "bf16" else (torch.float32,)
    if X.dtype not in b16 or Y.dtype not in want or any(w.dtype not in b16 for w in Ws):
        raise ValueError("clock probe: operand types do not match the plan")
    if not (X.is_contiguous() and Y.is_contiguous() and all(w.is_contiguous() for w in Ws)):
        raise ValueError("clock probe: operands must be contiguous")
    fn = _build(N, K, dtype, name)[1]
    hip = _hip_lib()
    clk = torch.zeros(4 * grid, dtype=torch.int64, device=X.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch(w):
        args = [ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(Y.data_ptr()),
                ctypes.c_void_p(0), ctypes.c_void_p(0), ctypes.c_int(M), ctypes.c_void_p(clk.data_ptr())]
        arr = (ctypes.c_void_p * len(args))(*[ctypes.cast(ctypes.pointer(a), ctypes.c_void_p) for a in args])
        _check(hip.hipModuleLaunchKernel(fn, grid, 1, 1, threads, 1, 1, 0, stream, arr, None), "launch")

    t0, n = time.time(), 0
    while time.time() - t0 < warm_s:
        launch(Ws[n % len(Ws)])
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    per_wg, us, cyc_sum, rt_sum = [], [], 0.0, 0.0
    for i in range(launches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        launch(Ws[i % len(Ws)])
        e1.record()
        torch.cuda.synchronize()
        us.append(e0.elapsed_time(e1) * 1e3)
        t = clk.view(grid, 4).cpu().to(torch.float64)
        cyc, rt = t[:, 2] - t[:, 0], t[:, 3] - t[:, 1]
        if bool((rt <= 0).any()) or bool((cyc <= 0).any()):
            raise RuntimeError("clock probe: a workgroup left no readings")
        per_wg.extend((cyc / rt * REALTIME_MHZ).tolist())
        cyc_sum += float(cyc.sum())
        rt_sum += float(rt.sum())
    per_wg.sort()
    q = lambda f: per_wg[min(len(per_wg) - 1, int(f * len(per_wg)))]
    mean_mhz = cyc_sum / rt_sum * REALTIME_MHZ
    us_med = statistics.median(us)
    tflops = 2.0 * M * N * K / us_med / 1e6
    peak = CUS * FLOP_PER_CLK_PER_CU * mean_mhz * 1e6 / 1e12
    return dict(kernel=name, M=M, launches=launches, workgroups=grid,
                mhz_weighted=round(mean_mhz, 1), mhz_median=round(q(0.5), 1), mhz_p10=round(q(0.1), 1),
                mhz_p90=round(q(0.9), 1), probe_us_median=round(us_med, 2), probe_tflops=round(tflops, 1),
                peak_at_kernel_clock=round(peak, 1), frac_at_kernel_clock=round(tflops / peak, 4))
