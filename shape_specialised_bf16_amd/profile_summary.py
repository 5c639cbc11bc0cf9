"""Summaries of rocprofv3 output for the projection kernels.

    python -m shape_specialised_bf16_amd.profile_summary stats <dir-or-db> [--match S] [--stream last] [--last N]
        per-kernel dispatch count and mean/min/max duration (us) from a
        ``--kernel-trace`` run (rocpd ``*_results.db`` or ``*_kernel_trace.csv``);
        ``--stream last`` keeps only the stream of the last dispatch (the timed
        loop), dropping the load-time tuner's launches; ``--last N`` adds the mean
        of each kernel's last N dispatches (a benchmark's timed rounds come after
        its warm-up launches of the same kernel).

    python -m shape_specialised_bf16_amd.profile_summary counters <dir> --kernel NAME [--last N]
        per-launch medians (over the kernel's last N dispatches) of every counter
        of a ``--pmc ... --kernel-trace`` run, the kernel's duration from the same
        run, and what they imply: the engine clock GRBM_GUI_ACTIVE / duration
        (GRBM_GUI_ACTIVE counts busy cycles of each XCD's graphics engine, summed
        over the XCDs), and with SQ_VALU_MFMA_BUSY_CYCLES the share of SIMD cycles
        (CUs x 4 SIMDs x busy cycles of one XCD) that the matrix units were busy.

    python -m shape_specialised_bf16_amd.profile_summary steps <dir> --period P [--phase-gap-us G]
        a repeated sequence of P kernels (one step of a benchmark) in a
        ``--kernel-trace`` run: the dispatches of the GPU's busiest stretches are
        split into phases at idle gaps longer than G us, and in each phase the
        last complete steps give, per position in the step, the median kernel
        duration and the median gap from the end of the previous kernel to the
        start of this one -- what the step spends in kernels and between them.

    python -m shape_specialised_bf16_amd.profile_summary traffic --fetch <dir> --write <dir>
            --kernel NAME --calib NAME --calib-bytes B [--out profiles/traffic.json --key KEY]
        HBM bytes per launch of kernel NAME from two ``--pmc FETCH_SIZE`` /
        ``--pmc WRITE_SIZE`` runs.  Each counter (KiB per dispatch) is scaled by
        the ratio of the known bytes of a plain copy kernel (``--calib``, which
        reads and writes ``--calib-bytes``) to what the same counter reports for
        it.  With ``--out`` the result is merged into a JSON file keyed by KEY,
        together with the hash of the kernel sources it was measured on.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sqlite3
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def kernel_source_sha(kernel: str) -> str:
    """Hash of the device sources a kernel is built from (the shared helpers and
    its family's file), to tell whether a stored measurement is still current."""
    fam = "gemv.hip" if kernel.startswith("gemv") else "gemm.hip"
    h = hashlib.sha256()
    for f in ("device_common.hip", fam):
        with open(os.path.join(HERE, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _dispatches(path: str):
    """(name, stream, start, end, dispatch_id, grid) of every kernel dispatch."""
    dbs = [path] if path.endswith(".db") else glob.glob(os.path.join(path, "**", "*_results.db"), recursive=True)
    if dbs:
        db = sqlite3.connect(dbs[0])
        return [tuple(r) for r in db.execute(
            "select name, stream_id, start, end, dispatch_id, grid_x * grid_y from kernels order by start")]
    csvs = glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True)
    if not csvs:
        raise SystemExit(f"no kernel trace under {path}")
    out = []
    for r in csv.DictReader(open(csvs[0])):
        grid = int(r.get("Grid_Size_X", r.get("Grid_Size", 0)) or 0) * int(r.get("Grid_Size_Y", 1) or 1)
        out.append((r["Kernel_Name"], int(r.get("Stream_Id", 0) or 0), int(r["Start_Timestamp"]),
                    int(r["End_Timestamp"]), int(r["Dispatch_Id"]), grid))
    return sorted(out, key=lambda t: t[2])


def stats(path: str, match: str = "", stream: str = "all", last: int = 0):
    rows = _dispatches(path)
    if stream == "last" and rows:
        s = rows[-1][1]
        rows = [r for r in rows if r[1] == s]
    by = {}
    for name, _, a, b, _, grid in rows:
        if match and match not in name:
            continue
        by.setdefault((name, grid), []).append((b - a) / 1e3)   # one entry per kernel and launch size
    out = []
    for (name, grid), d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        out.append(dict(kernel=name, grid=grid, calls=len(d), mean_us=statistics.mean(d), min_us=min(d),
                        max_us=max(d), total_us=sum(d), last_mean_us=statistics.mean(d[-last:]) if last else None))
    return out


def _counter(path: str, counter: str):
    """{dispatch_id: (kernel name, value)} for one counter of a --pmc run."""
    csvs = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    out = {}
    if csvs:
        for r in csv.DictReader(open(csvs[0])):
            if r["Counter_Name"] == counter:
                out[int(r["Dispatch_Id"])] = (r["Kernel_Name"], float(r["Counter_Value"]))
        return out
    dbs = glob.glob(os.path.join(path, "**", "*_results.db"), recursive=True)
    if not dbs:
        raise SystemExit(f"no counter output under {path}")
    db = sqlite3.connect(dbs[0])
    for did, name, val in db.execute(
            "select dispatch_id, kernel_name, value from counters_collection where counter_name = ?", (counter,)):
        out[int(did)] = (name, float(val))
    return out


def _per_launch(vals, name, last):
    """Median over the last `last` dispatches of kernel `name` (the profiled
    loop's own launches; the load-time tuner runs the same kernel earlier, at
    other row counts).  The name must match exactly: a split-tail GEMM's second
    pass is named after it ("<name>_reduce")."""
    v = [vals[d][1] for d in sorted(vals) if vals[d][0].strip() == name][-last:]
    if not v:
        raise SystemExit(f"kernel {name!r} not found in counter output")
    return statistics.median(v)


def counters(path, kernel, last=5, cus=256, xcds=8):
    """Medians of every counter over the kernel's last `last` dispatches, its
    duration, and the derived clock and matrix-unit busy share."""
    csvs = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not csvs:
        raise SystemExit(f"no counter output under {path}")
    names = sorted({r["Counter_Name"] for r in csv.DictReader(open(csvs[0]))})
    out = {n: _per_launch(_counter(path, n), kernel, last) for n in names}
    durs = [(b - a) / 1e3 for name, _, a, b, _, _ in _dispatches(path) if name.strip() == kernel][-last:]
    if durs:
        out["duration_us"] = statistics.median(durs)
    if "GRBM_GUI_ACTIVE" in out and durs:
        cyc = out["GRBM_GUI_ACTIVE"] / xcds              # busy cycles of one XCD's engine
        out["clock_ghz"] = cyc / (out["duration_us"] * 1e3)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in out:
            out["mfma_busy_share"] = out["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * cus * 4)
        if "SQ_BUSY_CYCLES" in out:
            out["sq_busy_share"] = out["SQ_BUSY_CYCLES"] / (cyc * xcds)
    return out


def steps(path, period, phase_gap_us=1000.0, last=40):
    """Per phase: [(kernel, median duration us, median gap before us)] over the
    phase's last `last` complete steps of `period` kernels."""
    rows = _dispatches(path)
    phases, cur = [], []
    for r in rows:
        if cur and (r[2] - cur[-1][3]) / 1e3 > phase_gap_us:
            phases.append(cur)
            cur = []
        cur.append(r)
    if cur:
        phases.append(cur)
    out = []
    for ph in phases:
        n = len(ph) // period
        if n < 4:
            continue
        # align on the step: the phase's last n * period dispatches
        ph = ph[len(ph) - n * period:]
        ph = ph[-min(last, n) * period:]
        # only stretches that repeat the same kernels in the same order
        if any(ph[i][0] != ph[i % period][0] or ph[i][5] != ph[i % period][5] for i in range(len(ph))):
            continue
        pos = []
        for j in range(period):
            d = [(ph[i][3] - ph[i][2]) / 1e3 for i in range(j, len(ph), period)]
            g = [(ph[i][2] - ph[i - 1][3]) / 1e3 for i in range(max(j, 1), len(ph), period)]
            pos.append((ph[j][0], statistics.median(d), statistics.median(g) if g else 0.0))
        span = (ph[-1][3] - ph[0][2]) / 1e3 / (len(ph) / period)
        out.append(dict(steps=len(ph) // period, step_us=span, positions=pos))
    return out


def traffic(fetch_dir, write_dir, kernel, calib, calib_bytes, last=5):
    f = _counter(fetch_dir, "FETCH_SIZE")
    w = _counter(write_dir, "WRITE_SIZE")
    f_k, w_k = _per_launch(f, kernel, last), _per_launch(w, kernel, last)
    # the calibration copy is the largest dispatch of its name (small copies of the
    # same blit kernel also occur while plans are built)
    f_c = max(x for n, x in f.values() if calib in n)
    w_c = max(x for n, x in w.values() if calib in n)
    f_scale = calib_bytes / f_c
    w_scale = calib_bytes / w_c
    return dict(fetch_bytes=f_k * f_scale, write_bytes=w_k * w_scale,
                bytes_per_launch=f_k * f_scale + w_k * w_scale,
                raw_fetch_kib=f_k, raw_write_kib=w_k, calib_fetch_kib=f_c, calib_write_kib=w_c,
                fetch_scale=f_scale, write_scale=w_scale, calib_kernel=calib, calib_bytes=calib_bytes)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("path")
    s.add_argument("--match", default="")
    s.add_argument("--stream", default="all", choices=["all", "last"])
    s.add_argument("--last", type=int, default=0, help="also the mean of each kernel's last N dispatches")
    st = sub.add_parser("steps")
    st.add_argument("path")
    st.add_argument("--period", type=int, required=True)
    st.add_argument("--phase-gap-us", type=float, default=1000.0)
    st.add_argument("--last", type=int, default=40)
    c = sub.add_parser("counters")
    c.add_argument("path")
    c.add_argument("--kernel", required=True)
    c.add_argument("--last", type=int, default=5)
    c.add_argument("--out")
    c.add_argument("--key")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--calib", required=True)
    t.add_argument("--calib-bytes", type=float, required=True)
    t.add_argument("--out")
    t.add_argument("--key")
    t.add_argument("--last", type=int, default=5, help="dispatches of the kernel to use, counted from the end")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        for r in stats(a.path, a.match, a.stream, a.last):
            tail = f"  last{a.last} {r['last_mean_us']:9.3f}" if a.last else ""
            print(f"{r['kernel'][:48]:48s} grid {r['grid']:10d} calls {r['calls']:5d}  mean {r['mean_us']:9.3f} us  "
                  f"min {r['min_us']:10.3f}  max {r['max_us']:10.3f}  total {r['total_us']:12.1f}{tail}")
    elif a.cmd == "steps":
        for k, ph in enumerate(steps(a.path, a.period, a.phase_gap_us, a.last)):
            print(f"phase {k}: {ph['steps']} steps, {ph['step_us']:.2f} us per step (first kernel start to last end)")
            for name, d, g in ph["positions"]:
                print(f"    {name[:44]:44s} kernel {d:8.3f} us   gap before {g:7.3f} us")
            tot_k = sum(d for _, d, _ in ph["positions"])
            tot_g = sum(g for _, _, g in ph["positions"])
            print(f"    sum: kernels {tot_k:.3f} us, gaps {tot_g:.3f} us")
    elif a.cmd == "counters":
        r = counters(a.path, a.kernel, a.last)
        for k, v in r.items():
            print(f"{k:28s} {v:.6g}")
        if a.out:
            r["source_sha"] = kernel_source_sha(a.kernel)
            d = json.load(open(a.out)) if os.path.exists(a.out) else {}
            d[a.key or a.kernel] = r
            with open(a.out, "w") as fh:
                json.dump(d, fh, indent=1, sort_keys=True)
                fh.write("\n")
    else:
        r = traffic(a.fetch, a.write, a.kernel, a.calib, a.calib_bytes, a.last)
        r["source_sha"] = kernel_source_sha(a.kernel)
        print(json.dumps(r, indent=1))
        if a.out:
            d = json.load(open(a.out)) if os.path.exists(a.out) else {}
            d[a.key or a.kernel] = r
            with open(a.out, "w") as fh:
                json.dump(d, fh, indent=1, sort_keys=True)
                fh.write("\n")


if __name__ == "__main__":
    sys.exit(main())
