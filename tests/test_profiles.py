"""The committed measurement records under profiles/ (CPU only).

profiles/traffic.json holds the HBM bytes per launch that the benchmark's
roofline reports, derived from rocprofv3 FETCH_SIZE / WRITE_SIZE counter runs
scaled by a device copy of known size.  These checks keep the file honest
against its own raw counts, and tie each entry to a kernel that the code
generator still emits for the named shape.
"""
import json
import os
import re

import pytest

import shape_specialised_bf16_amd as ssb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def _entries():
    with open(os.path.join(PROFILES, "traffic.json")) as f:
        return sorted(json.load(f).items())


@pytest.mark.parametrize("key,e", _entries(), ids=[k for k, _ in _entries()])
def test_traffic_entry_follows_from_its_raw_counts(key, e):
    assert e["fetch_scale"] == pytest.approx(e["calib_bytes"] / e["calib_fetch_kib"], rel=1e-9)
    assert e["write_scale"] == pytest.approx(e["calib_bytes"] / e["calib_write_kib"], rel=1e-9)
    # the copy reads and writes calib_bytes: FETCH_SIZE counts half of it, WRITE_SIZE all of it
    assert e["fetch_scale"] == pytest.approx(2048.0, rel=0.01)
    assert e["write_scale"] == pytest.approx(1024.0, rel=0.01)
    assert e["fetch_bytes"] == pytest.approx(e["raw_fetch_kib"] * e["fetch_scale"], rel=1e-9)
    assert e["write_bytes"] == pytest.approx(e["raw_write_kib"] * e["write_scale"], rel=1e-9)
    assert e["bytes_per_launch"] == pytest.approx(e["fetch_bytes"] + e["write_bytes"], rel=1e-9)
    assert re.fullmatch(r"[0-9a-f]{16}", e["source_sha"])


@pytest.mark.parametrize("key", [k for k, _ in _entries()])
def test_traffic_entry_names_an_emitted_kernel(key):
    m = re.fullmatch(r"(\w+)@(\d+)x(\d+)(?:m\d+)?", key)
    assert m, key
    kernel, N, K = m.group(1), int(m.group(2)), int(m.group(3))
    dtype = "f32" if kernel.startswith("gemv") else "bf16"      # the head at decode: f32 logits
    src = ssb.emit_source(N, K, dtype)
    assert re.search(rf"void {kernel}\(", src), f"{kernel} is no longer a candidate for {N}x{K}"


def test_every_summary_gives_its_command():
    for name in os.listdir(PROFILES):
        if not name.endswith(".txt"):
            continue
        text = open(os.path.join(PROFILES, name)).read()
        assert "rocprofv3" in text and "bench.py" in text, name


def _counter_entries():
    p = os.path.join(PROFILES, "counters.json")
    return sorted(json.load(open(p)).items()) if os.path.exists(p) else []


@pytest.mark.parametrize("key,e", _counter_entries(), ids=[k for k, _ in _counter_entries()])
def test_counter_entry_follows_from_its_raw_counts(key, e):
    """The clock and matrix-unit busy share the benchmark quotes are what the
    raw counters of the entry give (8 XCDs, 256 CUs of 4 SIMDs)."""
    cyc = e["GRBM_GUI_ACTIVE"] / 8
    assert e["clock_ghz"] == pytest.approx(cyc / (e["duration_us"] * 1e3), rel=1e-9)
    assert e["mfma_busy_share"] == pytest.approx(e["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * 256 * 4), rel=1e-9)
    assert 0 < e["mfma_busy_share"] <= 1.0
    m = re.fullmatch(r"(gemm_\w+)@(\d+)x(\d+)m\d+", key)
    assert m, key
    assert re.search(rf"void {m.group(1)}\(", ssb.emit_source(int(m.group(2)), int(m.group(3)), "bf16")), key
    assert re.fullmatch(r"[0-9a-f]{16}", e["source_sha"])
