"""The in-kernel clock probe used by the benchmark (CPU only: source and grid).

The probe copy of a GEMM candidate must hold exactly that candidate's template
call, with the counter readings around it, in a unit that the library's
compile helper builds; its grid must be the plan's grid for that candidate.
"""
import os
import re
import subprocess

import pytest

import shape_specialised_bf16_amd as ssb
from shape_specialised_bf16_amd import clock_probe

HELPER = os.path.join(os.path.dirname(ssb.__file__), "proj_rtc")


def test_probe_source_wraps_the_candidates_own_call(tmp_path):
    name = "gemm_256x192x64_st2_w4x2_sw1_g8_sk1_b3"
    full = ssb.emit_source(18432, 2560, "bf16")
    call = re.search(r"void " + name + r"\(.*?\n\{ (gemm_mfma<[^;]*;) \}", full).group(1)
    src = clock_probe.probe_source(full, name)
    body = src[src.index('void clk_probe('):]
    assert body.count(call) == 1
    # readings before and after the call, the GEMM itself unchanged
    assert body.index("s_memtime") < body.index(call) < body.rindex("s_memtime")
    assert body.index("s_memrealtime") < body.index(call) < body.rindex("s_memrealtime")
    # no other candidate wrapper is compiled into the probe
    assert not re.search(r"^// (gemv|gemm)_\w+: ", src, re.M)
    assert src.count("__global__") == full[:full.index("// gemv_")].count("__global__") + 1
    if not os.access(HELPER, os.X_OK):
        pytest.skip("proj_rtc not built")
    sp, cp = tmp_path / "p.hip", tmp_path / "p.co"
    sp.write_text(src)
    r = subprocess.run([HELPER, "gfx950", str(sp), str(cp)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    assert cp.stat().st_size > 0


def test_probe_grid_is_the_plans_grid():
    # whole 256 x 256 tiles: ceil(M / 256) x N / 256 workgroups of 8 waves
    assert clock_probe.geometry("gemm_256x256x64_st2_w2x4_sw1_g8_sk1_b3", 34816, 8192) == (32 * 136, 512)
    assert clock_probe.geometry("gemm_256x192x64_st2_w4x2_sw1_g8_sk1_b3", 18432, 2047) == (8 * 96, 512)
    assert clock_probe.geometry("gemm_128x64x64_st3_w2x2_sw1_g8_sk1_b4", 2560, 128) == (40, 256)
    # split-K, split tail and GEMV candidates are not covered
    for name in ("gemm_128x128x64_st2_w2x2_sw1_g8_sk2", "gemm_256x256x64_st2_w2x4_sw1_g8_sk1_b3_tail2_r256",
                 "gemv_valu_r2_s1_m1_u2_nt1", "gemm_plain"):
        assert clock_probe.geometry(name, 5120, 512) is None


def test_unknown_candidate_is_refused():
    with pytest.raises(ValueError):
        clock_probe.probe_source(ssb.emit_source(5120, 2560, "bf16"), "gemm_999x999x64_st2_w2x4_sw1_g8_sk1")
