"""Plan compilation without a GPU (proj_compile_only): the modules a plan would
load compile for gfx950 through the parallel helper processes and in this
process alike, and a compilation failure comes back as PROJ_ECOMPILE with a
message naming the module -- never as a plan built from partial code."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(code: str, env_extra: dict) -> subprocess.CompletedProcess:
    env = dict(os.environ, **env_extra)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=600)


_PROBE = r"""
import ctypes, json
import shape_specialised_bf16_amd as ssb
lib = ssb._lib
out = {}
for arch in ("gfx950", "gfx9999"):
    sec = ctypes.c_double(0)
    rc = lib.proj_compile_only(1920, 1104, 0, 0, 0.0, arch.encode(), ctypes.byref(sec))
    out[arch] = [rc, lib.proj_last_error().decode(errors="replace")]
rc = lib.proj_compile_only(1024, 1001, 0, 0, 0.0, b"gfx950", None)
out["bad_k"] = [rc, lib.proj_last_error().decode(errors="replace")]
print(json.dumps(out))
"""


@pytest.mark.parametrize("jobs", ["8", "1"])
def test_compile_only_through_the_helpers(jobs):
    import json
    r = _run(_PROBE, {"PROJ_RTC_JOBS": jobs})
    assert r.returncode == 0, r.stderr
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["gfx950"] == [0, ""]
    rc, msg = out["gfx9999"]
    assert rc == -3, out                                   # PROJ_ECOMPILE
    assert "hipRTC compile of proj_1920x1104_f32_flags0" in msg and "module" in msg, msg
    assert "HIPRTC_ERROR" in msg, msg
    assert out["bad_k"][0] == -1 and "invalid shape" in out["bad_k"][1]


def test_compile_only_in_process():
    """PROJ_RTC_JOBS=0: every module compiled by the hipRTC this process loaded
    (torch's, here), one after another."""
    code = ("import ctypes, shape_specialised_bf16_amd as ssb\n"
            "sec = ctypes.c_double(0)\n"
            "rc = ssb._lib.proj_compile_only(1920, 1104, 1, 0, 0.0, b'gfx950', ctypes.byref(sec))\n"
            "print(rc, ssb._lib.proj_last_error().decode())\n")
    r = _run(code, {"PROJ_RTC_JOBS": "0"})
    assert r.returncode == 0, r.stderr
    assert r.stdout.split()[0] == "0", r.stdout


def test_helper_is_built_beside_the_library():
    import shape_specialised_bf16_amd as ssb
    helper = os.path.join(os.path.dirname(ssb.LIB_PATH), "proj_rtc")
    assert os.access(helper, os.X_OK)
    r = subprocess.run([helper], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr
    r = subprocess.run([helper, "gfx950", "/nonexistent.hip", "/tmp/x.co"], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 2 and "cannot read" in r.stderr


def test_module_split_covers_every_candidate_once():
    """The modules together hold each candidate's wrapper exactly once and the
    support kernels exactly once (module 0)."""
    import re
    import shape_specialised_bf16_amd as ssb
    full = ssb.emit_source(2560, 9216, "bf16")
    names = re.findall(r'extern "C" __global__ __launch_bounds__\(\d+\) void (\w+)\(', full)
    assert len(names) == len(set(names)) and "gemm_plain" in names and "proj_check_bf16" in names
