"""The GEMM's workgroup -> tile mapping, compiled from its own source and run
on the CPU (no GPU).

gemm_mfma (csrc/gemm.hip) maps workgroup ids to tiles in three steps: the
split of the T tiles into whole rounds and a tail (tail_split), a remap that
gives each of the 8 XCDs a contiguous range of tile ids (xcd_remap), and a
grouped row-major order over the tile grid (group_order).  Every output tile
must be computed exactly once, so each step must be a bijection onto its range.
The GPU parity tests see a few shapes; this test takes the three functions'
text from gemm.hip, compiles it for the host with hipcc, and checks the
bijections over many tile counts, grid shapes and group sizes -- and that the
host's copy of the split (Candidate::tail_split, used to size launches and
workspaces) agrees with the device's.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "shape_specialised_bf16_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _function(src: str, name: str) -> str:
    """The text of one helper of gemm_detail (template line included)."""
    m = re.search(r"(template <int GROUP_M>\n)?__device__ __forceinline__ \w+ " + name + r"\(.*?\n}\n", src, re.S)
    assert m, f"{name} not found in gemm.hip"
    return m.group(0).replace("__device__ __forceinline__", "static inline")


PROGRAM = r"""
#include <cstdio>
#include <cstdint>
#include <vector>
#include "proj_internal.h"
namespace gemm_detail {
%(functions)s
}
using namespace gemm_detail;

static int fail(const char* what, long a, long b, long c) {
    std::printf("FAIL %%s %%ld %%ld %%ld\n", what, a, b, c);
    return 1;
}

template <int G> static int check_group(long tiles_m, long tiles_n) {
    const long T = tiles_m * tiles_n;
    std::vector<int> seen(T, 0);
    for (long pid = 0; pid < T; ++pid) {
        long tm, tn;
        group_order<G>(pid, tiles_m, tiles_n, &tm, &tn);
        if (tm < 0 || tm >= tiles_m || tn < 0 || tn >= tiles_n) return fail("group_order range", G, tiles_m, pid);
        if (seen[tm * tiles_n + tn]++) return fail("group_order twice", G, tiles_m, pid);
    }
    return 0;
}

int main() {
    long checked = 0;
    for (long n = 0; n <= 5000; ++n) {                     // xcd_remap: a bijection on [0, n)
        std::vector<int> seen(n, 0);
        for (long p = 0; p < n; ++p) {
            const long t = xcd_remap(p, n);
            if (t < 0 || t >= n) return fail("xcd_remap range", n, p, t);
            if (seen[t]++) return fail("xcd_remap twice", n, p, t);
        }
        // consecutive ids of one XCD (p, p + 8) get consecutive tiles
        for (long p = 0; p + 8 < n; ++p)
            if (xcd_remap(p + 8, n) != xcd_remap(p, n) + 1) return fail("xcd_remap contiguity", n, p, 0);
        checked += n;
    }
    for (long tm = 1; tm <= 48; ++tm)                     // group_order: a bijection onto the grid
        for (long tn = 1; tn <= 160; tn += (tn < 16 ? 1 : 9)) {
            if (check_group<1>(tm, tn) || check_group<4>(tm, tn) || check_group<8>(tm, tn)) return 1;
            checked += 3 * tm * tn;
        }
    const long rounds[] = {1, 7, 256, 304, 512, 608};
    for (long round : rounds)                             // tail_split, device and host copies
        for (long T = 0; T <= 5000; ++T) {
            long nf, rem;
            tail_split(T, round, &nf, &rem);
            if (nf + rem != T || rem < 0 || nf < 0) return fail("tail_split sum", T, round, rem);
            if (T >= round ? (nf %% round != 0 || rem >= round) : (nf != 0 || rem != T))
                return fail("tail_split rounds", T, round, rem);
            proj::Candidate c;
            c.BM = 128; c.BN = 128; c.ROUND = (int)round;
            int64_t hT, hnf, hrem;
            const int64_t M = T * 128, N = 128;             // T tile-rows of one tile column
            c.tail_split(M, N, &hT, &hnf, &hrem);
            if (hT != T || hnf != nf || hrem != rem) return fail("host tail_split", T, round, hrem);
            ++checked;
        }
    std::printf("ok %%ld\n", checked);
    return 0;
}
"""


def _build(d, mutate=None):
    """Compile the check program for the host; mutate(text) plants a mistake in
    the helpers' text first (for the tests that show the check catches one)."""
    src = open(os.path.join(CSRC, "gemm.hip")).read()
    functions = "\n".join(_function(src, f) for f in ("tail_split", "group_order", "xcd_remap"))
    if mutate:
        changed = mutate(functions)
        assert changed != functions, "the planted mistake did not apply"
        functions = changed
    cpp = d / "tile_order.hip"
    cpp.write_text(PROGRAM % {"functions": functions})
    exe = d / "tile_order"
    subprocess.run([HIPCC, "--cuda-host-only", "-O2", "-std=c++17", f"-I{CSRC}", str(cpp), "-o", str(exe)],
                   check=True, capture_output=True)
    return subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)


@pytest.fixture(autouse=True)
def _hipcc():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")


def test_tile_order_helpers_are_bijections(tmp_path):
    r = _build(tmp_path)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


@pytest.mark.parametrize("old,new", [
    ("rem * (q + 1) + (xcd - rem) * q", "rem * q + (xcd - rem) * q"),       # xcd ranges overlap
    ("% gsz;", "% GROUP_M;"),                                              # short last group
    ("*rem = T >= round ? T % round : T;", "*rem = T > round ? T % round : T;"),   # exactly one round
])
def test_a_planted_mistake_is_caught(tmp_path, old, new):
    r = _build(tmp_path, lambda text: text.replace(old, new))
    assert r.returncode != 0 and "FAIL" in r.stdout, r.stdout


def test_extraction_finds_the_kernel_helpers():
    src = open(os.path.join(CSRC, "gemm.hip")).read()
    for name in ("tail_split", "group_order", "xcd_remap"):
        text = _function(src, name)
        assert "static inline" in text and name in text
