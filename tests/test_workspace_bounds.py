"""Workspace and launch sizing of the split GEMM and split GEMV candidates, checked on the CPU.

A plan allocates one workspace at creation, sized by Candidate::ws_bound over
the largest block (8192 rows), and every launch writes split-K or split-tail
partials into it.  A launch at any smaller M must therefore need no more than
that bound, or it would write past the allocation.  The device side of the
same arithmetic -- the partial index of a split-tail piece, ws[piece][BM*BN],
with piece < rem * TAILS, and the split-K layout ws[z][M][N] -- fixes what a
launch needs, so this test recomputes that need from the grid the host
launches (the device's own tail split) and checks it against ws_bytes and
ws_bound for every candidate the generator enumerates, over every M up to
8192.  The candidates come from the library's own enumerate_candidates,
compiled for the host with hipcc together with codegen.cpp.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "shape_specialised_bf16_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

PROGRAM = r"""
#include <cstdio>
#include "proj_internal.h"
// the device sources are not needed to enumerate candidates
namespace proj {
const char* const kDeviceCommonSrc = "";
const char* const kKernelsHeadSrc = "";
const char* const kGemvSrc = "";
const char* const kGemmSrc = "";
const char* const kGateSrc = "";
const char* const kSupportSrc = "";
}
using namespace proj;

int main() {
    const long shapes[][2] = {{2048, 1024}, {151936, 1024}, {5120, 2560}, {2560, 4096}, {18432, 2560},
                              {2560, 9216}, {10240, 5120}, {5120, 8192}, {34816, 5120}, {5120, 17408},
                              {7168, 1024}, {1000, 520}, {1920, 1104}, {151936, 2560}};
    long checked = 0;
    for (auto& sh : shapes)
        for (int fusion : {0, 1, 4}) {
            const long N = sh[0], K = sh[1];
            if ((fusion & 1) && N % 2) continue;
            if ((fusion & 4) && (N % 128 || K % 64)) continue;
            for (const Candidate& c : enumerate_candidates(N, K, 256, fusion)) {
                if (!c.needs_ws()) continue;
                const size_t bound = c.ws_bound(kMaxBlockRows, N);
                for (long M = 1; M <= c.max_m; ++M) {
                    // what the launch at M writes, from the grid the host launches
                    size_t need;
                    if (c.fam == Family::GemvValu) {
                        // K split across KX workgroups: partials ws[x][n], one row of Y (M = 1)
                        need = (size_t)c.KX * M * N * sizeof(float);
                        if (c.KX < 2 || c.max_m != 1 || N % 4 || c.reduce_name.empty()) {
                            std::printf("FAIL split GEMV %s\n", c.name.c_str());
                            return 1;
                        }
                    } else if (c.SK > 1) {
                        need = (size_t)c.SK * M * N * sizeof(float);          // ws[z][M][N]
                    } else {
                        int64_t T, nf, rem;
                        c.tail_split(M, N, &T, &nf, &rem);
                        const long tiles_m = (M + c.BM - 1) / c.BM;
                        if (T != tiles_m * (N / c.BN) || nf + rem != T) {
                            std::printf("FAIL split %s M=%ld\n", c.name.c_str(), M);
                            return 1;
                        }
                        need = (size_t)rem * c.TAILS * c.BM * c.BN * sizeof(float);   // ws[piece][BM*BN]
                    }
                    if (need > c.ws_bytes(M, N) || c.ws_bytes(M, N) > bound) {
                        std::printf("FAIL %s N=%ld K=%ld M=%ld need %zu ws_bytes %zu bound %zu\n", c.name.c_str(),
                                    N, K, M, need, c.ws_bytes(M, N), bound);
                        return 1;
                    }
                    ++checked;
                }
            }
        }
    std::printf("ok %ld\n", checked);
    return 0;
}
"""


@pytest.fixture(autouse=True)
def _hipcc():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")


def _run(tmp_path, header_edit=None):
    """Build and run the check; header_edit(text) plants a mistake in the
    sizing functions as the check program sees them (codegen.cpp still
    enumerates with the real header)."""
    inc = CSRC
    if header_edit:
        text = open(os.path.join(CSRC, "proj_internal.h")).read()
        changed = header_edit(text)
        assert changed != text, "the planted mistake did not apply"
        (tmp_path / "proj_internal.h").write_text(changed)
        inc = str(tmp_path)
    src = tmp_path / "ws_bounds.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "ws_bounds"
    subprocess.run([HIPCC, "--cuda-host-only", "-O2", "-std=c++17", f"-I{inc}", str(src),
                    os.path.join(CSRC, "codegen.cpp"), "-o", str(exe)], check=True, capture_output=True)
    return subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)


def test_every_split_launch_fits_the_workspace_bound(tmp_path):
    r = _run(tmp_path)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


@pytest.mark.parametrize("old,new", [
    ("return (size_t)KX * (size_t)M * (size_t)N * sizeof(float);",             # one split GEMV slice forgotten
     "return (size_t)(KX - 1) * (size_t)M * (size_t)N * sizeof(float);"),
    ("return (size_t)rem * TAILS * BM * BN * sizeof(float);",                  # a tail piece forgotten
     "return (size_t)rem * BM * BN * sizeof(float);"),
    ("return (size_t)std::min<int64_t>(T, ROUND) * TAILS * BM * BN * sizeof(float);",   # bound from half a round
     "return (size_t)std::min<int64_t>(T, ROUND / 2) * TAILS * BM * BN * sizeof(float);"),
])
def test_a_planted_sizing_mistake_is_caught(tmp_path, old, new):
    r = _run(tmp_path, lambda text: text.replace(old, new))
    assert r.returncode != 0 and "FAIL" in r.stdout, r.stdout
