"""The GEMM's k-tile order (KP > 1 candidates), compiled from its own source
and run on the CPU (no GPU).

A tile of a ``_kp`` candidate reads, at step t of its k loop, the k-tile
``ktile_order<KP>(t, kpb, ph)`` (csrc/gemm.hip): inside each whole block of KP
k-tiles the block rotated by the tile's phase ph = (tile-row + tile-column) mod
KP.  The sum over k must still take every k-tile of the tile's range exactly
once, and every copy must stay inside that range, so the order must be a
permutation of [0, nkt) for every phase and every k-tile count the shapes and
the split-tail pieces use.  The point of the order is that tiles sharing a
panel do not ask for the same k-tile first: within a block, the KP phases must
send the KP tiles to KP different k-tiles at every step.  The function's text
is taken from gemm.hip and compiled for the host with hipcc, as the tile-order
test does for the workgroup mapping.
"""
import os
import re
import shutil
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM = os.path.join(ROOT, "shape_specialised_bf16_amd", "csrc", "gemm.hip")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

PROGRAM = r"""
#include <cstdio>
#include <vector>
%(function)s

static int fail(const char* what, int kp, long nkt, long ph, long t) {
    std::printf("FAIL %%s KP=%%d nkt=%%ld ph=%%ld t=%%ld\n", what, kp, nkt, ph, t);
    return 1;
}

template <int KP> static int check(long nkt) {
    const long kpb = KP > 1 ? nkt - nkt %% KP : 0;
    for (long ph = 0; ph < (KP > 1 ? KP : 1); ++ph) {
        std::vector<int> seen(nkt, 0);
        for (long t = 0; t < nkt; ++t) {
            const long k = ktile_order<KP>(t, kpb, ph);
            if (k < 0 || k >= nkt) return fail("range", KP, nkt, ph, t);
            if (seen[k]++) return fail("twice", KP, nkt, ph, t);
            if (t >= kpb && k != t) return fail("trailing k-tile moved", KP, nkt, ph, t);
            if (t < kpb && k / KP != t / KP) return fail("left its block", KP, nkt, ph, t);
        }
    }
    // at every step of a whole block, the KP phases read KP different k-tiles
    for (long t = 0; t < kpb; ++t) {
        std::vector<int> seen(nkt, 0);
        for (long ph = 0; ph < KP; ++ph)
            if (seen[ktile_order<KP>(t, kpb, ph)]++) return fail("phases collide", KP, nkt, ph, t);
    }
    return 0;
}

int main() {
    long n = 0;
    for (long nkt = 1; nkt <= 400; ++nkt) {
        if (check<0>(nkt) || check<2>(nkt) || check<4>(nkt) || check<8>(nkt)) return 1;
        ++n;
    }
    std::printf("ok %%ld\n", n);
    return 0;
}
"""


def _function(src: str) -> str:
    m = re.search(r"template <int KP>\n__device__ __forceinline__ long ktile_order\(.*?\n}\n", src, re.S)
    assert m, "ktile_order not found in gemm.hip"
    return m.group(0).replace("__device__ __forceinline__", "static inline")


def _run(function: str, tmp_path) -> subprocess.CompletedProcess:
    cpp = tmp_path / "kto.cpp"
    cpp.write_text(PROGRAM % {"function": function})
    exe = tmp_path / "kto"
    r = subprocess.run([HIPCC, "-x", "c++", "--std=c++17", "-O1", str(cpp), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)


def test_ktile_order_is_a_permutation_for_every_phase(tmp_path):
    r = _run(_function(open(GEMM).read()), tmp_path)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout


def test_planted_mistakes_are_caught(tmp_path):
    """A rotation not folded back into its block, a phase that ignores the
    tile, and a permutation applied past the whole blocks must each fail."""
    f = _function(open(GEMM).read())
    good = "t = (t & ~(long)(KP - 1)) | ((t + ph) & (KP - 1));"
    assert good in f
    for bad in ("t = t + ph;",                                  # leaves the block / the range
                "t = (t & ~(long)(KP - 1)) | (t & (KP - 1));",  # every phase reads the same k-tile
                "t = (t & ~(long)(KP - 1)) | ((t + ph) & KP);"):   # a wrong mask: k-tiles lost and doubled
        r = _run(f.replace(good, bad), tmp_path)
        assert r.returncode != 0 and "FAIL" in r.stdout, bad
    r = _run(f.replace("if (t < kpb)", "if (true)"), tmp_path)    # the trailing k-tiles rotated too
    assert r.returncode != 0 and "FAIL" in r.stdout
