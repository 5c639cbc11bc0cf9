"""The load-time gate's reject path, exercised on the CPU with planted outputs.

The tuner accepts a candidate only if its probe runs pass the gate ("#004 the
same compiler on Apple's chips", section "The night the engine chose wrong").
On the GPU every candidate of every tested shape passes, so the reject path is
shown here instead: the gate's check and hash kernels (gate.hip, with
device_common.hip) are compiled for the host -- one "thread" walking the whole
output -- together with the host decision (gate_rule.h, the function the tuner
calls), and fed outputs with planted mistakes: an element two bf16 steps off, an
f32 element just outside the tolerance, one f32 step off on the integer probe, a
sentinel left in row M-1, a written guard row, an integer-probe output that
differs from the plain kernel's only outside the sampled rows (one changed
element, two swapped elements).  Each must be rejected with the "[autotune] ...
never picked" line; exact outputs and the allowed one-step bf16 difference must
pass.  A second set of tests removes or loosens one clause of the gate at a time
and checks that some planted mistake then gets through.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "shape_specialised_bf16_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"

SHIM = r"""
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>
// HIP spellings for a host build: one thread walks every grid-stride loop.
#define __device__
#define __forceinline__ inline
#define __global__
#define __launch_bounds__(...)
struct Dim3 { unsigned x, y, z; };
static const Dim3 blockIdx = {0, 0, 0}, threadIdx = {0, 0, 0}, blockDim = {1, 1, 1}, gridDim = {1, 1, 1};
template <class T> static T atomicAdd(T* p, T v) { T o = *p; *p = o + v; return o; }
static unsigned atomicMax(unsigned* p, unsigned v) { unsigned o = *p; if (v > o) *p = v; return o; }
static float __shfl_xor(float v, int) { return v; }
static void __syncthreads() {}
constexpr long N = %(N)d;
constexpr long K = %(K)d;
constexpr long NOUT = N;
constexpr int EPI = 0;
constexpr int OUT_SEL = %(OUT)d;
"""

MAIN = r"""
#include "gate_rule.h"
namespace {
constexpr int M = 5, GUARD = 3;
const int listed[] = {0, 2, 4};                 // the reference rows of the probe
constexpr int NR = 3;
std::vector<float> ref(NR * N);

u32 f2u(float f) { u32 u; memcpy(&u, &f, 4); return u; }
float u2f(u32 u) { float f; memcpy(&f, &u, 4); return f; }

struct Out {
    std::vector<u32> f;   // f32 output bits
    std::vector<u16> b;   // bf16 output bits
};

// The correct output: listed rows from the reference, other rows a value of
// their own (what the plain kernel wrote there), guard rows the sentinel.
Out exact(bool integer) {
    Out o;
    o.f.assign((M + GUARD) * N, SENTINEL_F32);
    o.b.assign((M + GUARD) * N, SENTINEL_BF16);
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            float v = integer ? (float)((m * 7 + n * 3) %% 9 - 4) * 13.0f : 0.37f * (float)(n - 31) + (float)m;
            for (int j = 0; j < NR; ++j) if (listed[j] == m) v = ref[j * N + n];
            o.f[m * N + n] = f2u(v);
            o.b[m * N + n] = dev::to_bf16(v);
        }
    return o;
}

std::string run(const Out& o, bool integer, bool have_base, uint64_t base) {
    CheckStats st;
    memset(&st, 0, sizeof st);
    const void* y = OUT_SEL == OUT_BF16 ? (const void*)o.b.data() : (const void*)o.f.data();
    if (OUT_SEL == OUT_BF16) proj_check_bf16(y, M + GUARD, M, ref.data(), listed, NR, integer ? 1 : 0, &st);
    else proj_check_f32(y, M + GUARD, M, ref.data(), listed, NR, integer ? 1 : 0, &st);
    if (integer) proj_hash_out(y, (long)M * NOUT, &st);
    proj::CheckStats hs;
    static_assert(sizeof hs == sizeof st, "host and device CheckStats differ");
    memcpy(&hs, &st, sizeof hs);
    return proj::gate_reject_line(hs, integer, have_base, base, N, K, 8, "planted", M);
}

uint64_t hash_of(const Out& o) {
    CheckStats st;
    memset(&st, 0, sizeof st);
    const void* y = OUT_SEL == OUT_BF16 ? (const void*)o.b.data() : (const void*)o.f.data();
    proj_hash_out(y, (long)M * NOUT, &st);
    return st.hash;
}

int failures = 0;
void expect(const char* name, const std::string& line, bool reject) {
    const bool rejected = !line.empty();
    const bool wellformed = !rejected || (line.find("[autotune] proj") == 0 && line.find("never picked: planted") != std::string::npos);
    if (rejected != reject || !wellformed) {
        printf("FAIL %%s: %%s\n", name, rejected ? line.c_str() : "passed the gate");
        ++failures;
    } else {
        printf("ok %%s: %%s\n", name, rejected ? line.c_str() : "passed");
    }
}
}  // namespace

int main() {
    for (int j = 0; j < NR; ++j)
        for (int n = 0; n < N; ++n) ref[j * N + n] = 0.731f * (float)(n - 30) + 5.0f * (float)j + 0.1f;
    std::vector<float> iref(ref);
    // random probe
    {
        Out o = exact(false);
        expect("exact output", run(o, false, false, 0), false);
        const int e = 2 * N + 17;                      // a listed element (row 2)
        const float r = ref[1 * N + 17];
        if (OUT_SEL == OUT_BF16) {
            Out a = o, b = o;
            a.b[e] = (u16)(o.b[e] + 2);                // two bf16 steps away
            b.b[e] = (u16)(o.b[e] + 1);                // one step: allowed
            expect("bf16 two steps off in a listed row", run(a, false, false, 0), true);
            expect("bf16 one step off in a listed row", run(b, false, false, 0), false);
        } else {
            Out a = o, b = o;
            a.f[e] = f2u(r + 1.5e-3f * (std::fabs(r) + 1.f));
            b.f[e] = f2u(r + 0.5e-3f * (std::fabs(r) + 1.f));
            expect("f32 outside the tolerance in a listed row", run(a, false, false, 0), true);
            expect("f32 inside the tolerance in a listed row", run(b, false, false, 0), false);
        }
        Out s = o;
        s.f[(M - 1) * N + N - 1] = SENTINEL_F32;       // last element of row M-1 never written
        s.b[(M - 1) * N + N - 1] = SENTINEL_BF16;
        expect("sentinel left in row M-1", run(s, false, false, 0), true);
        Out s2 = o;
        s2.f[1 * N + 5] = SENTINEL_F32;                // an unlisted row left unwritten
        s2.b[1 * N + 5] = SENTINEL_BF16;
        expect("sentinel left in an unlisted row", run(s2, false, false, 0), true);
        Out g = o;
        g.f[(M + 1) * N + 3] = f2u(1.0f);              // a guard row written
        g.b[(M + 1) * N + 3] = dev::to_bf16(1.0f);
        expect("guard row written", run(g, false, false, 0), true);
    }
    // integer probe: bit equality and the whole-output hash against the plain kernel's
    {
        for (int j = 0; j < NR; ++j)
            for (int n = 0; n < N; ++n) ref[j * N + n] = (float)((listed[j] * 7 + n * 3) %% 9 - 4) * 13.0f;
        Out o = exact(true);
        const uint64_t base = hash_of(o);
        expect("exact integer output", run(o, true, true, base), false);
        Out a = o;
        if (OUT_SEL == OUT_BF16) a.b[4 * N + 9] = (u16)(o.b[4 * N + 9] + 1);
        else a.f[4 * N + 9] = o.f[4 * N + 9] + 1;      // one step off in a listed row
        expect("integer probe one step off in a listed row", run(a, true, true, base), true);
        expect("the same without the plain kernel's hash", run(a, true, false, 0), true);
        Out h = o;                                     // differs only in row 3 (not listed)
        if (OUT_SEL == OUT_BF16) h.b[3 * N + 40] = dev::to_bf16(u2f((u32)dev::to_bf16(u2f(o.f[3 * N + 40])) << 16) + 13.0f);
        else h.f[3 * N + 40] = f2u(u2f(o.f[3 * N + 40]) + 13.0f);
        expect("integer probe differing outside the listed rows", run(h, true, true, base), true);
        expect("differing outside the listed rows, without the plain kernel's hash", run(h, true, false, 0), false);
        Out w = o;                                     // two unlisted elements swapped
        std::swap(w.f[1 * N + 2], w.f[3 * N + 7]);
        std::swap(w.b[1 * N + 2], w.b[3 * N + 7]);
        if (w.f[1 * N + 2] == o.f[1 * N + 2]) { printf("FAIL setup: swapped values are equal\n"); return 1; }
        expect("integer probe with two unlisted elements swapped", run(w, true, true, base), true);
    }
    (void)iref;
    printf(failures ? "FAILED %%d\n" : "ALL OK\n", failures);
    return failures ? 1 : 0;
}
"""


def _build_and_run(d, out_sel: int, mutate=None):
    common = open(os.path.join(CSRC, "device_common.hip")).read()
    gate = open(os.path.join(CSRC, "gate.hip")).read()
    rule = open(os.path.join(CSRC, "gate_rule.h")).read()
    if mutate:
        which, old, new = mutate
        texts = {"gate.hip": gate, "gate_rule.h": rule}
        assert old in texts[which], f"planted mistake not applicable: {old!r}"
        texts[which] = texts[which].replace(old, new)
        gate, rule = texts["gate.hip"], texts["gate_rule.h"]
    (d / "gate_rule.h").write_text(rule)
    src = d / "gate_host.cpp"
    src.write_text(SHIM % {"N": 64, "K": 32, "OUT": out_sel} + common + "\n" + gate + "\n" + MAIN % {})
    exe = d / "gate_host"
    r = subprocess.run([CLANG, "-std=c++17", "-O1", "-w", f"-I{d}", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)


@pytest.fixture(autouse=True)
def _clang():
    if not os.path.exists(CLANG):
        pytest.skip("clang++ not available")


@pytest.mark.parametrize("out_sel", [0, 1], ids=["f32", "bf16"])
def test_gate_rejects_every_planted_mistake_and_passes_exact_outputs(tmp_path, out_sel):
    r = _build_and_run(tmp_path, out_sel)
    assert r.returncode == 0 and "ALL OK" in r.stdout, r.stdout + r.stderr
    rejected = [l for l in r.stdout.splitlines() if "never picked" in l]
    assert len(rejected) >= 7, r.stdout


# One clause of the gate removed or loosened at a time: some planted mistake
# must then pass the gate, so the test above would notice the change.
MUTATIONS = [
    ("gate_rule.h", "cs.bad || ", ""),
    ("gate_rule.h", "cs.unwritten || ", ""),
    ("gate_rule.h", "cs.guard || ", ""),
    ("gate_rule.h", "integer && have_base && cs.hash != base_hash", "false"),
    ("gate.hip", "if (row < M) unw += sent ? 1u : 0u;", "if (row < M - 1) unw += sent ? 1u : 0u;"),
    ("gate.hip", "else grd += sent ? 0u : 1u;", "else grd += 0u;"),
    ("gate.hip", "ok = err <= 1e-3f * (__builtin_fabsf(r) + 1.f);", "ok = err <= 2e-3f * (__builtin_fabsf(r) + 1.f);"),
    ("gate.hip", "(__builtin_fabsf(y - R) <= bf16_spacing(R))", "(__builtin_fabsf(y - R) <= 2.f * bf16_spacing(R))"),
    ("gate.hip", "h += mix64(((u64)i << 32) ^ v ^ 0x9E3779B97F4A7C15ull);", "h += mix64(v ^ 0x9E3779B97F4A7C15ull);"),
    ("gate.hip", "if constexpr (OUT == OUT_F32) ok = __builtin_bit_cast(u32, y) == __builtin_bit_cast(u32, r);",
     "if constexpr (OUT == OUT_F32) ok = __builtin_fabsf(y - r) <= 1e-6f * (__builtin_fabsf(r) + 1.f);"),
]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda m: m[2][:40] or ("drop " + m[1][:30]))
def test_a_weakened_gate_lets_a_planted_mistake_through(tmp_path, mutation):
    results = [_build_and_run(tmp_path, out_sel, mutation) for out_sel in (0, 1)]
    assert any(r.returncode != 0 and "FAIL" in r.stdout for r in results), \
        "\n".join(r.stdout for r in results)
