"""The library's host code built with AddressSanitizer and UndefinedBehaviorSanitizer
(g++, no device code) and driven on the CPU: candidate enumeration and source
emission for many shapes and every combination of plan options, the module
split, the C entry points' argument checks, a compilation (in process: the helper is
looked up beside the binary holding the library code), the tuning-cache file reader and writer (round trip, corrupt and
hostile files) and the ELF check that guards the compiled-module cache.  Any
sanitizer report fails the run (-fno-sanitize-recover)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "shape_specialised_bf16_amd", "csrc")
BUILD = os.path.join(ROOT, "shape_specialised_bf16_amd", "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

DRIVER = r"""
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <random>
#include <string>
#include <vector>
#include "proj.h"
#include "proj_internal.h"

// the static device scratch is device code (scratch.hip); the host build stands it in
namespace proj {
size_t scratch_capacity() { return 0; }
int scratch_address(int, void** p) { *p = nullptr; return PROJ_EINVAL; }
}

static int fails = 0;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

static std::string slurp(const std::string& p) { std::ifstream f(p); return std::string(std::istreambuf_iterator<char>(f), {}); }

int main(int argc, char** argv) {
    const std::string dir = argv[1];
    // 1. enumeration, emission and the module split for many shapes and options
    const long shapes[][2] = {{1, 8}, {7, 8}, {64, 64}, {1000, 520}, {1920, 1104}, {7168, 1024}, {2560, 9216},
                              {18432, 2560}, {5120, 17408}, {151936, 1024}, {34816, 5120}, {128, 64}, {256, 1024}};
    size_t total = 0;
    for (auto& sh : shapes)
        for (int fusion = 0; fusion < 8; ++fusion) {
            if ((fusion & 1) && sh[0] % 2) continue;
            if ((fusion & 4) && (sh[0] % 128 || sh[1] % 64)) continue;
            for (int cus : {256, 304, 80}) {
                std::vector<proj::Candidate> c = proj::enumerate_candidates(sh[0], sh[1], cus, fusion);
                CHECK(!c.empty() && c.back().fam == proj::Family::Plain);
                for (const auto& x : c) {
                    CHECK(x.max_m >= 1);
                    for (long M : {1L, 16L, 17L, 512L, 8191L, 8192L}) total += x.ws_bytes(M, sh[0]) > 0;
                    (void)x.ws_bound(8192, sh[0]);
                }
                for (int dtype = 0; dtype < 2; ++dtype) {
                    std::string src = proj::emit_source(sh[0], sh[1], dtype, "gfx950", cus, c, fusion, 1e-6f);
                    std::vector<std::string> mods = proj::emit_module_sources(sh[0], sh[1], dtype, "gfx950", cus, c,
                                                                              fusion, 1e-6f, proj::kMaxModules);
                    CHECK(!mods.empty() && (int)mods.size() <= proj::kMaxModules);
                    for (const auto& x : c) CHECK(x.module >= 0 && x.module < (int)mods.size());
                    total += src.size();
                }
            }
        }
    for (long M = 1; M <= 20000; M += 7) CHECK(proj::bucket_of(M) >= 0 && proj::bucket_of(M) < proj::kNumBuckets);
    // 2. the C entry points' argument checks (no device call is reached)
    size_t need = 0;
    CHECK(proj_emit_source_ex(128, 64, 0, 7, 1e-6f, "gfx950", nullptr, 0, &need) == PROJ_OK && need > 1000);
    std::vector<char> buf(need);
    CHECK(proj_emit_source_ex(128, 64, 0, 7, 1e-6f, "gfx950", buf.data(), buf.size(), nullptr) == PROJ_OK);
    CHECK(proj_emit_source_ex(128, 64, 0, 7, 1e-6f, "gfx950", buf.data(), 5, nullptr) == PROJ_EINVAL);
    CHECK(proj_emit_source_ex(64, 64, 0, 7, 1e-6f, "gfx950", nullptr, 0, &need) == PROJ_EINVAL);   // packed: N % 128
    CHECK(proj_emit_source_ex(64, 60, 0, 0, 0.f, "gfx950", nullptr, 0, &need) == PROJ_EINVAL);
    CHECK(proj_emit_source_ex(65, 64, 0, 1, 0.f, "gfx950", nullptr, 0, &need) == PROJ_EINVAL);
    CHECK(proj_emit_source_ex(64, 64, 0, 64, 0.f, "gfx950", nullptr, 0, &need) == PROJ_EINVAL);
    CHECK(proj_emit_source_ex(64, 64, 3, 0, 0.f, nullptr, nullptr, 0, &need) == PROJ_EINVAL);
    CHECK(proj_plan_create_ex(0, 64, 0, 0, 0.f) == nullptr);
    CHECK(proj_plan_create_ex(64, 64, 0, 2, -1.f) == nullptr);
    CHECK(proj_run(nullptr, nullptr, nullptr, nullptr, 1, nullptr) == PROJ_EINVAL);
    CHECK(proj_run_noalloc(nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr) == PROJ_EINVAL);
    CHECK(proj_swiglu((void*)0x100000, (void*)0x100040, 4, 8, 0, nullptr) == PROJ_EINVAL);
    CHECK(proj_round_bf16((const float*)0x100000, (uint16_t*)0x100020, 16, nullptr) == PROJ_EINVAL);
    proj_plan_destroy(nullptr);
    {   // proj_run's size and overlap checks on a plan built here (they come before any device call)
        proj_plan q;
        q.N = 5120; q.NO = 5120; q.K = 17408; q.dtype = 0;
        char* const base = (char*)(uintptr_t(1) << 40);
        CHECK(proj_run(&q, base, base + (1 << 30), base + (2 << 30), int64_t(1) << 60, nullptr) == PROJ_EINVAL);
        CHECK(std::strstr(proj_last_error(), "2^48") != nullptr);
        // the largest M the bound allows for K = 17408 is 2^48 / (4 K) = 4042322160
        CHECK(proj_run(&q, base, base + (1 << 30), base + (2 << 30), 4042322161LL, nullptr) == PROJ_EINVAL);
        CHECK(std::strstr(proj_last_error(), "2^48") != nullptr);
        CHECK(proj_run(&q, base, base + (1 << 30), base + (2 << 30), 4042322160LL, nullptr) == PROJ_EINVAL);
        CHECK(std::strstr(proj_last_error(), "overlaps") != nullptr);    // past the bound check, X reaches W
        CHECK(proj_run(&q, base, base + (1 << 30), base + 4096, 4, nullptr) == PROJ_EINVAL);   // Y inside X
        CHECK(std::strstr(proj_last_error(), "overlaps") != nullptr);
        // separate buffers pass every argument check; what follows is the device lookup
        (void)proj_run(&q, base, base + (1 << 30), base + (2 << 30), 4, nullptr);
        CHECK(std::strstr(proj_last_error(), "2^48") == nullptr && std::strstr(proj_last_error(), "overlaps") == nullptr);
    }
    // 3. one plan's modules compiled (the helper is looked up beside the binary
    //    that holds the library code -- this driver -- so here in this process)
    double sec = 0;
    CHECK(proj_compile_only(1920, 1104, 1, 0, 0.f, "gfx950", &sec) == PROJ_OK);
    CHECK(proj_compile_only(1920, 1104, 1, 0, 0.f, "gfx9999", &sec) == PROJ_ECOMPILE);
    CHECK(std::strstr(proj_last_error(), "module") != nullptr);
    // 4. the ELF check: real code object, truncations, corrupt headers, random bytes
    {
        std::string co = slurp(argv[2]);
        std::vector<char> v(co.begin(), co.end());
        CHECK(proj::whole_elf64(v));
        std::mt19937 rng(7);
        for (size_t cut : {(size_t)0, (size_t)1, (size_t)63, (size_t)64, v.size() / 2, v.size() - 1}) {
            std::vector<char> t(v.begin(), v.begin() + std::min(cut, v.size()));
            (void)proj::whole_elf64(t);
        }
        for (int i = 0; i < 2000; ++i) {
            std::vector<char> t = v;
            for (int k = 0; k < 8; ++k) t[rng() % 64] = (char)rng();
            (void)proj::whole_elf64(t);
            std::vector<char> r(rng() % 200);
            for (char& ch : r) ch = (char)rng();
            if (r.size() >= 5) std::memcpy(r.data(), "\x7f" "ELF\x02", 5);
            (void)proj::whole_elf64(r);
        }
    }
    // 5. the tuning cache: round trip, then corrupt and hostile files
    {
        proj_plan p;
        p.N = 2560; p.K = 9216; p.dtype = 1; p.arch = "gfx950";
        p.cands = proj::enumerate_candidates(p.N, p.K, 256, 0);
        for (int b = 0; b < proj::kNumBuckets; ++b) { p.choice[b] = b % 3 == 2 ? -1 : b % (int)p.cands.size(); p.choice_us[b] = 1.5 * b; }
        p.cache_path = dir + "/proj-cache.txt";
        proj::cache_write(&p);
        std::vector<std::string> names;
        CHECK(proj::cache_read(p.cache_path, &names));
        CHECK((int)names.size() == proj::kNumBuckets);
        for (int b = 0; b < proj::kNumBuckets; ++b)
            CHECK(names[b] == (p.choice[b] >= 0 ? p.cands[p.choice[b]].name : std::string()));
        CHECK(!proj::cache_read(dir + "/no-such-file.txt", &names));
        const std::string bad[] = {"", "not a cache\n", "libproj tuning cache 1\nbucket 99 x\nbucket -1 y\n",
                                   "libproj tuning cache 1\nbucket 2 " + std::string(5000, 'a') + "\n",
                                   "libproj tuning cache 1\nbucket 3\nbucket\n\n\nbucket 1 ok extra words\n",
                                   std::string("libproj tuning cache 1\n\0\0\0bucket 0 \xff\xfe\n", 38)};
        int i = 0;
        for (const std::string& text : bad) {
            const std::string f = dir + "/bad" + std::to_string(i++) + ".txt";
            std::ofstream(f, std::ios::binary) << text;
            std::vector<std::string> nm;
            if (proj::cache_read(f, &nm)) {
                CHECK((int)nm.size() == proj::kNumBuckets);
                for (const auto& n : nm) CHECK(n.size() < 160);
            }
        }
        p.cache_path = dir + "/no-such-dir/x.txt";     // unwritable: ignored
        proj::cache_write(&p);
    }
    std::printf(fails ? "FAILED %d\n" : "ok %zu\n", fails ? (size_t)fails : total);
    return fails ? 1 : 0;
}
"""


@pytest.fixture(autouse=True)
def _tools():
    if not shutil.which("g++") or not os.path.exists(os.path.join(ROCM, "include", "hip", "hiprtc.h")):
        pytest.skip("g++ or the ROCm headers not available")


def test_host_code_under_asan_and_ubsan(tmp_path):
    import shape_specialised_bf16_amd as ssb
    emb = os.path.join(BUILD, "embedded_sources.cpp")
    assert os.path.exists(emb), "build the library first (embeds the device sources)"
    drv = tmp_path / "driver.cpp"
    drv.write_text(DRIVER)
    exe = tmp_path / "driver"
    srcs = [os.path.join(CSRC, f) for f in ("codegen.cpp", "plan.cpp", "api.cpp", "rtc.cpp")] + [emb, str(drv)]
    r = subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}",
                        f"-I{CSRC}", f"-I{os.path.join(ROCM, 'include')}", *srcs, "-o", str(exe),
                        f"-L{os.path.join(ROCM, 'lib')}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-lamdhip64",
                        "-lhiprtc", "-pthread"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    # a real code object for the ELF check, made by the helper built beside the library
    co = tmp_path / "k.co"
    hip = tmp_path / "k.hip"
    hip.write_text('extern "C" __global__ void k(float* p) { p[threadIdx.x] = 1.f; }\n')
    helper = os.path.join(os.path.dirname(ssb.LIB_PATH), "proj_rtc")
    r = subprocess.run([helper, "gfx950", str(hip), str(co)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe), str(tmp_path), str(co)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and r.stdout.strip().splitlines()[-1].startswith("ok"), \
        (r.stdout[-3000:] + r.stderr[-6000:])
