// proj_internal.h -- host-side structures of libproj (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <memory>
#include <string>
#include <algorithm>
#include <vector>

namespace proj {

// Row buckets of the tuner: each bucket gets its own validated, timed choice.
// Every configured M in the workloads is a bucket's upper end.
struct BucketRange {
    int64_t lo, hi;
};
constexpr int kNumBuckets = 7;
constexpr BucketRange kBuckets[kNumBuckets] = {
    {1, 1}, {2, 16}, {17, 128}, {129, 512}, {513, 1024}, {1025, 2048}, {2049, 8192}};
constexpr int64_t kMaxBlockRows = 8192;  // proj_run splits larger M into blocks of this size

enum class Family { GemvValu, GemvMfma, Gemm, Plain };

struct Candidate {
    Family fam = Family::Plain;
    // GEMV parameters
    int R = 1, S = 1, MMAX = 1, U = 1, NT = 1;
    int NW = 4;      // waves per block of the vector GEMV (NW / S row groups)
    int KX = 1;      // >1: the vector GEMV's K split across KX workgroups (M = 1)
    int P = 0;       // 1: software-pipelined batches of U trips (vector GEMV, M = 1)
    int PRO = 0;     // 1: RMSNorm folded into the kernel (vector GEMV, M = 1)
    // SwiGLU plans: E = 1, the activation fused into the kernel's epilogue (Y has
    // N/2 columns); UF = 1, the kernel writes all N sums into the plan's
    // intermediate and the separate activation kernel produces Y
    int E = 0, UF = 0;
    // GEMM parameters: block tile, k-tile, LDS buffers, wave grid, split-K,
    // tile-row group, LDS swizzle period
    int BM = 0, BN = 0, BK = 64, ST = 2, WM = 0, WN = 0, SK = 1, GM = 8, SWZ = 0;
    int DMA = 1;  // 1: global->LDS copies; 0: copies staged through registers
    int BST = 0;  // ST + 1: W in one LDS buffer more than X (0: X and W share each buffer)
    int TAILS = 1;   // >1: whole tiles plus a tail split TAILS ways along K
    int ROUND = 0;   // workgroups the device runs at once (CU count x blocks per CU)
    int KP = 0;      // >1: each tile visits the k-tiles of every block of KP in its own rotated order

    int module = 0;            // index of the compiled module that holds it
    std::string name;          // extern "C" wrapper name in the generated module
    std::string reduce_name;   // split-K reduce kernel (empty if SK == 1)
    int threads = 256;
    int64_t max_m = kMaxBlockRows;
    hipFunction_t fn = nullptr;
    hipFunction_t reduce_fn = nullptr;

    // partials in the workspace, which a second kernel sums (split-K or
    // split-tail GEMM, GEMV split across workgroups)
    bool needs_ws() const { return (fam == Family::Gemm && (SK > 1 || TAILS > 1)) || (fam == Family::GemvValu && KX > 1); }
    // Tiles, whole tiles and split tail tiles of a launch at M rows (the same
    // split as tail_split() in the device code).
    void tail_split(int64_t M, int64_t N, int64_t* T, int64_t* n_full, int64_t* rem) const
    {
        *T = ((M + BM - 1) / BM) * (N / BN);
        *rem = *T >= ROUND ? *T % ROUND : *T;
        *n_full = *T - *rem;
    }
    size_t ws_bytes(int64_t M, int64_t N) const
    {
        if (fam == Family::GemvValu && KX > 1) return (size_t)KX * (size_t)M * (size_t)N * sizeof(float);
        if (fam != Family::Gemm) return 0;
        if (SK > 1) return (size_t)SK * (size_t)M * (size_t)N * sizeof(float);
        if (TAILS > 1) {
            int64_t T, nf, rem;
            tail_split(M, N, &T, &nf, &rem);
            return (size_t)rem * TAILS * BM * BN * sizeof(float);
        }
        return 0;
    }
    // Largest workspace any M up to max_rows (and up to the candidate's own
    // limit) can need.
    size_t ws_bound(int64_t max_rows, int64_t N) const
    {
        max_rows = std::min(max_rows, max_m);
        if (TAILS > 1) {
            const int64_t T = ((max_rows + BM - 1) / BM) * (N / BN);
            return (size_t)std::min<int64_t>(T, ROUND) * TAILS * BM * BN * sizeof(float);
        }
        return ws_bytes(max_rows, N);
    }
};

// Enumerate the candidates that tile (N, K) exactly.  Always ends with the
// plain kernel, which fits any shape.
// `cus` is the device's compute-unit count (it sets the tail split's round size).
// fusion: bit 0 the SwiGLU epilogue (the families that have it fused, then every
// plain candidate again run unfused, "_uf"), bit 1 the
// RMSNorm prologue (every candidate unfused, plus the M = 1 GEMVs with it folded in),
// bit 2 weights in the panel layout (every family reads it; N % 128 == 0, K % 64 == 0)
std::vector<Candidate> enumerate_candidates(int64_t N, int64_t K, int cus, int fusion = 0);

// The full translation unit for (N, K, dtype): prelude with the shape as
// literals, device helpers, kernel templates, one wrapper per candidate.
std::string emit_source(int64_t N, int64_t K, int dtype, const std::string& arch, int cus,
                        const std::vector<Candidate>& cands, int fusion = 0, float norm_eps = 0.f);

// The same translation unit cut into at most `max_modules` modules that hipRTC
// compiles independently (in parallel processes): each module holds the
// prelude and the wrappers of some candidates, module 0 also the support
// kernels.  Sets each candidate's `module`.  The cut depends only on the
// candidate list and max_modules.
std::vector<std::string> emit_module_sources(int64_t N, int64_t K, int dtype, const std::string& arch, int cus,
                                             std::vector<Candidate>& cands, int fusion, float norm_eps,
                                             int max_modules);
constexpr int kMaxModules = 16;

// Compile HIP sources for `arch` with hipRTC, one code object each, in up to
// PROJ_RTC_JOBS child processes (proj_rtc, beside libproj.so) when there are
// several, else in this process; code objects already compiled in this
// process are reused.  PROJ_ECOMPILE with hipRTC's log on failure.
int compile_sources(const std::vector<std::string>& srcs, const std::string& arch, const std::string& name,
                    std::vector<std::shared_ptr<std::vector<char>>>* codes);

// Compute units assumed when no device is queried (MI355X).
constexpr int kDefaultCUs = 256;

// Shape-independent support module (probe, rounding check).
std::string emit_support_source();

// Embedded device sources (generated from the .hip files at build time).
extern const char* const kDeviceCommonSrc;
extern const char* const kKernelsHeadSrc;
extern const char* const kGemvSrc;
extern const char* const kGemmSrc;
extern const char* const kGateSrc;
extern const char* const kSupportSrc;

// Bucket index for M >= 1 (M > kMaxBlockRows maps to the last bucket).
int bucket_of(int64_t M);

// Device memory a launch may use besides X, W and Y: the f32 partials of a
// split-K or split-tail GEMM (`ws`), the normalised rows of an unfused
// RMSNorm candidate (`xn`) and the N-column projection of an unfused SwiGLU
// candidate (`gu`).  Either the plan's own buffers, allocated when the plan
// is created, or pieces of the library's static scratch (proj_run_noalloc).
struct Workspace {
    float* ws = nullptr;
    size_t ws_bytes = 0;
    void* xn = nullptr;
    int64_t xn_rows = 0;
    void* gu = nullptr;
    int64_t gu_rows = 0;
};

// The persistent tuning cache (plan.cpp): whether a buffer holds a whole ELF64
// image (a code-object cache file is checked before it is loaded); the cached
// choice names per bucket ("" where absent, false if the file is not a cache
// file); the plan's choices written to its cache_path.
bool whole_elf64(const std::vector<char>& buf);
bool cache_read(const std::string& path, std::vector<std::string>* names);

// The static scratch (scratch.hip): its size, and its address on `device`
// (looked up once per device, with that device current).
size_t scratch_capacity();
int scratch_address(int device, void** ptr);

}  // namespace proj

struct proj_plan;
namespace proj {
void cache_write(proj_plan* p);
}

struct proj_plan {
    int64_t N = 0, K = 0;
    int dtype = 0;
    int epi = 0;        // PROJ_EPI_NONE or PROJ_EPI_SWIGLU
    int pro = 0;        // 1: RMSNorm prologue (proj_run_ex needs gamma)
    int wpack = 0;      // 1: W in the panel layout (proj_pack_weights; run with proj_run_packed)
    hipFunction_t f_pack = nullptr;  // the module's repacking kernel (proj_pack_panels)
    float eps = 0.f;    // its epsilon
    void* xn = nullptr; // workspace: normalised X rows for the unfused candidates (kMaxBlockRows x K bf16)
    void* gu = nullptr; // workspace: the N-column projection of the unfused SwiGLU candidates
    int64_t gu_rows = 0;             // rows it holds
    hipFunction_t f_swiglu = nullptr;  // the module's separate activation kernel (proj_swiglu_*)
    hipFunction_t f_norm = nullptr;  // the module's separate norm kernel (proj_rmsnorm_rows)
    uint64_t key = 0;   // tuning-cache key: device, runtime and driver versions, emitted source
    std::string cache;  // tuning cache: "off", "miss", "hit", "stale" (a cached choice failed the gate)
    std::string code_cache;  // compiled-module cache: "off", "miss", "hit", "stale" (the file did not load)
    std::string cache_path;
    int64_t NO = 0;     // columns of Y: N, or N/2 with the SwiGLU epilogue
    int device = -1;
    std::string arch;
    hipModule_t module = nullptr;          // modules[0]: the support kernels and some candidates
    std::vector<hipModule_t> modules;      // every compiled module of the plan
    std::vector<proj::Candidate> cands;
    int choice[proj::kNumBuckets];
    double choice_us[proj::kNumBuckets];
    std::vector<std::vector<std::pair<int, double>>> timings;  // per bucket: (cand, us)
    std::vector<std::vector<std::pair<int, std::string>>> rejected;  // per bucket: (cand, why)
    void* ws = nullptr;
    size_t ws_bytes = 0;
    double compile_s = 0, tune_s = 0;
    size_t code_bytes = 0;
    std::vector<std::string> log;
};
