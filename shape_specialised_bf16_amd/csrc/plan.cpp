// plan.cpp -- plan creation (emit, hipRTC compile, load), the load-time tuner
// with its correctness gate, and run-time dispatch on M.
//
// The tuner follows "#004 the same compiler on Apple's chips" (blog series "On
// descend d'un cran"): at load time several variants of each kernel are
// measured per matrix shape and the fastest is kept (section "Catching up on
// prefill"), but a variant is first compared with a kernel known to be right,
// with the output cleared beforehand, at the bucket's whole block size and at
// a smaller row count, and a variant that disagrees is logged and never used
// (section "The night the engine chose wrong").  Here the trusted kernel is a
// plain one-thread-per-output reference that is itself checked against exact
// integer arithmetic on the host; the output is cleared to a NaN sentinel
// rather than zero, so an unwritten element cannot pass for a small value; and
// the acceptance rule is the elementwise tolerance of the numerical contract,
// with an integer probe that must match bit for bit.
#include <hip/hiprtc.h>
#include <dlfcn.h>
#include <fcntl.h>
#include <sched.h>
#include <spawn.h>
#include <sys/stat.h>
#include <sys/wait.h>
#include <unistd.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <iterator>
#include <map>
#include <memory>
#include <mutex>
#include <sstream>

#include "proj.h"
#include "gate_rule.h"
#include "proj_internal.h"
#include "rtc.h"

extern char** environ;

namespace proj {

// ---------------------------------------------------------------- errors
thread_local std::string g_last_error;

int set_error(int code, const char* f, ...) __attribute__((format(printf, 2, 3)));
int set_error(int code, const char* f, ...)
{
    char buf[2048];
    va_list ap;
    va_start(ap, f);
    vsnprintf(buf, sizeof buf, f, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

#define HIP_TRY(expr)                                                                         \
    do {                                                                                      \
        hipError_t e_ = (expr);                                                               \
        if (e_ != hipSuccess)                                                                 \
            return set_error(PROJ_EDEVICE, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_), \
                             __FILE__, __LINE__);                                             \
    } while (0)

static double now_s()
{
    return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

static int env_int(const char* name, int dflt)
{
    const char* v = getenv(name);
    return (v && *v) ? atoi(v) : dflt;
}

// ---------------------------------------------------------------- hipRTC
// Code objects compiled in this process, keyed by the full source text and
// architecture, so that two plans of the same shape compile once.
static std::mutex g_cache_mu;
static std::map<std::string, std::shared_ptr<std::vector<char>>> g_code_cache;

// The compile helper beside libproj.so ("" if it is not there).
static std::string helper_path()
{
    Dl_info info;
    if (!dladdr((void*)&helper_path, &info) || !info.dli_fname) return "";
    std::string lib = info.dli_fname;
    const size_t slash = lib.rfind('/');
    const std::string h = (slash == std::string::npos ? std::string(".") : lib.substr(0, slash)) + "/proj_rtc";
    return access(h.c_str(), X_OK) == 0 ? h : "";
}

// Compile helpers run at once: PROJ_RTC_JOBS, else the CPUs this process may
// run on, at most 16.  0: compile in this process.
static int rtc_jobs()
{
    if (const char* v = getenv("PROJ_RTC_JOBS"))
        if (*v) return std::max(0, atoi(v));
    cpu_set_t set;
    int n = 1;
    if (sched_getaffinity(0, sizeof set, &set) == 0) n = CPU_COUNT(&set);
    return std::max(1, std::min(16, n));
}

static std::string read_file(const std::string& path)
{
    std::ifstream f(path, std::ios::binary);
    return std::string((std::istreambuf_iterator<char>(f)), std::istreambuf_iterator<char>());
}

static int compile_error(const std::string& name, std::string log)
{
    if (log.size() > 1800) log = log.substr(0, 1800) + "...";
    return set_error(PROJ_ECOMPILE, "hipRTC compile of %s failed: %s", name.c_str(), log.c_str());
}

// The sources `todo` (indexes into srcs) compiled by proj_rtc child processes,
// at most `jobs` at a time, in a private temporary directory.  Returns
// PROJ_OK, PROJ_ECOMPILE, or 1 if the helpers could not be used at all (the
// caller then compiles in this process).
static int compile_in_children(const std::vector<std::string>& srcs, const std::vector<size_t>& todo,
                               const std::string& arch, const std::string& name, const std::string& helper,
                               int jobs, std::vector<std::shared_ptr<std::vector<char>>>* codes)
{
    const char* tmpdir = getenv("TMPDIR");
    std::string templ = std::string(tmpdir && *tmpdir ? tmpdir : "/tmp") + "/proj-rtc-XXXXXX";
    std::vector<char> dirbuf(templ.begin(), templ.end());
    dirbuf.push_back('\0');
    if (!mkdtemp(dirbuf.data())) return 1;
    const std::string dir = dirbuf.data();
    struct Job {
        size_t idx;
        std::string src, out, log;
        pid_t pid = -1;
    };
    std::vector<Job> js;
    for (size_t i = 0; i < todo.size(); ++i) {
        Job j;
        j.idx = todo[i];
        const std::string base = dir + "/" + name + ".m" + std::to_string(todo[i]);
        j.src = base + ".hip";
        j.out = base + ".co";
        j.log = base + ".log";
        js.push_back(j);
    }
    auto cleanup = [&]() {
        for (const Job& j : js) {
            std::remove(j.src.c_str());
            std::remove(j.out.c_str());
            std::remove(j.log.c_str());
            std::remove((j.out + ".tmp").c_str());
        }
        rmdir(dir.c_str());
    };
    for (Job& j : js) {
        std::ofstream f(j.src, std::ios::binary);
        if (!f || !f.write(srcs[j.idx].data(), (std::streamsize)srcs[j.idx].size())) {
            f.close();
            cleanup();
            return 1;
        }
    }
    // wait for one child (EINTR retried); true if it wrote its code object
    auto finish = [&](Job& j) -> bool {
        int status = 0;
        pid_t r;
        do r = waitpid(j.pid, &status, 0);
        while (r < 0 && errno == EINTR);
        const bool exited_ok = r == j.pid ? (WIFEXITED(status) && WEXITSTATUS(status) == 0) : true;
        j.pid = -1;
        return exited_ok && access(j.out.c_str(), R_OK) == 0;
    };
    int rc = PROJ_OK;
    bool spawn_failed = false;
    size_t next = 0, done = 0;
    std::vector<size_t> running;
    while (done < js.size()) {
        while (!spawn_failed && rc == PROJ_OK && next < js.size() && (int)running.size() < jobs) {
            Job& j = js[next];
            posix_spawn_file_actions_t fa;
            posix_spawn_file_actions_init(&fa);
            posix_spawn_file_actions_addopen(&fa, 1, j.log.c_str(), O_WRONLY | O_CREAT | O_TRUNC, 0600);
            posix_spawn_file_actions_adddup2(&fa, 1, 2);
            std::string a0 = helper, a1 = arch;
            char* argv[] = {&a0[0], &a1[0], &j.src[0], &j.out[0], nullptr};
            const int e = posix_spawn(&j.pid, helper.c_str(), &fa, nullptr, argv, environ);
            posix_spawn_file_actions_destroy(&fa);
            if (e != 0) {
                j.pid = -1;
                spawn_failed = true;
                break;
            }
            running.push_back(next++);
        }
        if (running.empty()) break;
        Job& j = js[running.front()];
        running.erase(running.begin());
        ++done;
        if (finish(j)) {
            const std::string co = read_file(j.out);
            (*codes)[j.idx] = std::make_shared<std::vector<char>>(co.begin(), co.end());
        } else if (rc == PROJ_OK) {
            rc = compile_error(name + " module " + std::to_string(j.idx), read_file(j.log));
        }
    }
    for (size_t r : running) finish(js[r]);
    cleanup();
    if (rc != PROJ_OK) return rc;
    // a spawn failure leaves some sources uncompiled: the caller compiles them here
    return spawn_failed ? 1 : PROJ_OK;
}

int compile_sources(const std::vector<std::string>& srcs, const std::string& arch, const std::string& name,
                    std::vector<std::shared_ptr<std::vector<char>>>* codes)
{
    codes->assign(srcs.size(), nullptr);
    std::vector<size_t> todo;
    {
        std::lock_guard<std::mutex> lk(g_cache_mu);
        for (size_t i = 0; i < srcs.size(); ++i) {
            auto it = g_code_cache.find(arch + "\n" + srcs[i]);
            if (it != g_code_cache.end()) (*codes)[i] = it->second;
            else todo.push_back(i);
        }
    }
    // The helper compiles with the hipRTC installed with ROCm; this process
    // may have bound another (the one of the framework that loaded libproj).
    // One compiler for every module: the helper whenever it is there.
    const int jobs = rtc_jobs();
    if (!todo.empty() && jobs > 0) {
        const std::string helper = helper_path();
        if (!helper.empty()) {
            const int rc = compile_in_children(srcs, todo, arch, name, helper, jobs, codes);
            if (rc < 0) return rc;
        }
    }
    for (size_t i : todo) {
        if ((*codes)[i]) continue;
        auto buf = std::make_shared<std::vector<char>>();
        std::string log;
        if (rtc_compile(srcs[i], arch, name, buf.get(), &log) != 0)
            return compile_error(srcs.size() > 1 ? name + " module " + std::to_string(i) : name, log);
        (*codes)[i] = buf;
    }
    std::lock_guard<std::mutex> lk(g_cache_mu);
    for (size_t i : todo) g_code_cache[arch + "\n" + srcs[i]] = (*codes)[i];
    return PROJ_OK;
}

int compile_source(const std::string& src, const std::string& arch, const char* name,
                   std::shared_ptr<std::vector<char>>* code)
{
    std::vector<std::shared_ptr<std::vector<char>>> codes;
    const int rc = compile_sources({src}, arch, name, &codes);
    if (rc == PROJ_OK) *code = codes[0];
    return rc;
}

int device_arch(int dev, std::string* arch, int* cus)
{
    hipDeviceProp_t p;
    HIP_TRY(hipGetDeviceProperties(&p, dev));
    std::string a = p.gcnArchName;
    const size_t colon = a.find(':');
    if (colon != std::string::npos) a = a.substr(0, colon);
    *arch = a;
    if (cus) *cus = p.multiProcessorCount;
    return PROJ_OK;
}

// ---------------------------------------------------------------- launching
struct LaunchGeom {
    unsigned gx, gy, threads;
};

static LaunchGeom geom(const Candidate& c, int64_t N, int64_t NO, int64_t M)
{
    switch (c.fam) {
    case Family::GemvValu: return {(unsigned)(N / (c.R * (c.NW / c.S))), (unsigned)c.KX, (unsigned)(64 * c.NW)};
    case Family::GemvMfma: return {(unsigned)(N / (16 * (4 / c.S))), 1u, 256u};
    case Family::Gemm: {
        if (c.TAILS > 1) {
            int64_t T, n_full, rem;
            c.tail_split(M, N, &T, &n_full, &rem);
            return {(unsigned)(n_full + rem * c.TAILS), 1u, (unsigned)c.threads};
        }
        const int64_t tm = (M + c.BM - 1) / c.BM;
        return {(unsigned)(tm * (N / c.BN)), (unsigned)c.SK, (unsigned)c.threads};
    }
    case Family::Plain:
    default: return {(unsigned)((M * (c.UF ? N : NO) + 255) / 256), 1u, 256u};
    }
}

// The plan's own workspace.
static Workspace plan_workspace(const proj_plan* p)
{
    Workspace w;
    w.ws = (float*)p->ws;
    w.ws_bytes = p->ws_bytes;
    w.xn = p->xn;
    w.xn_rows = p->xn ? kMaxBlockRows : 0;
    w.gu = p->gu;
    w.gu_rows = p->gu_rows;
    return w;
}

// Enqueue candidate c for one block of M <= c.max_m rows, with workspace wk.
static int launch_candidate_ws(const proj_plan* p, const Candidate& c, const void* X, const void* W, void* Y,
                               int64_t M, hipStream_t stream, const float* gamma, const Workspace& wk)
{
    if (M > c.max_m) return set_error(PROJ_EINVAL, "M=%lld exceeds %s's limit of %lld rows",
                                      (long long)M, c.name.c_str(), (long long)c.max_m);
    if (c.ws_bytes(M, p->N) > wk.ws_bytes)
        return set_error(PROJ_EINVAL, "%s needs %zu bytes of split-K workspace at M=%lld, has %zu",
                         c.name.c_str(), c.ws_bytes(M, p->N), (long long)M, wk.ws_bytes);
    if (c.UF && M > wk.gu_rows)
        return set_error(PROJ_EINVAL, "%s needs %lld rows of the SwiGLU intermediate, has %lld", c.name.c_str(),
                         (long long)M, (long long)wk.gu_rows);
    if (p->pro && !c.PRO && M > wk.xn_rows)
        return set_error(PROJ_EINVAL, "%s needs %lld rows of normalised X, has %lld", c.name.c_str(),
                         (long long)M, (long long)wk.xn_rows);
    const LaunchGeom g = geom(c, p->N, p->NO, M);
    const void* x = X;
    const void* w = W;
    void* y = c.UF ? wk.gu : Y;    // unfused SwiGLU: the N-column projection goes to the intermediate
    float* ws = wk.ws;
    const float* gam = gamma;
    int m = (int)M;
    if (p->pro && !c.PRO) {
        // unfused: the norm kernel writes the normalised rows into the workspace
        const void* xin = X;
        void* xo = wk.xn;
        long kk = (long)p->K;
        float eps = p->eps;
        void* nargs[] = {&xin, &gam, &xo, &kk, &eps};
        HIP_TRY(hipModuleLaunchKernel(p->f_norm, (unsigned)M, 1, 1, 256, 1, 1, 0, stream, nargs, nullptr));
        x = wk.xn;
    }
    void* args[] = {&x, &w, &y, &ws, &gam, &m};
    HIP_TRY(hipModuleLaunchKernel(c.fn, g.gx, g.gy, 1, g.threads, 1, 1, 0, stream, args, nullptr));
    if (c.needs_ws()) {
        int64_t total4 = M * p->N / 4;              // split-K: every output
        if (c.TAILS > 1) {                          // split tail: the tail tiles only
            int64_t T, n_full, rem;
            c.tail_split(M, p->N, &T, &n_full, &rem);
            total4 = rem * c.BM * c.BN / 4;
        }
        if (total4 > 0) {
            const unsigned gx = (unsigned)((total4 + 255) / 256);
            const float* wsc = ws;
            void* rargs[] = {&wsc, &y, &m};
            HIP_TRY(hipModuleLaunchKernel(c.reduce_fn, gx, 1, 1, 256, 1, 1, 0, stream, rargs, nullptr));
        }
    }
    if (c.UF) {
        // the separate activation kernel: Y[M, N/2] = silu(gate) * up of the intermediate
        const void* gsrc = wk.gu;
        void* h = Y;
        long mm = (long)M, nn = (long)p->N;
        void* sargs[] = {&gsrc, &h, &mm, &nn};
        const unsigned gx = (unsigned)std::min<int64_t>(65536, (M * (p->N / 2) + 255) / 256);
        HIP_TRY(hipModuleLaunchKernel(p->f_swiglu, gx, 1, 1, 256, 1, 1, 0, stream, sargs, nullptr));
    }
    return PROJ_OK;
}

int launch_candidate(const proj_plan* p, const Candidate& c, const void* X, const void* W, void* Y, int64_t M,
                     hipStream_t stream, const float* gamma)
{
    return launch_candidate_ws(p, c, X, W, Y, M, stream, gamma, plan_workspace(p));
}

// The workspace candidate c needs at M rows, carved from the static scratch:
// split partials, then normalised rows, then the SwiGLU intermediate, each
// starting on a 256-byte boundary.  PROJ_EINVAL if it does not fit.
static int scratch_workspace(const proj_plan* p, const Candidate& c, int64_t M, Workspace* wk)
{
    void* base = nullptr;
    int rc = scratch_address(p->device, &base);
    if (rc) return rc;
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const size_t ws = up(c.ws_bytes(M, p->N));
    const size_t xn = (p->pro && !c.PRO) ? up((size_t)M * p->K * 2) : 0;
    const size_t gu = c.UF ? up((size_t)M * p->N * (p->dtype == PROJ_OUT_BF16 ? 2 : 4)) : 0;
    const size_t cap = scratch_capacity();
    if (ws + xn + gu > cap)
        return set_error(PROJ_EINVAL,
                         "proj_run_noalloc: %s needs %zu bytes of scratch at M=%lld (partials %zu, normalised rows "
                         "%zu, SwiGLU intermediate %zu); the static scratch holds %zu: use fewer rows per call",
                         c.name.c_str(), ws + xn + gu, (long long)M, ws, xn, gu, cap);
    char* b = (char*)base;
    wk->ws = ws ? (float*)b : nullptr;
    wk->ws_bytes = ws;
    wk->xn = xn ? b + ws : nullptr;
    wk->xn_rows = xn ? M : 0;
    wk->gu = gu ? b + ws + xn : nullptr;
    wk->gu_rows = gu ? M : 0;
    return PROJ_OK;
}

// ---------------------------------------------------------------- the tuner
static float bits_f(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static float bf16_to_f(uint16_t b) { return bits_f((uint32_t)b << 16); }

// Device buffers and helper kernels used while tuning one plan.
struct Tuner {
    proj_plan* p;
    hipStream_t st = nullptr;
    hipFunction_t f_fill_probe = nullptr, f_fill_u32 = nullptr, f_ref = nullptr,
                  f_check = nullptr, f_probe = nullptr, f_hash = nullptr;
    void *Xr = nullptr, *Xi = nullptr, *Wr = nullptr, *Wi = nullptr, *Y = nullptr;
    // the weights as the candidates read them: Wr and Wi themselves, or their
    // copies in the panel layout (the reference kernel always reads row-major)
    void *Wrc = nullptr, *Wic = nullptr;
    void *Wrp = nullptr, *Wip = nullptr;
    float* gamma = nullptr;            // RMSNorm prologue: the probe's norm weights (K floats)
    void *Xnr = nullptr, *Xni = nullptr; // and the normalised probe rows the reference reads
    float *ref_r = nullptr, *ref_i = nullptr;
    int* rows_d = nullptr;
    CheckStats* stats_d = nullptr;
    void* flush = nullptr;
    size_t flush_bytes = 0;
    bool flush_tried = false;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    int64_t mmax = 0;
    static constexpr int64_t kGuardRows = 3;

    // copies of the probe weights (in the candidates' layout) for the decode
    // buckets' timing: one launch after another, each on the next copy, the
    // copies together larger than the last-level cache (allocated on first use)
    std::vector<void*> wrot;
    void* wrot_buf = nullptr;
    int next_copy = 0;

    ~Tuner()
    {
        for (void* q : {Xr, Xi, Wr, Wi, Y, (void*)ref_r, (void*)ref_i, (void*)rows_d, (void*)stats_d, flush,
                        (void*)gamma, Xnr, Xni, Wrp, Wip})
            if (q) (void)hipFree(q);
        if (wrot_buf) (void)hipFree(wrot_buf);
        if (e0) (void)hipEventDestroy(e0);
        if (e1) (void)hipEventDestroy(e1);
        if (st) (void)hipStreamDestroy(st);
    }

    size_t ysize() const { return p->dtype == PROJ_OUT_BF16 ? 2 : 4; }

    int fill_probe(void* buf, int64_t n, uint32_t seed, int kind, float scale)
    {
        unsigned gx = (unsigned)std::min<int64_t>((n + 255) / 256, 65536);
        long nn = (long)n;
        void* args[] = {&buf, &nn, &seed, &kind, &scale};
        HIP_TRY(hipModuleLaunchKernel(f_fill_probe, gx, 1, 1, 256, 1, 1, 0, st, args, nullptr));
        return PROJ_OK;
    }

    int pack(const void* w, void* wp)
    {
        long n = (long)p->N, k = (long)p->K;
        void* args[] = {&w, &wp, &n, &k};
        const unsigned gx = (unsigned)std::min<int64_t>((p->N * p->K / 8 + 255) / 256, 65536);
        HIP_TRY(hipModuleLaunchKernel(p->f_pack, gx, 1, 1, 256, 1, 1, 0, st, args, nullptr));
        return PROJ_OK;
    }

    int fill_sentinel(int64_t rows)
    {
        // whole 32-bit words: with bf16 output and an odd element count the last
        // word also covers the 2 bytes after the rows (the buffer is padded for it)
        const int64_t bytes = rows * p->NO * (int64_t)ysize();
        long n32 = (long)((bytes + 3) / 4);
        uint32_t v = p->dtype == PROJ_OUT_BF16 ? 0x7FBA7FBAu : 0x7FBADBADu;
        unsigned gx = (unsigned)std::min<int64_t>((n32 + 255) / 256, 65536);
        void* yp = Y;
        void* args[] = {&yp, &n32, &v};
        HIP_TRY(hipModuleLaunchKernel(f_fill_u32, gx, 1, 1, 256, 1, 1, 0, st, args, nullptr));
        return PROJ_OK;
    }

    int setup(int64_t max_rows)
    {
        mmax = max_rows;
        HIP_TRY(hipStreamCreate(&st));
        HIP_TRY(hipEventCreate(&e0));
        HIP_TRY(hipEventCreate(&e1));
        HIP_TRY(hipModuleGetFunction(&f_fill_probe, p->module, "proj_fill_probe"));
        HIP_TRY(hipModuleGetFunction(&f_fill_u32, p->module, "proj_fill_u32"));
        HIP_TRY(hipModuleGetFunction(&f_ref, p->module, "proj_ref_rows"));
        HIP_TRY(hipModuleGetFunction(&f_probe, p->module, "proj_probe_read"));
        HIP_TRY(hipModuleGetFunction(&f_hash, p->module, "proj_hash_out"));
        HIP_TRY(hipModuleGetFunction(&f_check, p->module,
                                     p->dtype == PROJ_OUT_BF16 ? "proj_check_bf16" : "proj_check_f32"));
        const size_t xb = (size_t)mmax * p->K * 2, wb = (size_t)p->N * p->K * 2;
        const size_t yb = ((size_t)(mmax + kGuardRows) * p->NO * ysize() + 3) / 4 * 4;   // whole words
        if (hipMalloc(&Xr, xb) != hipSuccess || hipMalloc(&Xi, xb) != hipSuccess ||
            hipMalloc(&Wr, wb) != hipSuccess || hipMalloc(&Wi, wb) != hipSuccess ||
            hipMalloc(&Y, yb) != hipSuccess || hipMalloc(&ref_r, 8 * p->N * 4) != hipSuccess ||
            hipMalloc(&ref_i, 8 * p->N * 4) != hipSuccess || hipMalloc(&rows_d, 8 * 4) != hipSuccess ||
            hipMalloc(&stats_d, sizeof(CheckStats)) != hipSuccess)
            return set_error(PROJ_ENOMEM, "tuner probe buffers (%zu MiB) could not be allocated",
                             (2 * xb + 2 * wb + yb) >> 20);
        int rc;
        if ((rc = fill_probe(Xr, mmax * p->K, 1, 0, 1.0f))) return rc;
        if ((rc = fill_probe(Wr, p->N * p->K, 2, 0, 0.0625f))) return rc;
        if ((rc = fill_probe(Xi, mmax * p->K, 3, 1, 1.0f))) return rc;
        if ((rc = fill_probe(Wi, p->N * p->K, 4, 1, 1.0f))) return rc;
        Wrc = Wr;
        Wic = Wi;
        if (p->wpack) {
            if (hipMalloc(&Wrp, wb) != hipSuccess || hipMalloc(&Wip, wb) != hipSuccess)
                return set_error(PROJ_ENOMEM, "tuner panel-layout weights (%zu MiB) could not be allocated",
                                 (2 * wb) >> 20);
            if ((rc = pack(Wr, Wrp)) || (rc = pack(Wi, Wip))) return rc;
            Wrc = Wrp;
            Wic = Wip;
        }
        if (p->pro) {
            // norm weights uniform in [0.5, 1.5): fill K bf16 values in [-0.5, 0.5),
            // widen on the host, add 1
            std::vector<uint16_t> hb(p->K);
            void* tmp = nullptr;
            if (hipMalloc(&gamma, p->K * 4) != hipSuccess || hipMalloc(&tmp, p->K * 2) != hipSuccess ||
                hipMalloc(&Xnr, xb) != hipSuccess || hipMalloc(&Xni, xb) != hipSuccess) {
                if (tmp) (void)hipFree(tmp);
                return set_error(PROJ_ENOMEM, "tuner norm buffers could not be allocated");
            }
            if ((rc = fill_probe(tmp, p->K, 5, 0, 0.5f))) { (void)hipFree(tmp); return rc; }
            HIP_TRY(hipStreamSynchronize(st));
            hipError_t e = hipMemcpy(hb.data(), tmp, p->K * 2, hipMemcpyDeviceToHost);
            (void)hipFree(tmp);
            HIP_TRY(e);
            std::vector<float> hg(p->K);
            for (int64_t k = 0; k < p->K; ++k) hg[k] = 1.0f + bf16_to_f(hb[k]);
            HIP_TRY(hipMemcpy(gamma, hg.data(), p->K * 4, hipMemcpyHostToDevice));
        }
        HIP_TRY(hipStreamSynchronize(st));
        return PROJ_OK;
    }

    // With the RMSNorm prologue: the reference reads the probe rows normalised
    // by the separate norm kernel (recomputed per bucket, after the reference
    // kernel's self-check on the raw integer rows).
    int reference_norm(const std::vector<int>& rows)
    {
        if (!p->pro) return PROJ_OK;
        for (int pass = 0; pass < 2; ++pass) {
            const void* xin = pass ? Xi : Xr;
            const float* g = gamma;
            void* xo = pass ? Xni : Xnr;
            long kk = (long)p->K;
            float eps = p->eps;
            void* nargs[] = {&xin, &g, &xo, &kk, &eps};
            HIP_TRY(hipModuleLaunchKernel(p->f_norm, (unsigned)mmax, 1, 1, 256, 1, 1, 0, st, nargs, nullptr));
        }
        HIP_TRY(hipMemcpyAsync(rows_d, rows.data(), rows.size() * 4, hipMemcpyHostToDevice, st));
        int nr = (int)rows.size();
        unsigned gx = (unsigned)((p->N + 255) / 256);
        for (int pass = 0; pass < 2; ++pass) {
            const void* x = pass ? Xni : Xnr;
            const void* w = pass ? Wi : Wr;
            float* r = pass ? ref_i : ref_r;
            int* rd = rows_d;
            void* args[] = {&x, &w, &rd, &nr, &r};
            HIP_TRY(hipModuleLaunchKernel(f_ref, gx, 1, 1, 256, 1, 1, 0, st, args, nullptr));
        }
        HIP_TRY(hipStreamSynchronize(st));
        return PROJ_OK;
    }

    // Reference rows (f32) for both probes; rows must be < mmax, at most 8.
    int reference(const std::vector<int>& rows)
    {
        HIP_TRY(hipMemcpyAsync(rows_d, rows.data(), rows.size() * 4, hipMemcpyHostToDevice, st));
        int nr = (int)rows.size();
        unsigned gx = (unsigned)((p->N + 255) / 256);
        for (int pass = 0; pass < 2; ++pass) {
            const void* x = pass ? Xi : Xr;
            const void* w = pass ? Wi : Wr;
            float* r = pass ? ref_i : ref_r;
            int* rd = rows_d;
            void* args[] = {&x, &w, &rd, &nr, &r};
            HIP_TRY(hipModuleLaunchKernel(f_ref, gx, 1, 1, 256, 1, 1, 0, st, args, nullptr));
        }
        HIP_TRY(hipStreamSynchronize(st));
        return PROJ_OK;
    }

    // The reference kernel itself is checked on the integer probe, where the
    // exact result is an integer computed here with int64 arithmetic.
    int self_check_reference(const std::vector<int>& rows)
    {
        const int64_t K = p->K, N = p->N;
        std::vector<uint16_t> xrow(K), wrow(K);
        std::vector<float> refrow(N);
        const int64_t cols[] = {0, N - 1, N / 2, N / 3, (N * 7) / 11};
        for (size_t j = 0; j < rows.size(); ++j) {
            HIP_TRY(hipMemcpy(xrow.data(), (char*)Xi + (size_t)rows[j] * K * 2, K * 2, hipMemcpyDeviceToHost));
            HIP_TRY(hipMemcpy(refrow.data(), ref_i + j * N, N * 4, hipMemcpyDeviceToHost));
            for (int64_t n : cols) {
                HIP_TRY(hipMemcpy(wrow.data(), (char*)Wi + (size_t)n * K * 2, K * 2, hipMemcpyDeviceToHost));
                int64_t acc = 0;
                for (int64_t k = 0; k < K; ++k)
                    acc += (int64_t)bf16_to_f(xrow[k]) * (int64_t)bf16_to_f(wrow[k]);
                if ((float)acc != refrow[n])
                    return set_error(PROJ_EDEVICE,
                                     "reference kernel self-check failed at row %d col %lld: %g vs exact %lld",
                                     rows[j], (long long)n, refrow[n], (long long)acc);
            }
        }
        return PROJ_OK;
    }

    // Run candidate c at M rows on one probe, then compare against the reference.
    int run_and_check(const Candidate& c, int64_t M, bool integer, int nrows, CheckStats* out)
    {
        int rc;
        if ((rc = fill_sentinel(M + kGuardRows))) return rc;
        HIP_TRY(hipMemsetAsync(stats_d, 0, sizeof(CheckStats), st));
        if ((rc = launch_candidate(p, c, integer ? Xi : Xr, integer ? Wic : Wrc, Y, M, st, gamma))) return rc;
        const void* yp = Y;
        long ra = (long)(M + kGuardRows);
        int m = (int)M;
        const float* r = integer ? ref_i : ref_r;
        const int* rd = rows_d;
        // normalised rows are not integers: with the norm prologue the integer
        // probe is held to the tolerance, not to bit equality
        int ex = (integer && !p->pro) ? 1 : 0;
        CheckStats* sd = stats_d;
        void* args[] = {&yp, &ra, &m, &r, &rd, &nrows, &ex, &sd};
        HIP_TRY(hipModuleLaunchKernel(f_check, 1024, 1, 1, 256, 1, 1, 0, st, args, nullptr));
        if (integer) {
            // the whole output of rows < M, for the comparison with the plain kernel
            long n = (long)(M * p->NO);
            void* hargs[] = {&yp, &n, &sd};
            HIP_TRY(hipModuleLaunchKernel(f_hash, 1024, 1, 1, 256, 1, 1, 0, st, hargs, nullptr));
        }
        HIP_TRY(hipMemcpyAsync(out, stats_d, sizeof(CheckStats), hipMemcpyDeviceToHost, st));
        HIP_TRY(hipStreamSynchronize(st));
        return PROJ_OK;
    }

    // A read of more than the 256 MB last-level cache before a timed launch, so
    // the launch reads its weights from HBM (only where the rotating weight
    // copies could not be allocated; the buffer is allocated on first use).
    int flush_cache()
    {
        if (!flush && !flush_tried) {
            flush_tried = true;
            flush_bytes = (size_t)512 << 20;
            if (hipMalloc(&flush, flush_bytes) != hipSuccess) {
                // timed without the flush; clear the runtime's last error so that a
                // caller checking it later does not see this tolerated failure
                (void)hipGetLastError();
                flush = nullptr;
                flush_bytes = 0;
            } else {
                HIP_TRY(hipMemsetAsync(flush, 0, flush_bytes, st));
            }
        }
        if (!flush) return PROJ_OK;
        const void* fp = flush;
        long n16 = (long)(flush_bytes / 16);
        uint32_t never = 0x9E3779B9u;
        uint32_t* sink = (uint32_t*)stats_d;  // written only if the XOR equals `never`
        void* args[] = {&fp, &n16, &never, &sink};
        const unsigned gx = (unsigned)((n16 + 2047) / 2048);  // one 32 KiB span per block
        HIP_TRY(hipModuleLaunchKernel(f_probe, gx, 1, 1, 256, 1, 1, 0, st, args, nullptr));
        return PROJ_OK;
    }

    // The projections of a model run one after another, each on weights that no
    // cache holds: a decode step streams every weight once, and a prompt block
    // meets each layer's weights after the other layers' have gone through the
    // 256 MB last-level cache.  So every candidate is timed in that regime:
    // launches back to back, each on the next of several weight copies that
    // together exceed that cache (1 GiB), in rounds of L launches -- all copies
    // for a decode GEMV (M <= 16), about 0.5 ms of work (at least 2 launches)
    // for a GEMM -- and the median over `reps` rounds of the mean per launch.
    // (Timed one launch at a time after a cache flush instead, the ranking of
    // near-equal kernels differed from the one measured back to back: a
    // 10240x5120 GEMV with cached loads came out first and ran 6 % slower than
    // the back-to-back pick, and a single launch of a 5120x2560 GEMM at 512 rows
    // took 24 us where back to back on rotating weights it takes 29.5 us, on
    // the same weights left in the last-level cache 21 us.)
    int time_rotating(const Candidate& c, int64_t M, int reps, double* us)
    {
        const size_t wb = (size_t)p->N * p->K * 2;
        if (wrot.empty()) {
            // copies 256-byte aligned in one buffer of 1 GiB, at most 128 copies (weights
            // under 8 MB then rotate through less: their launches are dominated by
            // fixed costs, not by where the bytes come from)
            const size_t wbs = (wb + 255) & ~(size_t)255;
            const size_t n = std::min<size_t>(128, std::max<size_t>(2, (((size_t)1 << 30) + wbs - 1) / wbs));
            if (hipMalloc(&wrot_buf, n * wbs) != hipSuccess) {
                (void)hipGetLastError();
                wrot_buf = nullptr;
                return PROJ_ENOMEM;   // not enough memory: the caller times cold launches
            }
            for (size_t i = 0; i < n; ++i) {
                wrot.push_back((char*)wrot_buf + i * wbs);
                HIP_TRY(hipMemcpyAsync(wrot.back(), Wrc, wb, hipMemcpyDeviceToDevice, st));
            }
            HIP_TRY(hipStreamSynchronize(st));
        }
        const int n = (int)wrot.size();
        int rc;
        // the next copy to read: the rotation goes on across rounds and candidates
        auto launch_next = [&](int i) -> int {
            const int w = next_copy;
            next_copy = (next_copy + 1) % n;
            return launch_candidate(p, c, (i & 1) ? Xi : Xr, wrot[w], Y, M, st, gamma);
        };
        int L = n;
        if (M > 16) {
            // two launches estimate the time per launch; rounds of about 0.5 ms
            HIP_TRY(hipEventRecord(e0, st));
            for (int i = 0; i < 2; ++i)
                if ((rc = launch_next(i))) return rc;
            HIP_TRY(hipEventRecord(e1, st));
            HIP_TRY(hipEventSynchronize(e1));
            float ms = 0;
            HIP_TRY(hipEventElapsedTime(&ms, e0, e1));
            const double est = std::max(1.0, ms * 1000.0 / 2);
            L = (int)std::min<double>(n, std::max(2.0, std::ceil(500.0 / est)));
        }
        for (int i = 0; i < L; ++i)   // one untimed round
            if ((rc = launch_next(i))) return rc;
        std::vector<double> t;
        for (int r = 0; r < reps; ++r) {
            HIP_TRY(hipEventRecord(e0, st));
            for (int i = 0; i < L; ++i)
                if ((rc = launch_next(i))) return rc;
            HIP_TRY(hipEventRecord(e1, st));
            HIP_TRY(hipEventSynchronize(e1));
            float ms = 0;
            HIP_TRY(hipEventElapsedTime(&ms, e0, e1));
            t.push_back(ms * 1000.0 / L);
        }
        std::sort(t.begin(), t.end());
        *us = t[t.size() / 2];
        return PROJ_OK;
    }

    // Median launch time in microseconds at M rows: back to back on rotating
    // weights, or (if the copies do not fit in memory) one launch at a time
    // after a cache flush.
    int time_candidate(const Candidate& c, int64_t M, int reps, double* us)
    {
        int rc = time_rotating(c, M, reps, us);
        if (rc != PROJ_ENOMEM) return rc;
        for (int i = 0; i < 2; ++i)
            if ((rc = launch_candidate(p, c, Xr, Wrc, Y, M, st, gamma))) return rc;
        std::vector<double> t;
        for (int i = 0; i < reps; ++i) {
            if ((rc = flush_cache())) return rc;
            HIP_TRY(hipEventRecord(e0, st));
            if ((rc = launch_candidate(p, c, (i & 1) ? Xi : Xr, (i & 1) ? Wic : Wrc, Y, M, st, gamma))) return rc;
            HIP_TRY(hipEventRecord(e1, st));
            HIP_TRY(hipEventSynchronize(e1));
            float ms = 0;
            HIP_TRY(hipEventElapsedTime(&ms, e0, e1));
            t.push_back(ms * 1000.0);
        }
        std::sort(t.begin(), t.end());
        *us = t[t.size() / 2];
        return PROJ_OK;
    }
};

static bool applies(const Candidate& c, int b, const proj_plan* p)
{
    const BucketRange br = kBuckets[b];
    if (c.max_m < br.hi) return false;
    // every M of the bucket must fit the workspace (a split tail's need is not
    // monotonic in M, so its bound over the bucket is used)
    if (c.ws_bound(br.hi, p->N) > p->ws_bytes) return false;
    switch (c.fam) {
    case Family::GemvValu:
        if (b == 0) return c.MMAX == 1;
        return b == 1 && c.MMAX == 16;
    case Family::GemvMfma: return b <= 1;
    case Family::Gemm:
        if (b == 0) return false;
        if (b <= 2) return c.BM <= 128;
        if (b == 3) return c.BM <= 256;
        return c.BM >= 128 && c.SK <= 2;
    case Family::Plain: return false;  // only as a last resort
    }
    return false;
}

static void plog(proj_plan* p, const std::string& line)
{
    p->log.push_back(line);
    if (env_int("PROJ_LOG", 0)) fprintf(stderr, "%s\n", line.c_str());
}

// ---------------------------------------------------------------- tuning cache
// The choices of a tuned plan, kept in a text file per key (the persistent
// tuning cache the pages propose -- and doubt, because the machine's state
// drifts -- in "#004 the same compiler on Apple's chips", section "So, does it
// start up more slowly?").  The key hashes the device (full architecture name, CU count),
// the HIP runtime and driver versions and the complete emitted source, which
// fixes the shape, output type, epilogue and every candidate's code; so a
// library or driver change is a different key.  On a hit every cached choice
// still goes through the load-time gate before it is used ("re-validation");
// a choice that is missing or fails it sends its bucket back to full tuning.
// Off unless PROJ_CACHE_DIR names a directory.
static uint64_t fnv1a(uint64_t h, const std::string& s)
{
    for (unsigned char c : s) {
        h ^= c;
        h *= 0x100000001b3ull;
    }
    return h;
}

// Whether buf holds a whole ELF64 image: the magic, and the program and section
// header tables inside the buffer.  (hipModuleLoadData takes no size, so a
// truncated or foreign cache file must not reach it.)
bool whole_elf64(const std::vector<char>& buf)
{
    if (buf.size() < 64 || memcmp(buf.data(), "\x7f" "ELF", 4) != 0 || buf[4] != 2) return false;
    auto u64 = [&](size_t o) { uint64_t v; memcpy(&v, buf.data() + o, 8); return v; };
    auto u16 = [&](size_t o) { uint16_t v; memcpy(&v, buf.data() + o, 2); return (uint64_t)v; };
    const uint64_t n = buf.size();
    const uint64_t ph = u64(32), sh = u64(40), phe = u16(54), phn = u16(56), she = u16(58), shn = u16(60);
    return ph <= n && phe * phn <= n - ph && sh <= n && she * shn <= n - sh;
}

static int cache_key(proj_plan* p, const std::string& src)
{
    hipDeviceProp_t prop;
    HIP_TRY(hipGetDeviceProperties(&prop, p->device));
    int rt = 0, drv = 0;
    HIP_TRY(hipRuntimeGetVersion(&rt));
    HIP_TRY(hipDriverGetVersion(&drv));
    char head[512];
    // which compiler: the helper (its file size and time identify the build)
    // or the hipRTC loaded in this process (its version)
    std::string compiler = "in-process";
    const std::string helper = rtc_jobs() > 0 ? helper_path() : "";
    struct stat hs;
    if (!helper.empty() && stat(helper.c_str(), &hs) == 0) {
        compiler = "helper:" + std::to_string((long long)hs.st_size) + ":" + std::to_string((long long)hs.st_mtime);
    } else {
        int ma = 0, mi = 0;
        if (hiprtcVersion(&ma, &mi) == HIPRTC_SUCCESS) compiler += ":" + std::to_string(ma) + "." + std::to_string(mi);
    }
    snprintf(head, sizeof head, "%s|cus=%d|runtime=%d|driver=%d|options=%s|compiler=%s|", prop.gcnArchName,
             prop.multiProcessorCount, rt, drv, kRtcOptionText, compiler.c_str());
    p->key = fnv1a(fnv1a(0xcbf29ce484222325ull, head), src);
    return PROJ_OK;
}

// Cached choice names per bucket ("" where absent); false if there is no usable file.
bool cache_read(const std::string& path, std::vector<std::string>* names)
{
    std::ifstream f(path);
    if (!f) return false;
    std::string line;
    if (!std::getline(f, line) || line != "libproj tuning cache 1") return false;
    names->assign(kNumBuckets, "");
    while (std::getline(f, line)) {
        int b = -1;
        char name[160] = {0};
        if (sscanf(line.c_str(), "bucket %d %159s", &b, name) == 2 && b >= 0 && b < kNumBuckets) (*names)[b] = name;
    }
    return true;
}

void cache_write(proj_plan* p)
{
    const std::string tmp = p->cache_path + ".tmp";
    {
        std::ofstream f(tmp);
        if (!f) return;
        f << "libproj tuning cache 1\n";
        f << "# N=" << p->N << " K=" << p->K << " dtype=" << (p->dtype ? "bf16" : "f32")
          << " epilogue=" << (p->epi ? "swiglu" : "none") << " layout=" << (p->wpack ? "panels" : "rows")
          << " arch=" << p->arch << "\n";
        for (int b = 0; b < kNumBuckets; ++b)
            if (p->choice[b] >= 0)
                f << "bucket " << b << " " << p->cands[p->choice[b]].name << " " << p->choice_us[b] << "\n";
        if (!f) return;
    }
    if (std::rename(tmp.c_str(), p->cache_path.c_str()) != 0) std::remove(tmp.c_str());
}

int tune_plan(proj_plan* p)
{
    const double t0 = now_s();
    const size_t ws_cap = (size_t)env_int("PROJ_WS_MB", 256) << 20;
    const bool do_time = env_int("PROJ_TUNE", 1) != 0;
    const int reps = std::max(3, env_int("PROJ_TUNE_REPS", 10));
    const char* force = getenv("PROJ_FORCE");

    // split-K workspace: enough for every split-K candidate at the largest block,
    // capped; a candidate then runs up to the row count the workspace holds.
    size_t need = 0;
    for (const Candidate& c : p->cands) need = std::max(need, c.ws_bound(kMaxBlockRows, p->N));
    need = std::min(need, ws_cap);
    if (need) {
        if (hipMalloc(&p->ws, need) != hipSuccess) {
            p->ws = nullptr;
            return set_error(PROJ_ENOMEM, "split-K workspace of %zu bytes", need);
        }
        p->ws_bytes = need;
    }
    // SwiGLU plans: the intermediate of the unfused candidates, as many rows as
    // fit the same cap; an unfused candidate serves up to that many rows
    if (p->epi) {
        const size_t row_bytes = (size_t)p->N * (p->dtype == PROJ_OUT_BF16 ? 2 : 4);
        p->gu_rows = std::min<int64_t>(kMaxBlockRows, (int64_t)(ws_cap / row_bytes));
        if (p->gu_rows > 0 && hipMalloc(&p->gu, (size_t)p->gu_rows * row_bytes) != hipSuccess) {
            p->gu = nullptr;
            return set_error(PROJ_ENOMEM, "SwiGLU intermediate of %zu bytes", (size_t)p->gu_rows * row_bytes);
        }
        for (Candidate& c : p->cands)
            if (c.UF) c.max_m = std::min<int64_t>(c.max_m, p->gu_rows);
        HIP_TRY(hipModuleGetFunction(&p->f_swiglu, p->module,
                                     p->dtype == PROJ_OUT_BF16 ? "proj_swiglu_bf16" : "proj_swiglu_f32"));
    }

    Tuner T;
    T.p = p;
    int rc;
    if ((rc = T.setup(kBuckets[kNumBuckets - 1].hi))) return rc;

    std::vector<std::string> cached;
    p->cache = "off";
    if (const char* dir = getenv("PROJ_CACHE_DIR")) {
        if (*dir) {
            char file[64];
            snprintf(file, sizeof file, "/proj-%016llx.txt", (unsigned long long)p->key);
            p->cache_path = std::string(dir) + file;
            p->cache = cache_read(p->cache_path, &cached) ? "hit" : "miss";
        }
    }
    bool retuned = false;

    p->timings.assign(kNumBuckets, {});
    p->rejected.assign(kNumBuckets, {});
    bool ref_checked = false;
    char line[1024];
    for (int b = 0; b < kNumBuckets; ++b) {
        const BucketRange br = kBuckets[b];
        const int64_t Mfull = br.hi;
        const int64_t Mpart = br.lo == br.hi ? br.hi : br.hi - 1;
        const int64_t Modd = br.lo == br.hi ? br.hi : std::min<int64_t>(br.hi, br.lo + ((br.hi - br.lo) / 3 | 1));
        std::vector<int64_t> tests = {Mfull, Mpart, Modd};
        std::sort(tests.begin(), tests.end());
        tests.erase(std::unique(tests.begin(), tests.end()), tests.end());
        std::vector<int> rows = {0, (int)(Mfull - 1), (int)(Mpart - 1), (int)(Modd - 1), (int)(Modd / 2),
                                 (int)std::min<int64_t>(Mfull - 1, 31), (int)std::min<int64_t>(Mfull - 1, 32),
                                 (int)(Mfull / 2)};
        std::sort(rows.begin(), rows.end());
        rows.erase(std::unique(rows.begin(), rows.end()), rows.end());
        if ((rc = T.reference(rows))) return rc;
        if (!ref_checked) {
            if ((rc = T.self_check_reference(rows))) return rc;
            ref_checked = true;
        }
        const int nrows = (int)rows.size();
        if ((rc = T.reference_norm(rows))) return rc;

        // The reference rows cover a few rows only.  On the integer probe every
        // summation order gives the same bits, so the whole output of every
        // candidate must also equal the plain kernel's (one thread per output,
        // k ascending; itself checked on the reference rows here): compared by
        // an order-independent hash of all rows < M.  Not with the norm
        // prologue, whose normalised rows are not integers.
        bool have_base = false;
        uint64_t base_hash = 0;
        if (!p->pro) {
            CheckStats bs{};
            if ((rc = T.run_and_check(p->cands.back(), Mpart, true, nrows, &bs))) return rc;
            if (bs.bad || bs.unwritten || bs.guard) {
                snprintf(line, sizeof line,
                         "[autotune] proj %lldx%lld %lld rows: the plain kernel fails the integer probe; whole-output "
                         "comparison off for this bucket",
                         (long long)p->N, (long long)p->K, (long long)br.hi);
                plog(p, line);
            } else {
                have_base = true;
                base_hash = bs.hash;
            }
        }

        std::vector<int> ok;
        auto validate = [&](int ci) -> int {
            const Candidate& c = p->cands[ci];
            for (int64_t M : tests) {
                for (int integer = 0; integer < 2; ++integer) {
                    if (integer && M != Mpart) continue;
                    CheckStats cs{};
                    int r2 = T.run_and_check(c, M, integer != 0, nrows, &cs);
                    if (r2) return r2;
                    const std::string why =
                        gate_reject_line(cs, integer != 0, have_base, base_hash, p->N, p->K, br.hi, c.name, M);
                    if (!why.empty()) {
                        plog(p, why);
                        p->rejected[b].push_back({ci, why});
                        return 1;
                    }
                }
            }
            return 0;
        };

        if (!cached.empty() && !cached[b].empty() && !(force && *force)) {
            int ci = -1;
            for (int i = 0; i < (int)p->cands.size(); ++i)
                if (p->cands[i].name == cached[b]) ci = i;
            if (ci >= 0 && (applies(p->cands[ci], b, p) || p->cands[ci].fam == Family::Plain)) {
                const int v = validate(ci);
                if (v < 0) return v;
                if (v == 0) {
                    snprintf(line, sizeof line, "[autotune] proj %lldx%lld %lld..%lld rows: %s (cached, re-validated)",
                             (long long)p->N, (long long)p->K, (long long)br.lo, (long long)br.hi, cached[b].c_str());
                    plog(p, line);
                    p->choice[b] = ci;
                    p->choice_us[b] = -1;
                    continue;
                }
            }
            p->cache = "stale";
        }
        retuned = true;
        for (int ci = 0; ci < (int)p->cands.size(); ++ci) {
            const Candidate& c = p->cands[ci];
            if (!applies(c, b, p)) continue;
            if (force && *force && c.name != force) continue;
            int v = validate(ci);
            if (v < 0) return v;
            if (v == 0) ok.push_back(ci);
        }
        if (ok.empty()) {
            // last resort: the plain kernel
            const int pi = (int)p->cands.size() - 1;
            int v = validate(pi);
            if (v < 0) return v;
            if (v) return set_error(PROJ_ENOCAND, "no candidate passed validation for %lld..%lld rows",
                                    (long long)br.lo, (long long)br.hi);
            ok.push_back(pi);
        }

        int best = ok[0];
        double best_us = -1;
        if (do_time && ok.size() > 1) {
            std::string tl;
            // A screen of three rounds per candidate, then the full `reps`
            // rounds for those within 10 % of the screen's best (most of the
            // list is far slower and needs no more than the screen to say so).
            const int screen = std::min(3, reps);
            double screen_best = -1;
            for (int ci : ok) {
                double us = 0;
                if ((rc = T.time_candidate(p->cands[ci], Mfull, screen, &us))) return rc;
                p->timings[b].push_back({ci, us});
                if (screen_best < 0 || us < screen_best) screen_best = us;
            }
            for (auto& t : p->timings[b]) {
                if (reps > screen && t.second <= screen_best * 1.10)
                    if ((rc = T.time_candidate(p->cands[t.first], Mfull, reps, &t.second))) return rc;
                if (best_us < 0 || t.second < best_us) {
                    best_us = t.second;
                    best = t.first;
                }
            }
            // Finalists: the (at most four) candidates within 5 % of the fastest,
            // timed again in three interleaved rounds, so that a drifting clock
            // weighs on all of them alike; the lowest median of the rounds wins,
            // and a later candidate must beat an earlier one by 1 % (near-equal
            // variants then do not flip the choice from one load to the next).
            std::vector<std::pair<double, int>> fin;
            for (const auto& t : p->timings[b])
                if (t.second <= best_us * 1.05) fin.push_back({t.second, t.first});
            std::sort(fin.begin(), fin.end());
            if (fin.size() > 4) fin.resize(4);
            if (fin.size() > 1) {
                std::sort(fin.begin(), fin.end(), [](const std::pair<double, int>& a, const std::pair<double, int>& c) {
                    return a.second < c.second;   // list order
                });
                std::vector<std::vector<double>> rt(fin.size());
                for (int round = 0; round < 3; ++round)
                    for (size_t f = 0; f < fin.size(); ++f) {
                        double us = 0;
                        if ((rc = T.time_candidate(p->cands[fin[f].second], Mfull, reps, &us))) return rc;
                        rt[f].push_back(us);
                    }
                best_us = -1;
                for (size_t f = 0; f < fin.size(); ++f) {
                    std::sort(rt[f].begin(), rt[f].end());
                    const double med = rt[f][1];
                    if (best_us < 0 || med < best_us * 0.99) {
                        best_us = med;
                        best = fin[f].second;
                    }
                }
            }
            std::ostringstream os;
            os << "[autotune] proj " << p->N << "x" << p->K << " " << br.lo << ".." << br.hi << " rows at "
               << Mfull << ":";
            for (size_t i = 0; i < p->timings[b].size(); ++i) {
                char t[64];
                snprintf(t, sizeof t, " %.3f us", p->timings[b][i].second);
                os << (i ? "," : "") << " " << p->cands[p->timings[b][i].first].name
                   << (p->timings[b][i].first == best ? "*" : "") << t;
            }
            os << " -> " << p->cands[best].name;
            plog(p, os.str());
        } else {
            snprintf(line, sizeof line, "[autotune] proj %lldx%lld %lld..%lld rows: %s (validated, not timed)",
                     (long long)p->N, (long long)p->K, (long long)br.lo, (long long)br.hi,
                     p->cands[best].name.c_str());
            plog(p, line);
        }
        p->choice[b] = best;
        p->choice_us[b] = best_us;
    }
    if (!p->cache_path.empty() && retuned && do_time && !(force && *force)) cache_write(p);
    p->tune_s = now_s() - t0;
    return PROJ_OK;
}

int create_plan(int64_t N, int64_t K, int dtype, int fusion, float norm_eps, proj_plan** out)
{
    const int epi = fusion & PROJ_EPI_SWIGLU;
    *out = nullptr;
    if (N < 1 || K < 8 || K % 8 != 0 || N > (int64_t)1 << 30 || K > (int64_t)1 << 24)
        return set_error(PROJ_EINVAL, "invalid shape N=%lld K=%lld (need N >= 1, K >= 8, K %% 8 == 0)",
                         (long long)N, (long long)K);
    if (dtype != PROJ_OUT_F32 && dtype != PROJ_OUT_BF16)
        return set_error(PROJ_EINVAL, "invalid dtype %d (PROJ_OUT_F32=0 or PROJ_OUT_BF16=1)", dtype);
    if (fusion & ~(PROJ_EPI_SWIGLU | PROJ_PRO_RMSNORM | PROJ_W_PACKED))
        return set_error(PROJ_EINVAL, "invalid flags %d (PROJ_EPI_SWIGLU=1 | PROJ_PRO_RMSNORM=2 | PROJ_W_PACKED=4)",
                         fusion);
    if ((fusion & PROJ_W_PACKED) && (N % 128 || K % 64))
        return set_error(PROJ_EINVAL, "the packed weight layout needs N %% 128 == 0 and K %% 64 == 0, got N=%lld K=%lld",
                         (long long)N, (long long)K);
    if ((fusion & PROJ_PRO_RMSNORM) && !(norm_eps >= 0.f && norm_eps < 1e30f))
        return set_error(PROJ_EINVAL, "invalid RMSNorm epsilon %g", (double)norm_eps);
    if (epi == PROJ_EPI_SWIGLU && N % 2)
        return set_error(PROJ_EINVAL, "the SwiGLU epilogue needs an even N (gate and up halves), got N=%lld",
                         (long long)N);
    std::unique_ptr<proj_plan> p(new proj_plan());
    // until the plan is handed out, any early return releases what it holds
    struct Release {
        proj_plan* p;
        ~Release()
        {
            if (!p) return;
            if (p->ws) (void)hipFree(p->ws);
            if (p->gu) (void)hipFree(p->gu);
            if (p->xn) (void)hipFree(p->xn);
            for (hipModule_t m : p->modules)
                if (m) (void)hipModuleUnload(m);
        }
    } release{p.get()};
    p->N = N;
    p->K = K;
    p->dtype = dtype;
    p->epi = epi;
    p->pro = (fusion & PROJ_PRO_RMSNORM) ? 1 : 0;
    p->eps = p->pro ? norm_eps : 0.f;
    p->wpack = (fusion & PROJ_W_PACKED) ? 1 : 0;
    p->NO = epi == PROJ_EPI_SWIGLU ? N / 2 : N;
    HIP_TRY(hipGetDevice(&p->device));
    int rc;
    int cus = kDefaultCUs;
    if ((rc = device_arch(p->device, &p->arch, &cus))) return rc;
    for (int b = 0; b < kNumBuckets; ++b) p->choice[b] = -1, p->choice_us[b] = -1;

    {
        // set-up of the static scratch on this device (proj_run_noalloc), with
        // the device current; a failure here only matters to proj_run_noalloc,
        // which looks again and reports it
        void* sp = nullptr;
        if (scratch_address(p->device, &sp) != PROJ_OK) {
            plog(p.get(), "[proj] static scratch not available: " + g_last_error);
            g_last_error.clear();
            (void)hipGetLastError();
        }
    }
    p->cands = enumerate_candidates(N, K, cus, fusion);
    // the whole translation unit keys the caches and is what PROJ_DUMP_DIR
    // writes; it is compiled as modules, each holding some candidates
    const std::string src = emit_source(N, K, dtype, p->arch, cus, p->cands, fusion, p->eps);
    const std::vector<std::string> msrcs =
        emit_module_sources(N, K, dtype, p->arch, cus, p->cands, fusion, p->eps, kMaxModules);
    if ((rc = cache_key(p.get(), src))) return rc;
    const double t0 = now_s();
    std::vector<std::shared_ptr<std::vector<char>>> codes;
    char name[96];
    snprintf(name, sizeof name, "proj_%lldx%lld_%s%s%s%s", (long long)N, (long long)K, dtype ? "bf16" : "f32",
             epi ? "_swiglu" : "", p->pro ? "_rmsnorm" : "", p->wpack ? "_panels" : "");
    // With PROJ_CACHE_DIR, the compiled modules are kept beside the tuned
    // choices under the same key (device, runtime and driver versions, compile
    // options, emitted source): a later plan of the same key loads them
    // instead of compiling.  Files that do not load are compiled afresh and
    // replaced.
    std::string co_base;
    if (const char* dir = getenv("PROJ_CACHE_DIR")) {
        if (*dir) {
            char file[64];
            snprintf(file, sizeof file, "/proj-%016llx", (unsigned long long)p->key);
            co_base = std::string(dir) + file;
        }
    }
    auto co_path = [&](size_t g) { return co_base + ".m" + std::to_string(g) + ".co"; };
    auto unload_all = [&]() {
        for (hipModule_t m : p->modules)
            if (m) (void)hipModuleUnload(m);
        p->modules.clear();
        p->module = nullptr;
    };
    p->code_cache = co_base.empty() ? "off" : "miss";
    if (!co_base.empty()) {
        std::vector<std::shared_ptr<std::vector<char>>> cached(msrcs.size());
        bool all = true, any = false;
        for (size_t g = 0; g < msrcs.size(); ++g) {
            std::ifstream f(co_path(g), std::ios::binary);
            if (!f) { all = false; continue; }
            any = true;
            cached[g] = std::make_shared<std::vector<char>>((std::istreambuf_iterator<char>(f)),
                                                            std::istreambuf_iterator<char>());
            if (!whole_elf64(*cached[g])) all = false;
        }
        if (all) {
            for (size_t g = 0; g < msrcs.size() && all; ++g) {
                hipModule_t m = nullptr;
                if (hipModuleLoadData(&m, cached[g]->data()) != hipSuccess) {
                    (void)hipGetLastError();
                    all = false;
                } else {
                    p->modules.push_back(m);
                }
            }
            if (all) {
                codes = cached;
                p->code_cache = "hit";
            } else {
                unload_all();
            }
        }
        if (!all && any) p->code_cache = "stale";
    }
    // write the compiled modules to the cache (temporary files renamed into
    // place, so readers never see a partial one)
    auto store_code = [&]() {
        if (co_base.empty()) return;
        for (size_t g = 0; g < codes.size(); ++g) {
            const std::string tmp = co_path(g) + ".tmp";
            bool ok = false;
            {
                std::ofstream f(tmp, std::ios::binary);
                ok = f && f.write(codes[g]->data(), (std::streamsize)codes[g]->size());
            }
            if (!ok || std::rename(tmp.c_str(), co_path(g).c_str()) != 0) std::remove(tmp.c_str());
        }
    };
    auto load_all = [&]() -> int {
        for (size_t g = 0; g < codes.size(); ++g) {
            hipModule_t m = nullptr;
            HIP_TRY(hipModuleLoadData(&m, codes[g]->data()));
            p->modules.push_back(m);
        }
        p->module = p->modules[0];
        return PROJ_OK;
    };
    if (codes.empty()) {
        if ((rc = compile_sources(msrcs, p->arch, name, &codes))) return rc;
        store_code();
    }
    p->compile_s = now_s() - t0;
    p->code_bytes = 0;
    for (const auto& c : codes) p->code_bytes += c->size();
    if (const char* dir = getenv("PROJ_DUMP_DIR")) {
        if (*dir) {
            const std::string base = std::string(dir) + "/" + name;
            std::ofstream(base + ".hip", std::ios::binary) << src;
            for (size_t g = 0; g < codes.size(); ++g)
                std::ofstream(base + ".m" + std::to_string(g) + "." + p->arch + ".co", std::ios::binary)
                    .write(codes[g]->data(), (std::streamsize)codes[g]->size());
        }
    }
    if (p->modules.empty()) {
        if ((rc = load_all())) return rc;
    } else {
        p->module = p->modules[0];
    }
    // every kernel the plan launches, from the loaded modules
    auto bind = [&]() -> int {
        HIP_TRY(hipModuleGetFunction(&p->f_pack, p->module, "proj_pack_panels"));
        if (p->pro) HIP_TRY(hipModuleGetFunction(&p->f_norm, p->module, "proj_rmsnorm_rows"));
        for (Candidate& c : p->cands) {
            HIP_TRY(hipModuleGetFunction(&c.fn, p->modules[c.module], c.name.c_str()));
            if (!c.reduce_name.empty())
                HIP_TRY(hipModuleGetFunction(&c.reduce_fn, p->modules[c.module], c.reduce_name.c_str()));
        }
        return PROJ_OK;
    };
    if ((rc = bind())) {
        if (p->code_cache != "hit") return rc;
        // cached modules that lack a kernel: compile afresh and replace the files
        (void)hipGetLastError();
        unload_all();
        p->code_cache = "stale";
        if ((rc = compile_sources(msrcs, p->arch, name, &codes))) return rc;
        store_code();
        p->code_bytes = 0;
        for (const auto& c : codes) p->code_bytes += c->size();
        if ((rc = load_all())) return rc;
        if ((rc = bind())) return rc;
    }
    if (p->pro) {
        if (hipMalloc(&p->xn, (size_t)kMaxBlockRows * K * 2) != hipSuccess) {
            p->xn = nullptr;
            return set_error(PROJ_ENOMEM, "RMSNorm workspace of %lld bytes", (long long)kMaxBlockRows * K * 2);
        }
    }
    char line[256];
    snprintf(line, sizeof line, "[proj] %lldx%lld %s: %zu candidates in %zu modules %s for %s in %.2f s (%zu bytes)",
             (long long)N, (long long)K, dtype ? "bf16" : "f32", p->cands.size(), p->modules.size(),
             p->code_cache == "hit" ? "loaded from the code cache" : "compiled", p->arch.c_str(), p->compile_s,
             p->code_bytes);
    plog(p.get(), line);
    if ((rc = tune_plan(p.get()))) return rc;
    snprintf(line, sizeof line, "[proj] %lldx%lld: tuned %d row buckets in %.2f s", (long long)N, (long long)K,
             kNumBuckets, p->tune_s);
    plog(p.get(), line);
    release.p = nullptr;
    *out = p.release();
    return PROJ_OK;
}

void destroy_plan(proj_plan* p)
{
    if (!p) return;
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != p->device) (void)hipSetDevice(p->device);
    // launches of this plan may still be pending on any stream of the device:
    // they read its modules and workspace
    (void)hipDeviceSynchronize();
    if (p->ws) (void)hipFree(p->ws);
    if (p->gu) (void)hipFree(p->gu);
    if (p->xn) (void)hipFree(p->xn);
    for (hipModule_t m : p->modules)
        if (m) (void)hipModuleUnload(m);
    if (cur >= 0 && cur != p->device) (void)hipSetDevice(cur);
    delete p;
}

int check_run_args(const proj_plan* p, const void* X, const void* W, void* Y, int64_t M)
{
    if (!p) return set_error(PROJ_EINVAL, "plan is NULL");
    if (M < 0) return set_error(PROJ_EINVAL, "M=%lld is negative", (long long)M);
    if (M == 0) return PROJ_OK;
    // X (M x K bf16) and Y (M x NO, at most 4 bytes each) must stay below 2^48
    // bytes, far beyond any device memory, so the size arithmetic below cannot wrap
    if (M > (int64_t(1) << 48) / (4 * std::max<int64_t>(p->K, p->NO)))
        return set_error(PROJ_EINVAL, "M=%lld: X or Y would exceed 2^48 bytes", (long long)M);
    if (!X || !W || !Y) return set_error(PROJ_EINVAL, "null pointer (X=%p W=%p Y=%p)", X, W, (void*)Y);
    if (((uintptr_t)X | (uintptr_t)W | (uintptr_t)Y) & 15)
        return set_error(PROJ_EINVAL, "X, W and Y must be 16-byte aligned (X=%p W=%p Y=%p)", X, W, (void*)Y);
    // Y is written while X and W are still read (by other workgroups): no overlap
    const uintptr_t x0 = (uintptr_t)X, w0 = (uintptr_t)W, y0 = (uintptr_t)Y;
    const uintptr_t x1 = x0 + (uintptr_t)M * (uintptr_t)p->K * 2u;
    const uintptr_t w1 = w0 + (uintptr_t)p->N * (uintptr_t)p->K * 2u;
    const uintptr_t y1 = y0 + (uintptr_t)M * (uintptr_t)p->NO * (p->dtype == PROJ_OUT_BF16 ? 2u : 4u);
    if ((y0 < x1 && x0 < y1) || (y0 < w1 && w0 < y1))
        return set_error(PROJ_EINVAL, "Y [%p, %p) overlaps X [%p, %p) or W [%p, %p)", (void*)y0, (void*)y1,
                         (void*)x0, (void*)x1, (void*)w0, (void*)w1);
    int cur = -1;
    HIP_TRY(hipGetDevice(&cur));
    if (cur != p->device)
        return set_error(PROJ_EINVAL, "current device %d is not the plan's device %d", cur, p->device);
    return PROJ_OK;
}

int run_plan(const proj_plan* p, const void* X, const void* W, void* Y, int64_t M, hipStream_t stream,
             const float* gamma, bool packed, bool noalloc)
{
    if (p && p->wpack != (packed ? 1 : 0))
        return set_error(PROJ_EINVAL, packed ? "this plan reads row-major weights: use proj_run or proj_run_ex"
                                             : "this plan reads weights in the packed layout: use proj_run_packed");
    int rc = check_run_args(p, X, W, Y, M);
    if (rc || M == 0) return rc;
    if (p->pro && !gamma) return set_error(PROJ_EINVAL, "this plan has the RMSNorm prologue: gamma is required");
    if (p->pro && ((uintptr_t)gamma & 15)) return set_error(PROJ_EINVAL, "gamma must be 16-byte aligned");
    const size_t ysz = p->dtype == PROJ_OUT_BF16 ? 2 : 4;
    if (noalloc) {
        // every block must fit the scratch before anything is enqueued
        for (int64_t off = 0; off < M; off += kMaxBlockRows) {
            const int64_t m = std::min<int64_t>(kMaxBlockRows, M - off);
            Workspace wk;
            if ((rc = scratch_workspace(p, p->cands[p->choice[bucket_of(m)]], m, &wk))) return rc;
        }
    }
    for (int64_t off = 0; off < M; off += kMaxBlockRows) {
        const int64_t m = std::min<int64_t>(kMaxBlockRows, M - off);
        const Candidate& c = p->cands[p->choice[bucket_of(m)]];
        Workspace wk = plan_workspace(p);
        if (noalloc && (rc = scratch_workspace(p, c, m, &wk))) return rc;
        rc = launch_candidate_ws(p, c, (const char*)X + (size_t)off * p->K * 2, W, (char*)Y + (size_t)off * p->NO * ysz,
                                 m, stream, gamma, wk);
        if (rc) return rc;
    }
    return PROJ_OK;
}

}  // namespace proj
