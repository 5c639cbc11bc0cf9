// api.cpp -- the extern "C" entry points declared in include/proj.h.
#include <algorithm>
#include <chrono>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <sstream>

#include "proj.h"
#include "proj_internal.h"

namespace proj {
extern thread_local std::string g_last_error;
int set_error(int code, const char* f, ...);
int compile_source(const std::string& src, const std::string& arch, const char* name,
                   std::shared_ptr<std::vector<char>>* code);
int device_arch(int dev, std::string* arch, int* cus);
int create_plan(int64_t N, int64_t K, int dtype, int fusion, float norm_eps, proj_plan** out);
void destroy_plan(proj_plan* p);
int run_plan(const proj_plan* p, const void* X, const void* W, void* Y, int64_t M, hipStream_t stream,
             const float* gamma, bool packed, bool noalloc = false);
int check_run_args(const proj_plan* p, const void* X, const void* W, void* Y, int64_t M);
int launch_candidate(const proj_plan* p, const Candidate& c, const void* X, const void* W, void* Y,
                     int64_t M, hipStream_t stream, const float* gamma);

// Shape-independent support module, one per device, loaded on first use.
struct SupportModule {
    hipModule_t mod = nullptr;
    hipFunction_t probe = nullptr, round = nullptr, swiglu_f32 = nullptr, swiglu_bf16 = nullptr, rmsnorm = nullptr,
                  pack = nullptr;
    int cus = 256;
};
static std::mutex g_support_mu;
static std::map<int, SupportModule> g_support;

static int support_module(SupportModule** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_error(PROJ_EDEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lk(g_support_mu);
    SupportModule& sm = g_support[dev];
    if (!sm.mod) {
        std::string arch;
        int rc = device_arch(dev, &arch, &sm.cus);
        if (rc) return rc;
        std::shared_ptr<std::vector<char>> code;
        rc = compile_source(emit_support_source(), arch, "proj_support.hip", &code);
        if (rc) return rc;
        if ((e = hipModuleLoadData(&sm.mod, code->data())) != hipSuccess)
            return set_error(PROJ_EDEVICE, "hipModuleLoadData(support): %s", hipGetErrorString(e));
        if ((e = hipModuleGetFunction(&sm.probe, sm.mod, "proj_probe_read")) != hipSuccess ||
            (e = hipModuleGetFunction(&sm.round, sm.mod, "proj_round_bf16")) != hipSuccess ||
            (e = hipModuleGetFunction(&sm.swiglu_f32, sm.mod, "proj_swiglu_f32")) != hipSuccess ||
            (e = hipModuleGetFunction(&sm.swiglu_bf16, sm.mod, "proj_swiglu_bf16")) != hipSuccess ||
            (e = hipModuleGetFunction(&sm.rmsnorm, sm.mod, "proj_rmsnorm_rows")) != hipSuccess ||
            (e = hipModuleGetFunction(&sm.pack, sm.mod, "proj_pack_panels")) != hipSuccess)
            return set_error(PROJ_EDEVICE, "hipModuleGetFunction(support): %s", hipGetErrorString(e));
    }
    *out = &sm;
    return PROJ_OK;
}

// Whether [a, a + na) and [b, b + nb) share a byte.
static bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

static int copy_text(const std::string& s, char* buf, size_t cap, size_t* needed)
{
    if (needed) *needed = s.size() + 1;
    if (!buf) return cap == 0 ? PROJ_OK : set_error(PROJ_EINVAL, "buffer is NULL");
    if (cap < s.size() + 1)
        return set_error(PROJ_EINVAL, "buffer of %zu bytes is too small (%zu needed)", cap, s.size() + 1);
    memcpy(buf, s.c_str(), s.size() + 1);
    return PROJ_OK;
}

static std::string json_escape(const std::string& s)
{
    std::string o;
    for (char c : s) {
        if (c == '"' || c == '\\') { o += '\\'; o += c; }
        else if (c == '\n') o += "\\n";
        else if ((unsigned char)c < 0x20) { char b[8]; snprintf(b, sizeof b, "\\u%04x", c); o += b; }
        else o += c;
    }
    return o;
}

static std::string describe(const proj_plan* p)
{
    std::ostringstream s;
    s << "{\"N\": " << p->N << ", \"K\": " << p->K << ", \"NO\": " << p->NO << ", \"epilogue\": \""
      << (p->epi ? "swiglu" : "none") << "\", \"prologue\": \"" << (p->pro ? "rmsnorm" : "none")
      << "\", \"norm_eps\": " << p->eps << ", \"layout\": \"" << (p->wpack ? "packed" : "rows")
      << "\", \"dtype\": \"" << (p->dtype ? "bf16" : "f32")
      << "\", \"arch\": \"" << p->arch << "\", \"device\": " << p->device << ", \"compile_s\": " << p->compile_s
      << ", \"tune_s\": " << p->tune_s << ", \"modules\": " << p->modules.size() << ", \"code_bytes\": " << p->code_bytes << ", \"ws_bytes\": " << p->ws_bytes
      << ", \"swiglu_intermediate_rows\": " << p->gu_rows
      << ", \"cache\": \"" << p->cache << "\", \"code_cache\": \"" << p->code_cache << "\", \"cache_path\": \""
      << json_escape(p->cache_path) << "\""
      << ",\n \"candidates\": [";
    for (size_t i = 0; i < p->cands.size(); ++i) s << (i ? ", " : "") << "\"" << p->cands[i].name << "\"";
    s << "],\n \"buckets\": [";
    for (int b = 0; b < kNumBuckets; ++b) {
        s << (b ? ",\n  " : "\n  ") << "{\"lo\": " << kBuckets[b].lo << ", \"hi\": " << kBuckets[b].hi
          << ", \"choice\": \"" << (p->choice[b] >= 0 ? p->cands[p->choice[b]].name : "") << "\", \"us\": "
          << p->choice_us[b] << ", \"timings_us\": {";
        if (b < (int)p->timings.size())
            for (size_t i = 0; i < p->timings[b].size(); ++i)
                s << (i ? ", " : "") << "\"" << p->cands[p->timings[b][i].first].name << "\": "
                  << p->timings[b][i].second;
        s << "}, \"rejected\": [";
        if (b < (int)p->rejected.size())
            for (size_t i = 0; i < p->rejected[b].size(); ++i)
                s << (i ? ", " : "") << "\"" << p->cands[p->rejected[b][i].first].name << "\"";
        s << "]}";
    }
    s << "],\n \"log\": [";
    for (size_t i = 0; i < p->log.size(); ++i) s << (i ? ",\n  " : "\n  ") << "\"" << json_escape(p->log[i]) << "\"";
    s << "]}\n";
    return s.str();
}

}  // namespace proj

using namespace proj;

extern "C" {

proj_plan* proj_plan_create(int64_t N, int64_t K, int dtype)
{
    return proj_plan_create_ex(N, K, dtype, PROJ_EPI_NONE, 0.f);
}

proj_plan* proj_plan_create_ex(int64_t N, int64_t K, int dtype, int fusion, float norm_eps)
{
    g_last_error.clear();
    proj_plan* p = nullptr;
    if (create_plan(N, K, dtype, fusion, norm_eps, &p) != PROJ_OK) return nullptr;
    return p;
}

int proj_run(const proj_plan* plan, const void* X, const void* W, void* Y, int64_t M, hipStream_t stream)
{
    return run_plan(plan, X, W, Y, M, stream, nullptr, false);
}

int proj_run_ex(const proj_plan* plan, const void* X, const void* W, void* Y, int64_t M, const float* gamma,
                hipStream_t stream)
{
    return run_plan(plan, X, W, Y, M, stream, gamma, false);
}

int proj_run_packed(const proj_plan* plan, const void* X, const void* Wp, void* Y, int64_t M, const float* gamma,
                    hipStream_t stream)
{
    return run_plan(plan, X, Wp, Y, M, stream, gamma, true);
}

int proj_run_noalloc(const proj_plan* plan, const void* X, const void* W, void* Y, int64_t M, const float* gamma,
                     hipStream_t stream)
{
    return run_plan(plan, X, W, Y, M, stream, gamma, false, true);
}

int proj_pack_weights(int64_t N, int64_t K, const void* W, void* Wp, hipStream_t stream)
{
    if (N < 0 || K < 0) return set_error(PROJ_EINVAL, "N and K must not be negative");
    if (N % 128 || K % 64)
        return set_error(PROJ_EINVAL, "the packed layout needs N %% 128 == 0 and K %% 64 == 0, got N=%lld K=%lld",
                         (long long)N, (long long)K);
    if (N == 0 || K == 0) return PROJ_OK;
    if (!W || !Wp) return set_error(PROJ_EINVAL, "null pointer (W=%p Wp=%p)", W, Wp);
    if (((uintptr_t)W | (uintptr_t)Wp) & 15) return set_error(PROJ_EINVAL, "W and Wp must be 16-byte aligned");
    const uintptr_t bytes = (uintptr_t)N * (uintptr_t)K * 2, a = (uintptr_t)W, b = (uintptr_t)Wp;
    if (a < b + bytes && b < a + bytes) return set_error(PROJ_EINVAL, "W and Wp overlap");
    SupportModule* sm = nullptr;
    int rc = support_module(&sm);
    if (rc) return rc;
    const void* w = W;
    void* wp = Wp;
    long nn = (long)N, kk = (long)K;
    void* args[] = {&w, &wp, &nn, &kk};
    const unsigned gx = (unsigned)std::min<int64_t>((N * K / 8 + 255) / 256, 65536);
    hipError_t e = hipModuleLaunchKernel(sm->pack, gx, 1, 1, 256, 1, 1, 0, stream, args, nullptr);
    if (e != hipSuccess) return set_error(PROJ_EDEVICE, "pack launch: %s", hipGetErrorString(e));
    return PROJ_OK;
}

void proj_plan_destroy(proj_plan* plan) { destroy_plan(plan); }

const char* proj_last_error(void) { return g_last_error.c_str(); }

int proj_emit_source(int64_t N, int64_t K, int dtype, const char* arch, char* buf, size_t cap, size_t* needed)
{
    return proj_emit_source_ex(N, K, dtype, PROJ_EPI_NONE, 0.f, arch, buf, cap, needed);
}

int proj_emit_source_ex(int64_t N, int64_t K, int dtype, int fusion, float norm_eps, const char* arch, char* buf,
                        size_t cap, size_t* needed)
{
    const int epilogue = fusion & PROJ_EPI_SWIGLU;
    if (fusion & ~(PROJ_EPI_SWIGLU | PROJ_PRO_RMSNORM | PROJ_W_PACKED))
        return set_error(PROJ_EINVAL, "invalid flags %d", fusion);
    if (N < 1 || K < 8 || K % 8 != 0)
        return set_error(PROJ_EINVAL, "invalid shape N=%lld K=%lld", (long long)N, (long long)K);
    if ((fusion & PROJ_W_PACKED) && (N % 128 || K % 64))
        return set_error(PROJ_EINVAL, "the packed layout needs N %% 128 == 0 and K %% 64 == 0");
    if (dtype != PROJ_OUT_F32 && dtype != PROJ_OUT_BF16) return set_error(PROJ_EINVAL, "invalid dtype %d", dtype);
    if (epilogue == PROJ_EPI_SWIGLU && N % 2)
        return set_error(PROJ_EINVAL, "the SwiGLU epilogue needs an even N, got N=%lld", (long long)N);
    const std::string a = (arch && *arch) ? arch : "gfx950";
    return copy_text(emit_source(N, K, dtype, a, kDefaultCUs, enumerate_candidates(N, K, kDefaultCUs, fusion),
                                 fusion, (fusion & PROJ_PRO_RMSNORM) ? norm_eps : 0.f),
                     buf, cap, needed);
}

int proj_compile_only(int64_t N, int64_t K, int dtype, int fusion, float norm_eps, const char* arch, double* seconds)
{
    g_last_error.clear();
    if (seconds) *seconds = 0;
    int rc = proj_emit_source_ex(N, K, dtype, fusion, norm_eps, arch, nullptr, 0, nullptr);
    if (rc) return rc;
    const std::string a = (arch && *arch) ? arch : "gfx950";
    std::vector<Candidate> cands = enumerate_candidates(N, K, kDefaultCUs, fusion);
    const std::vector<std::string> srcs =
        emit_module_sources(N, K, dtype, a, kDefaultCUs, cands, fusion,
                            (fusion & PROJ_PRO_RMSNORM) ? norm_eps : 0.f, kMaxModules);
    char name[96];
    snprintf(name, sizeof name, "proj_%lldx%lld_%s_flags%d", (long long)N, (long long)K, dtype ? "bf16" : "f32",
             fusion);
    const auto t0 = std::chrono::steady_clock::now();
    std::vector<std::shared_ptr<std::vector<char>>> codes;
    rc = compile_sources(srcs, a, name, &codes);
    if (seconds) *seconds = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    return rc;
}

int proj_plan_describe(const proj_plan* plan, char* buf, size_t cap, size_t* needed)
{
    if (!plan) return set_error(PROJ_EINVAL, "plan is NULL");
    return copy_text(describe(plan), buf, cap, needed);
}

int proj_plan_num_candidates(const proj_plan* plan)
{
    if (!plan) return set_error(PROJ_EINVAL, "plan is NULL");
    return (int)plan->cands.size();
}

int proj_plan_candidate_name(const proj_plan* plan, int idx, char* buf, size_t cap)
{
    if (!plan) return set_error(PROJ_EINVAL, "plan is NULL");
    if (idx < 0 || idx >= (int)plan->cands.size()) return set_error(PROJ_EINVAL, "candidate %d out of range", idx);
    return copy_text(plan->cands[idx].name, buf, cap, nullptr);
}

int64_t proj_plan_candidate_max_m(const proj_plan* plan, int idx)
{
    if (!plan) return set_error(PROJ_EINVAL, "plan is NULL");
    if (idx < 0 || idx >= (int)plan->cands.size()) return set_error(PROJ_EINVAL, "candidate %d out of range", idx);
    const Candidate& c = plan->cands[idx];
    int64_t m = c.max_m;
    if (c.SK > 1) m = std::min<int64_t>(m, (int64_t)(plan->ws_bytes / ((size_t)c.SK * plan->N * sizeof(float))));
    if (c.TAILS > 1)  // largest row count whose whole range fits the workspace
        while (m > 0 && c.ws_bound(m, plan->N) > plan->ws_bytes) m -= c.BM;
    return std::max<int64_t>(m, 0);
}

int proj_run_candidate(const proj_plan* plan, int idx, const void* X, const void* W, void* Y, int64_t M,
                       hipStream_t stream)
{
    return proj_run_candidate_ex(plan, idx, X, W, Y, M, nullptr, stream);
}

int proj_run_candidate_ex(const proj_plan* plan, int idx, const void* X, const void* W, void* Y, int64_t M,
                          const float* gamma, hipStream_t stream)
{
    int rc = check_run_args(plan, X, W, Y, M);
    if (rc || M == 0) return rc;
    if (idx < 0 || idx >= (int)plan->cands.size()) return set_error(PROJ_EINVAL, "candidate %d out of range", idx);
    if (plan->pro && (!gamma || ((uintptr_t)gamma & 15)))
        return set_error(PROJ_EINVAL, "this plan has the RMSNorm prologue: a 16-byte aligned gamma is required");
    return launch_candidate(plan, plan->cands[idx], X, W, Y, M, stream, gamma);
}

int proj_plan_choice(const proj_plan* plan, int64_t M)
{
    if (!plan) return set_error(PROJ_EINVAL, "plan is NULL");
    if (M < 1) return set_error(PROJ_EINVAL, "M=%lld must be >= 1", (long long)M);
    return plan->choice[bucket_of(std::min<int64_t>(M, kMaxBlockRows))];
}

int proj_probe_read(const void* buf, int64_t bytes, uint32_t never, void* sink, hipStream_t stream)
{
    if (!buf || !sink) return set_error(PROJ_EINVAL, "null pointer");
    if (bytes < 0 || bytes % 16 || ((uintptr_t)buf & 15) || ((uintptr_t)sink & 3))
        return set_error(PROJ_EINVAL, "buf must be 16-byte aligned with bytes %% 16 == 0, sink 4-byte aligned");
    if (bytes == 0) return PROJ_OK;
    SupportModule* sm = nullptr;
    int rc = support_module(&sm);
    if (rc) return rc;
    const int cus = sm->cus;
    const void* p = buf;
    long n16 = (long)(bytes / 16);
    uint32_t nv = never;
    void* s = sink;
    void* args[] = {&p, &n16, &nv, &s};
    (void)cus;
    const unsigned gx = (unsigned)((n16 + 2047) / 2048);  // one 32 KiB span per block
    hipError_t e = hipModuleLaunchKernel(sm->probe, gx, 1, 1, 256, 1, 1, 0, stream, args, nullptr);
    if (e != hipSuccess) return set_error(PROJ_EDEVICE, "probe launch: %s", hipGetErrorString(e));
    return PROJ_OK;
}

int proj_rmsnorm(const void* X, const float* gamma, void* Xn, int64_t M, int64_t K, float eps, hipStream_t stream)
{
    if (M < 0 || K < 0) return set_error(PROJ_EINVAL, "M and K must not be negative");
    if (!(eps >= 0.f && eps < 1e30f)) return set_error(PROJ_EINVAL, "invalid epsilon %g", (double)eps);
    if (M == 0 || K == 0) return PROJ_OK;
    if (M > 0x7fffffff) return set_error(PROJ_EINVAL, "M=%lld: at most 2^31-1 rows", (long long)M);
    if (!X || !gamma || !Xn) return set_error(PROJ_EINVAL, "null pointer");
    if (((uintptr_t)X | (uintptr_t)Xn) & 1 || (uintptr_t)gamma & 3)
        return set_error(PROJ_EINVAL, "X and Xn must be 2-byte aligned, gamma 4-byte aligned");
    const size_t xb = (size_t)M * (size_t)K * 2;
    if (overlaps(Xn, xb, X, xb) || overlaps(Xn, xb, gamma, (size_t)K * 4))
        return set_error(PROJ_EINVAL, "Xn overlaps X or gamma");
    SupportModule* sm = nullptr;
    int rc = support_module(&sm);
    if (rc) return rc;
    // one block of 256 threads per row, at most 2^20 rows per launch (a launch
    // holds fewer than 2^32 threads)
    constexpr int64_t kRowsPerLaunch = (int64_t)1 << 20;
    for (int64_t m0 = 0; m0 < M; m0 += kRowsPerLaunch) {
        const int64_t rows = std::min(kRowsPerLaunch, M - m0);
        const void* x = (const char*)X + (size_t)m0 * K * 2;
        const float* g = gamma;
        void* xo = (char*)Xn + (size_t)m0 * K * 2;
        long kk = (long)K;
        float e2 = eps;
        void* args[] = {&x, &g, &xo, &kk, &e2};
        hipError_t e = hipModuleLaunchKernel(sm->rmsnorm, (unsigned)rows, 1, 1, 256, 1, 1, 0, stream, args, nullptr);
        if (e != hipSuccess) return set_error(PROJ_EDEVICE, "rmsnorm launch: %s", hipGetErrorString(e));
    }
    return PROJ_OK;
}

int proj_swiglu(const void* G, void* H, int64_t M, int64_t N, int dtype, hipStream_t stream)
{
    if (M < 0 || N < 0) return set_error(PROJ_EINVAL, "M and N must not be negative");
    if (N % 2) return set_error(PROJ_EINVAL, "N=%lld must be even (gate and up halves)", (long long)N);
    if (dtype != PROJ_OUT_F32 && dtype != PROJ_OUT_BF16) return set_error(PROJ_EINVAL, "invalid dtype %d", dtype);
    if (M == 0 || N == 0) return PROJ_OK;
    if (!G || !H) return set_error(PROJ_EINVAL, "null pointer");
    const size_t es = dtype == PROJ_OUT_BF16 ? 2 : 4;
    if (((uintptr_t)G | (uintptr_t)H) & (es - 1))
        return set_error(PROJ_EINVAL, "G and H must be aligned to their element size (%zu bytes)", es);
    if (overlaps(G, (size_t)M * (size_t)N * es, H, (size_t)M * (size_t)(N / 2) * es))
        return set_error(PROJ_EINVAL, "H overlaps G");
    SupportModule* sm = nullptr;
    int rc = support_module(&sm);
    if (rc) return rc;
    const void* g = G;
    void* h = H;
    long mm = (long)M, nn = (long)N;
    void* args[] = {&g, &h, &mm, &nn};
    const unsigned gx = (unsigned)std::min<int64_t>(65536, (M * (N / 2) + 255) / 256);
    hipError_t e = hipModuleLaunchKernel(dtype == PROJ_OUT_BF16 ? sm->swiglu_bf16 : sm->swiglu_f32, gx, 1, 1, 256, 1,
                                         1, 0, stream, args, nullptr);
    if (e != hipSuccess) return set_error(PROJ_EDEVICE, "swiglu launch: %s", hipGetErrorString(e));
    return PROJ_OK;
}

int proj_round_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t stream)
{
    if (n < 0) return set_error(PROJ_EINVAL, "n is negative");
    if (n == 0) return PROJ_OK;
    if (!in || !out) return set_error(PROJ_EINVAL, "null pointer");
    if ((uintptr_t)in & 3 || (uintptr_t)out & 1) return set_error(PROJ_EINVAL, "in must be 4-byte, out 2-byte aligned");
    if (overlaps(in, (size_t)n * 4, out, (size_t)n * 2)) return set_error(PROJ_EINVAL, "out overlaps in");
    SupportModule* sm = nullptr;
    int rc = support_module(&sm);
    if (rc) return rc;
    const float* i = in;
    uint16_t* o = out;
    long nn = (long)n;
    void* args[] = {&i, &o, &nn};
    const unsigned gx = (unsigned)std::min<int64_t>(65536, (n + 255) / 256);
    hipError_t e = hipModuleLaunchKernel(sm->round, gx, 1, 1, 256, 1, 1, 0, stream, args, nullptr);
    if (e != hipSuccess) return set_error(PROJ_EDEVICE, "round launch: %s", hipGetErrorString(e));
    return PROJ_OK;
}

}  // extern "C"
