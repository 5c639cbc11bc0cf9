// codegen.cpp -- candidate enumeration and HIP source emission for one (N, K).
//
// The host writes the code that will compute, for one precise shape: the
// emitter idea of the blog series "On descend d'un cran" ("#001 un compilateur
// pour moteur de LLM", section "Un compilateur, pas une bibliotheque de
// kernels"), here producing HIP C++ for hipRTC instead of machine code.  Every
// known dimension -- N, K, the row length in 16-byte blocks, the last row
// index, per-candidate trip counts and strides -- appears in the emitted text
// as a literal; a candidate is only emitted when its tiles divide the shape, so
// no kernel carries remainder code for N or K.  Only M stays a run-time value.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <sstream>

#include "proj_internal.h"

namespace proj {

int bucket_of(int64_t M)
{
    for (int b = 0; b < kNumBuckets; ++b)
        if (M <= kBuckets[b].hi) return b;
    return kNumBuckets - 1;
}

static std::string fmt(const char* f, ...) __attribute__((format(printf, 1, 2)));
static std::string fmt(const char* f, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, f);
    vsnprintf(buf, sizeof buf, f, ap);
    va_end(ap);
    return buf;
}

static std::vector<Candidate> enumerate_family(int64_t N, int64_t K, int cus, int fusion);

std::vector<Candidate> enumerate_candidates(int64_t N, int64_t K, int cus, int fusion)
{
    if (!(fusion & 1)) return enumerate_family(N, K, cus, fusion);
    // SwiGLU plans: the candidates with the activation fused into their epilogue,
    // then every plain candidate (not the plain kernel) run unfused -- the
    // projection into the plan's intermediate, then the activation kernel --
    // so that the tuner measures the fusion against the kernels it replaces;
    // the fused plain kernel stays last (the tuner's last resort)
    std::vector<Candidate> out = enumerate_family(N, K, cus, fusion);
    Candidate plain = out.back();
    out.pop_back();
    for (Candidate& c : out) c.E = 1;
    for (Candidate c : enumerate_family(N, K, cus, fusion & ~1)) {
        if (c.fam == Family::Plain) continue;
        c.UF = 1;
        c.name += "_uf";
        if (c.TAILS > 1) c.reduce_name = c.name + "_reduce";
        out.push_back(c);
    }
    plain.E = 1;
    out.push_back(plain);
    return out;
}

static std::vector<Candidate> enumerate_family(int64_t N, int64_t K, int cus, int fusion)
{
    const int epi = fusion & 1, pro = (fusion & 2) ? 1 : 0, wpack = (fusion & 4) ? 1 : 0;
    std::vector<Candidate> out;
    const int64_t CH = K / 8;  // 16-byte chunks per row

    // ---- vector-ALU GEMV: (R rows per wave, S waves splitting K), MMAX rows of X
    struct VG { int R, S, MMAX, NT, NW, KX = 1; };
    // (listed in order of preference: the tuner keeps an earlier candidate unless
    //  a later one is clearly faster).  NW: waves per block; 5 and 8 make a whole
    //  number of blocks per CU where 4 does not (5120 rows in waves of 2 rows:
    //  640 blocks of 4 waves, 2.5 per CU; 512 blocks of 5 waves, 2 per CU).
    const VG vgs[] = {{2, 1, 1, 1, 4}, {1, 1, 1, 1, 4}, {4, 1, 1, 1, 4}, {2, 1, 1, 0, 4},
                      {1, 4, 1, 1, 4}, {2, 4, 1, 1, 4}, {1, 1, 16, 1, 4}, {2, 1, 16, 1, 4}, {1, 4, 16, 1, 4},
                      {2, 1, 1, 1, 5}, {1, 1, 1, 1, 5}, {4, 1, 1, 1, 5}, {2, 1, 1, 1, 8}, {1, 2, 1, 1, 8},
                      // K split across 2, 4 or 8 workgroups (CUs), the partials added in a fixed order
                      {2, 1, 1, 1, 4, 2}, {2, 1, 1, 1, 4, 4}, {1, 1, 1, 1, 4, 4}, {1, 1, 1, 1, 4, 8}};
    for (const VG& v : vgs) {
        if (CH % (v.S * v.KX)) continue;
        // split across workgroups: long rows only (K >= 8192: a row's slices
        // then still stream several KiB each), whole 64-lane trips per slice,
        // the plain epilogue, and N % 4 == 0 for the 4-wide split-K sum
        if (v.KX > 1 && (K < 8192 || epi || CH / v.KX < 64 || N % 4)) continue;
        if (epi && v.R % 2) continue;   // the fused epilogue pairs gate and up rows in a wave
        const int RG = v.NW / v.S;
        if (N % (v.R * RG)) continue;
        // other wave counts only where they change the block count per CU
        if (v.NW != 4 && (N / (v.R * RG)) % cus != 0) continue;
        const int64_t trips = CH / (v.S * v.KX) / 64;
        int U = 1;
        for (int u : {4, 2}) {
            if (trips > 0 && trips % u == 0 && u * v.R <= 8) { U = u; break; }
        }
        Candidate c;
        c.fam = Family::GemvValu;
        c.R = v.R; c.S = v.S; c.MMAX = v.MMAX; c.U = U; c.NT = v.NT; c.NW = v.NW; c.KX = v.KX;
        if (v.KX > 1) c.reduce_name = fmt("splitk_reduce_sk%d", v.KX);
        c.threads = 64 * v.NW;
        c.max_m = v.MMAX;
        const std::string wsuf = (v.NW != 4 ? fmt("_w%d", v.NW) : std::string()) +
                                 (v.KX > 1 ? fmt("_x%d", v.KX) : std::string());
        c.name = fmt("gemv_valu_r%d_s%d_m%d_u%d_nt%d", c.R, c.S, c.MMAX, c.U, c.NT) + wsuf;
        out.push_back(c);
        // the same with pipelined batches: the largest U that still leaves a
        // wave two batches or more
        if (v.MMAX == 1 && v.NT == 1) {
            int Up = 0;
            for (int u : {4, 2, 1})
                if (trips > 0 && trips % u == 0 && u * v.R <= 8 && trips / u >= 2) { Up = u; break; }
            if (Up) {
                c.U = Up;
                c.P = 1;
                c.name = fmt("gemv_valu_r%d_s%d_m%d_u%d_nt%d_p", c.R, c.S, c.MMAX, c.U, c.NT) + wsuf;
                out.push_back(c);
            }
        }
    }

    // ---- with the RMSNorm prologue: every candidate also runs unfused (the norm
    //      kernel into the plan's workspace, then the candidate on it); the M = 1
    //      vector GEMVs come a second time with the norm folded in ("_nf")
    if (pro) {
        const size_t n = out.size();
        for (size_t i = 0; i < n; ++i)
            if (out[i].fam == Family::GemvValu && out[i].MMAX == 1 && out[i].NW == 4 && out[i].KX == 1) {
                Candidate c = out[i];
                c.PRO = 1;
                c.name += "_nf";
                out.push_back(c);
            }
    }

    // ---- MFMA skinny GEMV for M <= 16: (S waves splitting K, U MFMA steps per load batch)
    for (int S : {1, 2, 4}) {
        if (epi) break;                 // no fused epilogue in the MFMA GEMV
        for (int U : {2, 4}) {
            if (wpack && U % 2) continue;   // panel layout: a batch is whole 8-chunk block rows
            const int RG = 4 / S;
            if (N % (16 * RG)) continue;
            if (K % (32 * U * S)) continue;
            Candidate c;
            c.fam = Family::GemvMfma;
            c.S = S; c.U = U; c.NT = 1;
            c.threads = 256;
            c.max_m = 16;
            c.name = fmt("gemv_mfma_s%d_u%d_nt%d", c.S, c.U, c.NT);
            out.push_back(c);
        }
    }

    // ---- MFMA GEMM: block tile BM x BN, k-tile BK, ST LDS buffers, WM x WN waves,
    //      LDS swizzle period SWZ, split-K SK (only for the smaller tiles).
    //      gfx950's LDS serves a 16-byte-per-lane read 16 lanes (256 bytes, all 64
    //      banks) at a time, so the 16 rows one operand read touches must land on
    //      distinct bank groups: XOR period 2 rows for 128-byte rows (BK = 64),
    //      4 rows for 64-byte rows (BK = 32).
    //      Each entry also lists the K-split factors of its split-tail variants
    //      (whole tiles for all full rounds of workgroups, the remaining tiles
    //      split along K so the last round is not mostly idle; a factor that does
    //      not divide the k-tile count gives pieces of two lengths, e.g. three or
    //      six pieces for the 40 tail tiles of 2560-column shapes at M = 512).
    // BST = ST + 1: one more LDS buffer for W than for X (W copies a k-tile further ahead).
    // At a few hundred rows the GEMM streams W from HBM much as the GEMV does, and
    // a 128 x 128 tile with four W buffers keeps more of it in flight per CU.
    // kp: the entry also gets whole-tile and split-tail variants whose tiles visit
    // the k-tiles of each block of four in a rotated order of their own (KP = 4),
    // so tiles sharing a W or X panel under one L2 do not all miss on the same
    // k-tile at once; given to the tiles the tuner picks across the workloads.
    struct GT { int BM, BN, BK, ST, WM, WN, SWZ, maxSK, GM, DMA; int tails[5]; int BST = 0; bool kp = false; };
    const GT gts[] = {
        {256, 256, 64, 2, 2, 4, 1, 1, 8, 1, {2, 4}}, {256, 256, 64, 2, 2, 4, 1, 1, 4, 1, {2}},
        {256, 256, 64, 2, 2, 4, 1, 1, 8, 1, {2, 4}, 3, true},
        {192, 256, 64, 2, 2, 4, 1, 1, 8, 1, {2, 4}, 3, true},
        {256, 128, 64, 3, 4, 2, 1, 1, 4, 1, {2, 3, 4, 6}, 0, true}, {256, 128, 64, 3, 4, 2, 1, 1, 8, 1, {}},
        {256, 128, 64, 3, 4, 2, 1, 1, 4, 1, {2, 4}, 4},
        {128, 256, 64, 3, 2, 4, 1, 1, 4, 1, {2, 4}},
        {128, 128, 64, 2, 2, 2, 1, 8, 8, 1, {2, 4}}, {128, 128, 64, 2, 2, 2, 1, 2, 8, 0, {}},
        {128, 128, 64, 3, 2, 2, 1, 8, 8, 1, {2, 3, 4, 6}, 4},
        {128, 64, 64, 3, 2, 2, 1, 8, 8, 1, {2, 3, 4, 6}, 4, true},
        {128, 128, 32, 3, 2, 2, 2, 4, 8, 1, {}}, {64, 128, 64, 2, 1, 2, 1, 8, 8, 1, {}},
        // tiles 160 or 192 wide make whole rounds of 256 CUs where the power-of-two
        // widths leave part of a round: 5120 columns at 2048 rows are 8 x 32
        // tiles of 256 x 160, 2560 columns 16 x 16 tiles of 128 x 160, 18432
        // columns 8 x 96 tiles of 256 x 192 (160 = five 32-column MFMA blocks:
        // one wave column, so four waves of 64 x 160 or 32 x 160)
        {256, 160, 64, 2, 4, 1, 1, 1, 8, 1, {2}, 3}, {128, 160, 64, 3, 4, 1, 1, 1, 8, 1, {2}, 4, true},
        {256, 192, 64, 2, 4, 2, 1, 1, 8, 1, {2}, 3},
        // four X and five W buffers: more k-tiles in flight per workgroup for the
        // few-hundred-row blocks, whose copies wait on HBM
        {128, 128, 64, 4, 2, 2, 1, 1, 8, 1, {2, 3, 4, 6}, 5}, {128, 64, 64, 4, 2, 2, 1, 1, 8, 1, {2, 3, 4, 6}, 5},
        // W rings two to four buffers deeper than X's (the tuner's choice: they
        // time within about 1 % of the one-deeper ring, because a wave's copies
        // complete in order and its wait for X also covers the W copies it issued
        // before; the 256 x 192 tile with four W buffers wins at 2048 rows)
        {128, 128, 64, 3, 2, 2, 1, 1, 8, 1, {2, 3, 4, 6}, 6}, {128, 128, 64, 2, 2, 2, 1, 1, 8, 1, {2, 3, 4, 6}, 5},
        {128, 64, 64, 2, 2, 2, 1, 1, 8, 1, {2, 3, 4, 6}, 6}, {128, 160, 64, 3, 4, 1, 1, 1, 8, 1, {2}, 5},
        {256, 128, 64, 2, 4, 2, 1, 1, 4, 1, {2, 3, 4, 6}, 5}, {256, 192, 64, 2, 4, 2, 1, 1, 8, 1, {2}, 4, true},
        // 96 columns (three 32-column MFMA blocks, four waves of 32 x 96)
        {128, 96, 64, 3, 4, 1, 1, 1, 8, 1, {2}, 4, true}};
    for (const GT& g : gts) {
        if (N % g.BN) continue;
        if (wpack && 64 % g.BK) continue;  // panel layout: a k-tile inside one 64-value block
        const int cpr = g.BK / 8, rpi = 64 * g.WM * g.WN / cpr;
        if ((rpi >> g.SWZ) % cpr) continue;  // the copy slots' swizzled column must not vary per copy
        const int lds = (g.BST ? g.ST * g.BM + g.BST * g.BN : g.ST * (g.BM + g.BN)) * g.BK * 2;
        if (lds > 160 * 1024) continue;   // the LDS of one workgroup
        const int per_cu = std::max(1, std::min(2, 160 * 1024 / lds));
        auto add = [&](int SK, int TL, int KP = 0) {
            Candidate c;
            c.fam = Family::Gemm;
            c.BM = g.BM; c.BN = g.BN; c.BK = g.BK; c.ST = g.ST; c.WM = g.WM; c.WN = g.WN;
            c.SK = SK; c.GM = g.GM; c.SWZ = g.SWZ; c.DMA = g.DMA; c.BST = g.BST;
            c.TAILS = TL;
            c.KP = KP;
            c.ROUND = TL > 1 ? cus * per_cu : 0;
            c.threads = 64 * g.WM * g.WN;
            c.max_m = kMaxBlockRows;
            c.name = fmt("gemm_%dx%dx%d_st%d_w%dx%d_sw%d_g%d_sk%d%s%s", c.BM, c.BN, c.BK, c.ST, c.WM, c.WN, c.SWZ,
                         c.GM, c.SK, c.DMA ? "" : "_reg", c.BST ? fmt("_b%d", c.BST).c_str() : "");
            if (KP > 1) c.name += fmt("_kp%d", KP);
            if (TL > 1) c.name += fmt("_tail%d_r%d", TL, c.ROUND);
            if (SK > 1) c.reduce_name = fmt("splitk_reduce_sk%d", SK);
            if (TL > 1) c.reduce_name = c.name + "_reduce";
            out.push_back(c);
        };
        if (epi) {                      // fused epilogue: whole tiles, gate/up halves per wave
            if ((g.BN / g.WN) % 64 == 0 && K % g.BK == 0) add(1, 1);
            continue;
        }
        for (int SK : {1, 2, 4, 8})
            if (SK <= g.maxSK && K % (g.BK * SK) == 0) add(SK, 1);
        for (int TL : g.tails)   // pieces of at least two k-tiles (KT / TL or one more)
            if (TL > 1 && K % g.BK == 0 && K / g.BK >= 2 * TL) add(1, TL);
        if (g.kp && K % (4 * g.BK) == 0) {   // whole tiles of whole blocks of four k-tiles
            add(1, 1, 4);
            for (int TL : g.tails)
                if (TL > 1 && K / g.BK >= 2 * TL) add(1, TL, 4);
        }
    }

    // ---- plain kernel, any shape (K % 8 == 0)
    Candidate p;
    p.fam = Family::Plain;
    p.threads = 256;
    p.max_m = kMaxBlockRows;
    p.name = "gemm_plain";
    out.push_back(p);
    return out;
}

std::string emit_support_source()
{
    std::string s;
    s += "// libproj support module (shape-independent)\n";
    s += kDeviceCommonSrc;
    s += "\n";
    s += kSupportSrc;
    return s;
}

// The shape prelude: the constants of (N, K, dtype, fusion) as literals, then
// the device helpers and kernel templates every module of the plan shares.
static std::string emit_prelude(int64_t N, int64_t K, int dtype, const std::string& arch, int cus, int fusion,
                                float norm_eps)
{
    const int epi = fusion & 1, wpack = (fusion & 4) ? 1 : 0;
    char eps_lit[64];
    snprintf(eps_lit, sizeof eps_lit, "%a", (double)norm_eps);
    std::ostringstream s;
    s << "// Generated by libproj for Y[M," << N << "] = X[M," << K << "] . W[" << N << "," << K
      << "]^T, output " << (dtype == 1 ? "bf16" : "f32") << ", target " << arch
      << (epi ? ", SwiGLU epilogue: Y[M, N/2] = silu(gate) * up" : "")
      << ((fusion & 2) ? ", RMSNorm prologue on X" : "")
      << (wpack ? ", W in the panel layout (128-row panels of 128 x 64 blocks)" : "") << ".\n";
    s << "// Every constant below is an immediate of the kernels; M is the only run-time size.\n";
    s << "constexpr long N = " << N << ";            // output rows = rows of W\n";
    s << "constexpr long K = " << K << ";            // row length (bf16 values)\n";
    s << "constexpr long K_BLOCKS16 = " << K / 8 << ";    // 16-byte (8 x bf16) blocks per weight row\n";
    s << "constexpr long N_LAST = " << N - 1 << ";       // last output row index\n";
    s << "constexpr long ROW_BYTES = " << 2 * K << ";    // stride between weight rows\n";
    s << "constexpr int DEVICE_CUS = " << cus << ";     // compute units of the device the code is for\n";
    s << "constexpr int EPI = " << epi << ";            // epilogue: 0 none, 1 SwiGLU of gate rows [0, N/2) and up rows [N/2, N)\n";
    s << "constexpr long NOUT = " << (epi ? N / 2 : N) << ";         // columns of Y\n";
    s << "constexpr int OUT_SEL = " << dtype << ";        // storage type of Y: 0 f32, 1 bf16\n";
    s << "constexpr int WPACK = " << wpack << ";          // layout of W: 0 row-major, 1 panels of 128 rows x 64-value blocks\n";
    s << "constexpr float NORM_EPS = " << eps_lit << "f;   // RMSNorm epsilon of the fused prologue ("
      << ((fusion & 2) ? "" : "unused: ") << norm_eps << ")\n\n";
    s << kDeviceCommonSrc << "\n";
    s << kKernelsHeadSrc << "\n";
    s << kGemvSrc << "\n";
    s << kGemmSrc << "\n";
    return s.str();
}

// The extern "C" wrapper(s) of one candidate: its template instantiated with
// literal arguments, plus its second-pass kernel.  A split-K reduce kernel is
// shared by the candidates of one split factor: `reduce_emitted` (indexed by
// SK) records which the module already holds.
static void emit_wrappers(std::ostringstream& s, const Candidate& c, int64_t N, int64_t K, int dtype, int wpack,
                          bool reduce_emitted[9])
{
    const char* out = dtype == 1 ? "OUT_BF16" : "OUT_F32";
    // how the candidate comments below describe the weight stream
    const std::string wdesc = wpack ? std::string("weights in 16 KiB panel blocks")
                                    : fmt("weight row stride %lld B", (long long)(2 * K));
    const char* sig = "(const u16* __restrict__ X, const u16* __restrict__ W, void* __restrict__ Y, "
                      "float* __restrict__ ws, const float* __restrict__ gamma, int M)";
    switch (c.fam) {
    case Family::GemvValu: {
        const int64_t chs = K / 8 / c.S;
        s << "// " << c.name << ": " << c.R << " row(s)/wave, K split " << c.S << " ways, "
          << chs << " blocks/slice = " << chs / 64 << " trip(s) of 64 lanes + " << chs % 64
          << " tail lanes, " << wdesc << "\n";
        s << "static_assert(K_BLOCKS16 / " << c.S << " / 64 == " << chs / 64 << ", \"trip count\");\n";
        s << "extern \"C\" __global__ __launch_bounds__(" << 64 * c.NW << ") void " << c.name << sig
          << "\n{ gemv_valu<" << c.R << ", " << c.S << ", " << c.MMAX << ", " << c.U << ", " << c.NT << ", " << out
          << ", " << c.P << ", " << c.PRO << ", " << c.E << ", " << c.NW << ", " << c.KX
          << ">(X, W, Y, gamma, M, ws); }\n";
        if (c.KX > 1 && !reduce_emitted[c.KX]) {   // the GEMM's split-K sum serves the split GEMV too
            reduce_emitted[c.KX] = true;
            s << "extern \"C\" __global__ __launch_bounds__(256) void " << c.reduce_name
              << "(const float* __restrict__ ws, void* __restrict__ Y, int M)\n{ splitk_reduce<" << c.KX
              << ", " << out << ">(ws, Y, M); }\n";
        }
        break;
    }
    case Family::GemvMfma: {
        const int64_t batches = K / c.S / (32 * c.U);
        s << "// " << c.name << ": 16 rows/wave on mfma_16x16x32_bf16, K split " << c.S << " ways, "
          << batches << " batch(es) of " << c.U << " MFMA steps, " << wdesc << ", next 16-row weight block at +"
          << (wpack ? 16 * 64 * 2 : 32 * K) << " B\n";
        s << "static_assert(K / " << c.S << " / " << 32 * c.U << " == " << batches << ", \"trip count\");\n";
        s << "extern \"C\" __global__ __launch_bounds__(256) void " << c.name << sig << "\n{ gemv_mfma<"
          << c.S << ", " << c.U << ", " << c.NT << ", " << out << ">(X, W, Y, M); }\n";
        break;
    }
    case Family::Gemm: {
        const int64_t kt = K / c.SK / c.BK;
        s << "// " << c.name << ": " << c.BM << "x" << c.BN << " tile, " << c.WM * c.WN << " waves, "
          << c.ST << " LDS buffers of " << (c.BM + c.BN) * c.BK * 2 << " B, K split " << c.SK << " ways, "
          << kt << " k-tile(s) of " << c.BK << ", " << N / c.BN << " tile column(s), " << wdesc << "\n";
        s << "static_assert(K / " << c.SK << " / " << c.BK << " == " << kt << ", \"trip count\");\n";
        s << "extern \"C\" __global__ __launch_bounds__(" << c.threads << ") void " << c.name << sig
          << "\n{ gemm_mfma<" << c.BM << ", " << c.BN << ", " << c.BK << ", " << c.ST << ", " << c.WM << ", "
          << c.WN << ", " << c.SK << ", " << c.GM << ", " << c.SWZ << ", " << out << ", " << c.DMA << ", "
          << c.TAILS << ", " << c.ROUND << ", " << c.E << ", " << c.BST << ", " << c.KP << ">(X, W, Y, ws, M); }\n";
        if (c.TAILS > 1) {
            s << "// " << c.reduce_name << ": tail tiles of " << c.name << ", " << c.TAILS
              << " pieces each, rounds of " << c.ROUND << " workgroups\n";
            s << "extern \"C\" __global__ __launch_bounds__(256) void " << c.reduce_name
              << "(const float* __restrict__ ws, void* __restrict__ Y, int M)\n{ tail_reduce<" << c.BM << ", "
              << c.BN << ", " << c.TAILS << ", " << c.ROUND << ", " << c.GM << ", " << out << ">(ws, Y, M); }\n";
        }
        if (c.SK > 1 && !reduce_emitted[c.SK]) {
            reduce_emitted[c.SK] = true;
            s << "extern \"C\" __global__ __launch_bounds__(256) void " << c.reduce_name
              << "(const float* __restrict__ ws, void* __restrict__ Y, int M)\n{ splitk_reduce<" << c.SK
              << ", " << out << ">(ws, Y, M); }\n";
        }
        break;
    }
    case Family::Plain:
        s << "// gemm_plain: one thread per output, " << K / 8 << " blocks of 16 bytes per dot product\n";
        s << "extern \"C\" __global__ __launch_bounds__(256) void " << c.name << sig
          << "\n{ gemm_plain<" << out << ", " << c.E << ">(X, W, Y, M); }\n";
        break;
    }
}

static const char* const kCandidatesBanner = "// ===================== candidates for this shape =====================\n";

std::string emit_source(int64_t N, int64_t K, int dtype, const std::string& arch, int cus,
                        const std::vector<Candidate>& cands, int fusion, float norm_eps)
{
    std::ostringstream s;
    s << emit_prelude(N, K, dtype, arch, cus, fusion, norm_eps);
    s << kGateSrc << "\n";
    s << kSupportSrc << "\n";
    s << kCandidatesBanner;
    bool reduce_emitted[9] = {};    // split-K reduce kernels already emitted, by SK (at most 8)
    for (const Candidate& c : cands) emit_wrappers(s, c, N, K, dtype, (fusion & 4) ? 1 : 0, reduce_emitted);
    return s.str();
}

// Rough relative compile cost of a candidate's wrappers (hipRTC time of one
// instantiation, measured: a tiled GEMM ~0.6 s, a 16-row vector GEMV ~0.7 s,
// a one-row GEMV ~0.25 s, an MFMA GEMV ~0.12 s), used to balance the modules.
static int compile_cost(const Candidate& c)
{
    switch (c.fam) {
    case Family::Gemm: return 6 + (c.TAILS > 1 ? 1 : 0);
    case Family::GemvValu: return c.MMAX > 1 ? 7 : 3;
    case Family::GemvMfma: return 2;
    case Family::Plain: default: return 1;
    }
}

std::vector<std::string> emit_module_sources(int64_t N, int64_t K, int dtype, const std::string& arch, int cus,
                                             std::vector<Candidate>& cands, int fusion, float norm_eps,
                                             int max_modules)
{
    const std::string prelude = emit_prelude(N, K, dtype, arch, cus, fusion, norm_eps);
    const int G = std::max(1, std::min<int>(max_modules, (int)cands.size()));
    // longest-first onto the least loaded module; module 0 also carries the
    // support kernels (validation gate, probes, pack, norm, activation)
    std::vector<int> order(cands.size());
    for (size_t i = 0; i < cands.size(); ++i) order[i] = (int)i;
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return compile_cost(cands[a]) > compile_cost(cands[b]); });
    std::vector<int> load(G, 0);
    load[0] = 5;
    for (int i : order) {
        int g = 0;
        for (int j = 1; j < G; ++j)
            if (load[j] < load[g]) g = j;
        cands[i].module = g;
        load[g] += compile_cost(cands[i]);
    }
    std::vector<std::string> out;
    for (int g = 0; g < G; ++g) {
        std::ostringstream s;
        s << prelude;
        if (g == 0) s << kGateSrc << "\n" << kSupportSrc << "\n";
        s << kCandidatesBanner;
        bool reduce_emitted[9] = {};
        for (const Candidate& c : cands)
            if (c.module == g) emit_wrappers(s, c, N, K, dtype, (fusion & 4) ? 1 : 0, reduce_emitted);
        out.push_back(s.str());
    }
    return out;
}

}  // namespace proj
