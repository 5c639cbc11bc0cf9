// kernels.hip -- device code of the projection library, Y[M,N] = X[M,K] . W[N,K]^T.
//
// This file is not compiled on its own.  At plan creation the host prepends a
// prelude that fixes the shape as literals,
//     constexpr long N = <rows of W>;  constexpr long K = <row length>;
// and appends one extern "C" wrapper per candidate whose template arguments
// (tile sizes, splits, trip counts) are literals too; hipRTC then compiles the
// whole translation unit for the GPU in front of it.  So every loop bound,
// trip count and weight-row stride below is a compile-time constant, and the
// only value read at run time is the row count M.  This is the blog series
// "On descend d'un cran" applied to gfx950: "#001 un compilateur pour moteur de
// LLM", section "Un compilateur, pas une bibliotheque de kernels" (trip counts
// and offsets to the next weight block are immediates; the row count of a
// block is the one run-time dimension) and "#002 le meme compilateur sur un
// GPU", section "Emettre pour un GPU" (one module per kernel, the shape and the
// device's properties written into it as constants).
//
// Layouts: X [M,K] and Y [M,N] are dense row-major; W [N,K] is row-major or,
// with WPACK = 1, in the panel layout (below); X and W hold bf16 bit
// patterns; Y holds f32 or bf16.  Products and sums are f32 (bf16 widens to
// f32 exactly); the bf16 output is one round-to-nearest-even of the final f32
// sum.  Contract: "On descend d'un cran" (post 0), section "Ce qu'il y aura
// dans le depot"; "#004 the same compiler on Apple's chips", opening section
// (IEEE-rounded add/mul/FMA, round only where the reference rounds).

// (types and the dev:: helpers come from device_common.hip, prepended by the host)


// Weight addressing in 16-byte chunks from W: chunk c of weight row n (values
// 8c .. 8c+7) is chunk w_row(n) + w_col(c).  WPACK (a constant of the
// prelude) selects the layout: 0 row-major, n * K/8 + c; 1 the panel layout of
// dev::kPanelRows x dev::kPanelCols blocks (see device_common), written once at
// load by proj_pack_panels.  Both terms are for n, c >= 0.  Moving 64 chunks
// along a row adds W_TRIP in either layout.
static_assert(dev::kPanelRows == 128 && dev::kPanelCols == 64, "the shifts below assume 128 x 64 blocks");
static_assert(WPACK == 0 || (N % dev::kPanelRows == 0 && K % dev::kPanelCols == 0),
              "the panel layout needs whole panels and blocks");
__device__ __forceinline__ long w_row(long n)
{
    if constexpr (WPACK) return (n >> 7) * (16 * K) + (n & 127) * 8;
    else return n * (K / 8);
}
__device__ __forceinline__ long w_col(long c)
{
    if constexpr (WPACK) return (c >> 3) * 1024 + (c & 7);
    else return c;
}
constexpr long W_TRIP = WPACK ? 8 * 1024 : 64;
