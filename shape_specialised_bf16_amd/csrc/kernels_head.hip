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
// Layouts: X [M,K], W [N,K] and Y [M,N] are dense row-major; X and W hold bf16
// bit patterns; Y holds f32 or bf16.  Products and sums are f32 (bf16 widens to
// f32 exactly); the bf16 output is one round-to-nearest-even of the final f32
// sum.  Contract: "On descend d'un cran" (post 0), section "Ce qu'il y aura
// dans le depot"; "#004 the same compiler on Apple's chips", opening section
// (IEEE-rounded add/mul/FMA, round only where the reference rounds).

// (types and the dev:: helpers come from device_common.hip, prepended by the host)

