// gemv.hip -- decode kernels for M <= 16 (part of the shape module; see kernels_head.hip)

// ---------------------------------------------------------------------------
// Decode GEMV on the vector ALU (M <= MMAX, MMAX small).
//
// One wave walks R rows of W; lane l reads 16-byte chunk l, l+64, l+128, ... of
// each row, so one load instruction covers 1 KiB of a row contiguously.  The
// GPU analogue of the pages' decode module: one subgroup per output row,
// lanes striding over 16-byte (8 x bf16) blocks of the weight row, the row
// length in blocks and the row count as constants ("#002 le meme compilateur
// sur un GPU", section "Emettre pour un GPU").  The S waves of a row group
// split K and combine through LDS in a fixed order.  With W in the panel
// layout the same chunks are read in the same order (so the sums are the
// same); a load instruction then covers 8 runs of 128 bytes, 16 KiB apart.
//
// With P = 1 (M = 1 only) the batches of U trips are software-pipelined: the
// loads of batch b+1 (weights and the matching X chunks) are issued before the
// dot products of batch b, so a wave keeps a batch in flight from its first
// load to its last instead of waiting out one memory round trip per batch --
// what long rows (K of several thousand) need.
//
// With the SwiGLU epilogue (E == 1, in a module whose W is a gate_up matrix)
// a wave's R rows are R/2 gate rows j.. and their up rows N/2 + j..; after the
// reduction the up sum of a gate value sits 32 lanes above it, and the wave
// stores silu(gate) * up in column j of Y [M, N/2].  With E == 0 the kernel
// writes all N sums (Y [M, N]).
//
// With the RMSNorm prologue (PRO == 1, M = 1 only) the block first
// normalises the X row into LDS with the same dev::rms_scale_block and
// dev::rms_apply as the separate norm kernel (gamma f32 [K], epsilon NORM_EPS),
// then reads X from there: the norm run inside the next projection's kernel
// ("#004 the same compiler on Apple's chips", section "Decode").  Each
// block re-reads the K-element row, the extra traffic the pages name as the
// reason the fused norm loses on larger models.
//
// With KX > 1 (M = 1) the K range is also split across workgroups, so across
// CUs: block (g, x) sums slice x of K for its rows and writes the f32 partials
// to ws[x][n]; a second kernel (splitk_reduce, the GEMM's) adds the KX
// partials of each output in ascending x, a fixed order, so the result does
// not depend on which block finished first.
//
// Block: NW waves = (NW/S) row groups x S K-slices (NW = 4 by default; other
// counts let the grid be a whole number of blocks per CU, e.g. 5 waves of 2
// rows make 512 blocks of 5120 rows: two per CU, all resident at once).
// Grid:  N / (R * NW/S) x KX blocks.
// ---------------------------------------------------------------------------
template <int R, int S, int MMAX, int U, int NT, int OUT, int P = 0, int PRO = 0, int E = 0, int NW = 4, int KX = 1>
__device__ __forceinline__ void gemv_valu(const u16* __restrict__ X, const u16* __restrict__ W,
                                          void* __restrict__ Y, const float* __restrict__ gamma, int M,
                                          float* __restrict__ ws = nullptr)
{
    constexpr long NO = E ? N / 2 : N;          // columns of Y
    static_assert(PRO == 0 || MMAX == 1, "the fused norm prologue serves M = 1");
    static_assert(PRO == 0 || NW == 4, "the norm prologue's block reduction takes 256 threads");
    static_assert(NW % S == 0 && NW >= 1 && NW <= 16, "S divides the NW waves of a block");
    static_assert(KX == 1 || (MMAX == 1 && S == 1 && PRO == 0 && E == 0),
                  "split across workgroups: M = 1, no in-block split, no fused prologue or epilogue");
    constexpr long CH = K / 8;                  // 16-byte chunks per row
    static_assert(K % 8 == 0 && CH % (S * KX) == 0, "K slice must be whole chunks");
    constexpr long CHS = CH / (S * KX);         // chunks per K-slice
    constexpr long TRIPS = CHS / 64;            // full 64-lane trips per slice
    constexpr int TAIL = (int)(CHS % 64);       // lanes busy in the last, partial trip
    static_assert(U >= 1 && TRIPS % U == 0, "U divides the trip count");
    constexpr int RG = NW / S;
    static_assert(N % (R * RG) == 0, "blocks tile N exactly");
    constexpr int V = R * MMAX;
    constexpr int LV = dev::log2_of<V>::value;
    static_assert(E == 0 || R % 2 == 0, "gate/up pairs: an even row count per wave");
    // weight row of the wave's row r, relative to the wave's first row
    auto rowoff = [](int r) -> long { return (E && r >= R / 2) ? NO - R / 2 + r : r; };

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int s = wave % S;
    const int rg = wave / S;
    const long n0 = ((long)blockIdx.x * RG + rg) * (E ? R / 2 : R);   // first weight row = first output column
    const int xk = KX > 1 ? (int)blockIdx.y : 0;                       // slice of K across workgroups
    const long slice = (long)xk * S + s;

    // this lane's chunks of the slice; W row n, trip t: Wl + w_row(n) + t * W_TRIP
    const u32x4* __restrict__ Wl = reinterpret_cast<const u32x4*>(W) + w_col(slice * CHS + lane);
    const u32x4* __restrict__ Xg = reinterpret_cast<const u32x4*>(X) + slice * CHS + lane;
    __shared__ u32x4 xs[PRO ? CH : 1];         // the normalised X row
    __shared__ float red[PRO ? 256 : 1];
    if constexpr (PRO) {
        const float r = dev::rms_scale_block(X, K, NORM_EPS, red);
        for (long c = threadIdx.x; c < CH; c += 256) {
            const u32x4 xv = reinterpret_cast<const u32x4*>(X)[c];
            const f32x4 g0 = reinterpret_cast<const f32x4*>(gamma)[2 * c];
            const f32x4 g1 = reinterpret_cast<const f32x4*>(gamma)[2 * c + 1];
            auto pair = [&](u32 v, float ga, float gb) -> u32 {
                return (u32)dev::rms_apply((u16)(v & 0xFFFFu), r, ga) | ((u32)dev::rms_apply((u16)(v >> 16), r, gb) << 16);
            };
            xs[c] = u32x4{pair(xv.x, g0.x, g0.y), pair(xv.y, g0.z, g0.w), pair(xv.z, g1.x, g1.y),
                          pair(xv.w, g1.z, g1.w)};
        }
        __syncthreads();
    }
    // X chunk i of this lane's slice (the normalised row in LDS with PRO)
    auto Xp = [&](long i) -> u32x4 {
        if constexpr (PRO) return xs[s * CHS + lane + i];
        else return Xg[i];
    };

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;

    constexpr long NB = TRIPS / U;              // batches of U trips
    static_assert(P == 0 || (MMAX == 1 && NB >= 2), "pipelined batches: M = 1, two batches or more");
    if constexpr (P) {
        u32x4 w[2][U][R], xv[2][U];
        auto ld = [&](int slot, long t0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int r = 0; r < R; ++r) w[slot][u][r] = dev::load16<NT>(Wl + w_row(n0 + rowoff(r)) + (t0 + u) * W_TRIP);
                xv[slot][u] = Xp((t0 + u) * 64);
            }
        };
        auto dot = [&](int slot) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = dev::dot8(w[slot][u][r], xv[slot][u], acc[r]);
        };
        ld(0, 0);
#pragma unroll
        for (long b = 0; b + 1 < NB; b += 2) {
            ld(1, (b + 1) * U);
            dot(0);
            if (b + 2 < NB) ld(0, (b + 2) * U);
            dot(1);
        }
        if constexpr (NB % 2) dot(0);
    }
    for (long t0 = 0; t0 < (P ? 0 : TRIPS); t0 += U) {
        u32x4 w[U][R];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r)
                w[u][r] = dev::load16<NT>(Wl + w_row(n0 + rowoff(r)) + (t0 + u) * W_TRIP);
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int m = 0; m < MMAX; ++m) {
                if (m < M) {
                    const u32x4 x = Xp(m * CH + (t0 + u) * 64);
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        acc[r * MMAX + m] = dev::dot8(w[u][r], x, acc[r * MMAX + m]);
                }
            }
        }
    }
    if constexpr (TAIL > 0) {
        if (lane < TAIL) {
            u32x4 w[R];
#pragma unroll
            for (int r = 0; r < R; ++r) w[r] = dev::load16<NT>(Wl + w_row(n0 + rowoff(r)) + TRIPS * W_TRIP);
#pragma unroll
            for (int m = 0; m < MMAX; ++m) {
                if (m < M) {
                    const u32x4 x = Xp(m * CH + TRIPS * 64);
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        acc[r * MMAX + m] = dev::dot8(w[r], x, acc[r * MMAX + m]);
                }
            }
        }
    }

    const float sum = dev::wave_reduce_scatter<V>(acc, lane);
    const int idx = lane >> (6 - LV);               // value index held by this lane
    const bool writer = (lane & ((64 >> LV) - 1)) == 0;
    const int r = idx / MMAX, m = idx % MMAX;

    if constexpr (KX > 1) {
        // this slice's partials; splitk_reduce adds the KX slices
        if (writer) ws[(long)xk * N + n0 + r] = sum;
    } else if constexpr (S == 1) {
        if constexpr (E) {
            const float up = __shfl_down(sum, 32);      // value idx + (R/2)*MMAX
            if (writer && r < R / 2 && m < M) dev::store1<OUT>(Y, (long)m * NO + n0 + r, dev::swiglu<OUT>(sum, up));
        } else {
            if (writer && m < M) dev::store1<OUT>(Y, (long)m * NO + n0 + r, sum);
        }
    } else {
        __shared__ float red[NW][V];
        if (writer) red[wave][idx] = sum;
        __syncthreads();
        if (s == 0 && writer && m < M && (!E || r < R / 2)) {
            float t = red[wave][idx];
#pragma unroll
            for (int j = 1; j < S; ++j) t += red[wave + j][idx];
            if constexpr (E) {
                float tu = red[wave][idx + (R / 2) * MMAX];
#pragma unroll
                for (int j = 1; j < S; ++j) tu += red[wave + j][idx + (R / 2) * MMAX];
                t = dev::swiglu<OUT>(t, tu);
            }
            dev::store1<OUT>(Y, (long)m * NO + n0 + r, t);
        }
    }
}

// ---------------------------------------------------------------------------
// Skinny GEMM on MFMA for M <= 16 (decode and tiny prefill blocks).
//
// One wave computes 16 rows of W (n) x 16 rows of X (m) with
// v_mfma_f32_16x16x32_bf16: W is the A operand, X the B operand.  Lane
// (r = l & 15, g = l >> 4) loads, for each batch of U MFMA steps, U contiguous
// 16-byte chunks of row r starting at k = batch*32U + g*8U, and MFMA u takes
// chunk u from every lane.  A and B use the same assignment of k to lanes, so
// each MFMA step sums 32 distinct k and the batch covers [batch*32U,
// (batch+1)*32U) exactly once: only the summation order differs from k
// ascending.  Rows of X at or past M are not read (the last real row is
// re-read) and their outputs are not stored.
//
// Block: 256 threads = 4 waves = (4/S) row tiles x S K-slices.
// Grid:  N / (16 * 4/S) blocks.
// ---------------------------------------------------------------------------
template <int S, int U, int NT, int OUT>
__device__ __forceinline__ void gemv_mfma(const u16* __restrict__ X, const u16* __restrict__ W,
                                          void* __restrict__ Y, int M)
{
    static_assert(4 % S == 0, "S divides the 4 waves of a block");
    constexpr int RG = 4 / S;
    static_assert(N % (16 * RG) == 0, "blocks tile N exactly");
    static_assert(K % (32 * U * S) == 0, "K slices are whole batches");
    constexpr long KS = K / S;
    constexpr long BATCHES = KS / (32 * U);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int s = wave % S;
    const int rg = wave / S;
    const long n0 = ((long)blockIdx.x * RG + rg) * 16;
    const int r = lane & 15, g = lane >> 4;
    const int mrow = r < M ? r : M - 1;

    // the lane's U consecutive chunks of batch b: Wl[b * W_BATCH + u] (in the
    // panel layout the U chunks stay inside one 8-chunk block row: U is even
    // and every batch starts at a multiple of 8 chunks)
    static_assert(WPACK == 0 || U % 2 == 0, "panel layout: whole 8-chunk block rows per batch");
    constexpr long W_BATCH = WPACK ? (4 * U / 8) * 1024 : 4 * U;
    const u32x4* __restrict__ Wl = reinterpret_cast<const u32x4*>(W) + w_row(n0 + r) + w_col(s * KS / 8 + g * U);
    const u16* __restrict__ Xrow = X + (long)mrow * K + s * KS + g * 8 * U;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (long b = 0; b < BATCHES; ++b) {
        u32x4 w[U], x[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            w[u] = dev::load16<NT>(Wl + b * W_BATCH + u);
#pragma unroll
        for (int u = 0; u < U; ++u)
            x[u] = *reinterpret_cast<const u32x4*>(Xrow + b * 32 * U + u * 8);
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w[u]),
                                                          __builtin_bit_cast(bf16x8, x[u]),
                                                          acc, 0, 0, 0);
    }

    // acc[i] of lane l is C[n = n0 + 4*(l>>4) + i][m = l & 15].
    const int m = lane & 15;
    const long nbase = n0 + 4 * (lane >> 4);
    if constexpr (S == 1) {
        if (m < M) dev::store4<OUT>(Y, (long)m * N + nbase, acc);
    } else {
        __shared__ f32x4 red[4][64];
        red[wave][lane] = acc;
        __syncthreads();
        if (s == 0 && m < M) {
            f32x4 t = red[wave][lane];
#pragma unroll
            for (int j = 1; j < S; ++j) t += red[wave + j][lane];
            dev::store4<OUT>(Y, (long)m * N + nbase, t);
        }
    }
}

