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

// ---------------------------------------------------------------------------
// Decode GEMV on the vector ALU (M <= MMAX, MMAX small).
//
// One wave walks R rows of W; lane l reads 16-byte chunk l, l+64, l+128, ... of
// each row, so one load instruction covers 1 KiB of a row contiguously.  The
// GPU analogue of the pages' decode module: one subgroup per output row,
// lanes striding over 16-byte (8 x bf16) blocks of the weight row, the row
// length in blocks and the row count as constants ("#002 le meme compilateur
// sur un GPU", section "Emettre pour un GPU").  The S waves of a row group
// split K and combine through LDS in a fixed order.
//
// Block: 256 threads = 4 waves = (4/S) row groups x S K-slices.
// Grid:  N / (R * 4/S) blocks.
// ---------------------------------------------------------------------------
template <int R, int S, int MMAX, int U, int NT, int OUT>
__device__ __forceinline__ void gemv_valu(const u16* __restrict__ X, const u16* __restrict__ W,
                                          void* __restrict__ Y, int M)
{
    static_assert(4 % S == 0, "S divides the 4 waves of a block");
    constexpr long CH = K / 8;                  // 16-byte chunks per row
    static_assert(K % 8 == 0 && CH % S == 0, "K slice must be whole chunks");
    constexpr long CHS = CH / S;                // chunks per K-slice
    constexpr long TRIPS = CHS / 64;            // full 64-lane trips per slice
    constexpr int TAIL = (int)(CHS % 64);       // lanes busy in the last, partial trip
    static_assert(U >= 1 && TRIPS % U == 0, "U divides the trip count");
    constexpr int RG = 4 / S;
    static_assert(N % (R * RG) == 0, "blocks tile N exactly");
    constexpr int V = R * MMAX;
    constexpr int LV = dev::log2_of<V>::value;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int s = wave % S;
    const int rg = wave / S;
    const long n0 = ((long)blockIdx.x * RG + rg) * R;

    const u32x4* __restrict__ Wp = reinterpret_cast<const u32x4*>(W) + n0 * CH + s * CHS + lane;
    const u32x4* __restrict__ Xp = reinterpret_cast<const u32x4*>(X) + s * CHS + lane;

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;

    for (long t0 = 0; t0 < TRIPS; t0 += U) {
        u32x4 w[U][R];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r)
                w[u][r] = dev::load16<NT>(Wp + r * CH + (t0 + u) * 64);
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int m = 0; m < MMAX; ++m) {
                if (m < M) {
                    const u32x4 x = Xp[m * CH + (t0 + u) * 64];
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
            for (int r = 0; r < R; ++r) w[r] = dev::load16<NT>(Wp + r * CH + TRIPS * 64);
#pragma unroll
            for (int m = 0; m < MMAX; ++m) {
                if (m < M) {
                    const u32x4 x = Xp[m * CH + TRIPS * 64];
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

    if constexpr (S == 1) {
        if (writer && m < M) dev::store1<OUT>(Y, (long)m * N + n0 + r, sum);
    } else {
        __shared__ float red[4][V];
        if (writer) red[wave][idx] = sum;
        __syncthreads();
        if (s == 0 && writer && m < M) {
            float t = red[wave][idx];
#pragma unroll
            for (int j = 1; j < S; ++j) t += red[wave + j][idx];
            dev::store1<OUT>(Y, (long)m * N + n0 + r, t);
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

    const u16* __restrict__ Wrow = W + (n0 + r) * K + s * KS + g * 8 * U;
    const u16* __restrict__ Xrow = X + (long)mrow * K + s * KS + g * 8 * U;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (long b = 0; b < BATCHES; ++b) {
        u32x4 w[U], x[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            w[u] = dev::load16<NT>(reinterpret_cast<const u32x4*>(Wrow + b * 32 * U + u * 8));
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

// ---------------------------------------------------------------------------
// Prefill GEMM on MFMA (any M; tiles of BM x BN, K step 64).
//
// Both operands are K-contiguous.  Each k-tile of X (BM x 64) and W (BN x 64)
// is staged through LDS in two buffers: while the waves run MFMAs on buffer t,
// the next tile's global loads are in flight in registers and land in buffer
// t^1 afterwards, with one barrier per k-tile.  LDS rows are 128 bytes (8
// chunks of 16 bytes); chunk c of row r is stored at slot c ^ (r & 7) so that
// the MFMA operand reads of 32 consecutive rows spread over all banks.
//
// WM x WN waves; each wave owns a (BM/WM) x (BN/WN) sub-tile of 32 x 32 MFMA
// blocks (v_mfma_f32_32x32x16_bf16, X as A operand, W as B operand).  Rows of X
// at or past M are clamped to M-1 on load and never stored.
//
// Split-K (SK > 1): block (tile, z) sums k in [z*K/SK, (z+1)*K/SK) and writes
// an f32 partial into ws[z][M][N]; splitk_reduce then adds the SK partials in
// ascending z, so the result does not depend on which block finishes first.
//
// Tile order: the hardware deals consecutive workgroup ids round-robin to the
// 8 XCDs, each with its own L2.  The id is first remapped so that each XCD gets
// a contiguous range, then that range walks the tiles GROUP_M tile-rows at a
// time, so tiles sharing X rows and W rows run together on one L2.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int SK, int GROUP_M, int OUT>
__device__ __forceinline__ void gemm_mfma(const u16* __restrict__ X, const u16* __restrict__ W,
                                          void* __restrict__ Y, float* __restrict__ ws, int M)
{
    constexpr int BK = 64;
    constexpr int NTHR = WM * WN * 64;
    static_assert(K % (SK * BK) == 0, "K splits are whole k-tiles");
    constexpr long KS = K / SK;
    constexpr long KT = KS / BK;                 // k-tiles per split (trip count)
    constexpr int WTM = BM / WM, WTN = BN / WN;  // wave sub-tile
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile is whole 32x32 blocks");
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(N % BN == 0, "tiles cover N exactly");
    constexpr int A_PER_T = BM * 8 / NTHR;
    constexpr int B_PER_T = BN * 8 / NTHR;
    static_assert(BM * 8 % NTHR == 0 && BN * 8 % NTHR == 0, "chunks split evenly over threads");
    constexpr long TILES_N = N / BN;

    __shared__ u32x4 lds[2][(BM + BN) * 8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // ---- tile index: XCD-contiguous remap, then grouped ordering
    const long tiles_m = (M + BM - 1) / BM;
    const long nblk = tiles_m * TILES_N;
    const long pid0 = blockIdx.x;
    const long q = nblk / 8, rem = nblk % 8;
    const long xcd = pid0 % 8, local = pid0 / 8;
    const long pid = (xcd < rem) ? xcd * (q + 1) + local : rem * (q + 1) + (xcd - rem) * q + local;
    const long in_group = (long)GROUP_M * TILES_N;
    const long group = pid / in_group;
    const long first_m = group * GROUP_M;
    const long gsz = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
    const long tm = first_m + (pid % in_group) % gsz;
    const long tn = (pid % in_group) / gsz;
    const long m0 = tm * BM, n0 = tn * BN;
    const int z = blockIdx.y;
    const long kbeg = (long)z * KS;

    // ---- global -> register staging of one k-tile
    u32x4 ra[A_PER_T], rb[B_PER_T];
    const u16* aptr[A_PER_T];
    const u16* bptr[B_PER_T];
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
        const int c = tid + i * NTHR;
        long row = m0 + (c >> 3);
        row = row < M ? row : M - 1;
        aptr[i] = X + row * K + kbeg + (c & 7) * 8;
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
        const int c = tid + i * NTHR;
        bptr[i] = W + (n0 + (c >> 3)) * K + kbeg + (c & 7) * 8;
    }
    auto gload = [&](long kt) {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) ra[i] = *reinterpret_cast<const u32x4*>(aptr[i] + kt * BK);
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bptr[i] + kt * BK);
    };
    auto lstore = [&](int st) {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int c = tid + i * NTHR;
            const int row = c >> 3, col = c & 7;
            lds[st][row * 8 + (col ^ (row & 7))] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const int c = tid + i * NTHR;
            const int row = c >> 3, col = c & 7;
            lds[st][(BM + row) * 8 + (col ^ (row & 7))] = rb[i];
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int lrow = lane & 31;      // operand row within a 32-row block
    const int lhalf = lane >> 5;     // which 8-wide k half of a 16-k step

    gload(0);
    lstore(0);
    __syncthreads();
    for (long kt = 0; kt < KT; ++kt) {
        const int st = (int)(kt & 1);
        if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int chunk = kk * 2 + lhalf;
            bf16x8 a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * WTM + i * 32 + lrow;
                a[i] = __builtin_bit_cast(bf16x8, lds[st][row * 8 + (chunk ^ (row & 7))]);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn * WTN + j * 32 + lrow;
                b[j] = __builtin_bit_cast(bf16x8, lds[st][(BM + row) * 8 + (chunk ^ (row & 7))]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) lstore(st ^ 1);
        __syncthreads();
    }

    // ---- epilogue.  acc[i][j][e] of lane l is C[row][col] of its 32x32 block with
    //      row = 8*(e>>2) + 4*(l>>5) + (e&3), col = l & 31.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const long col = n0 + wn * WTN + j * 32 + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const long row = m0 + wm * WTM + i * 32 + 8 * (e >> 2) + 4 * lhalf + (e & 3);
                if (row < M) {
                    if constexpr (SK == 1) dev::store1<OUT>(Y, row * N + col, acc[i][j][e]);
                    else ws[((long)z * M + row) * N + col] = acc[i][j][e];
                }
            }
        }
    }
}

// Sum of the SK split-K partials in ascending split order, then the epilogue.
template <int SK, int OUT>
__device__ __forceinline__ void splitk_reduce(const float* __restrict__ ws, void* __restrict__ Y, int M)
{
    const long total4 = (long)M * N / 4;
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total4) return;
    const long stride = (long)M * N;
    f32x4 t = reinterpret_cast<const f32x4*>(ws)[i];
#pragma unroll
    for (int z = 1; z < SK; ++z) t += reinterpret_cast<const f32x4*>(ws + z * stride)[i];
    dev::store4<OUT>(Y, i * 4, t);
}

// ---------------------------------------------------------------------------
// Plain kernel for any shape: one thread per output, k ascending, f32 FMA.
// Serves shapes no tiled candidate divides.
// ---------------------------------------------------------------------------
template <int OUT>
__device__ __forceinline__ void gemm_plain(const u16* __restrict__ X, const u16* __restrict__ W,
                                           void* __restrict__ Y, int M)
{
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)M * N) return;
    const long m = idx / N, n = idx % N;
    const u32x4* xp = reinterpret_cast<const u32x4*>(X + m * K);
    const u32x4* wp = reinterpret_cast<const u32x4*>(W + n * K);
    float acc = 0.f;
    for (long c = 0; c < K / 8; ++c) acc = dev::dot8(wp[c], xp[c], acc);
    dev::store1<OUT>(Y, idx, acc);
}

// ===========================================================================
// Support kernels: validation gate, probes, measurement.  Not templated on a
// candidate; one instance per module.
// ===========================================================================

// Reference rows for the validation gate: for each listed row rows[j], the f32
// dot products with every W row, k ascending, one thread per output column n.
// W is read once per launch (all listed rows share the thread's W row).
extern "C" __global__ __launch_bounds__(256) void proj_ref_rows(const u16* __restrict__ X,
                                                                const u16* __restrict__ W,
                                                                const int* __restrict__ rows,
                                                                int nrows, float* __restrict__ ref)
{
    constexpr int MAXR = 8;
    const long n = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    float acc[MAXR];
#pragma unroll
    for (int j = 0; j < MAXR; ++j) acc[j] = 0.f;
    const u32x4* wp = reinterpret_cast<const u32x4*>(W + n * K);
    for (long c = 0; c < K / 8; ++c) {
        const u32x4 w = wp[c];
#pragma unroll
        for (int j = 0; j < MAXR; ++j)
            if (j < nrows) {
                const u32x4 x = reinterpret_cast<const u32x4*>(X + (long)rows[j] * K)[c];
                acc[j] = dev::dot8(w, x, acc[j]);
            }
    }
#pragma unroll
    for (int j = 0; j < MAXR; ++j)
        if (j < nrows) ref[(long)j * N + n] = acc[j];
}

// Counter-based generator for probe inputs (SplitMix-style mixer of seed and
// index).  kind 0: uniform in [-scale, scale) rounded to bf16; kind 1: integers
// uniform in [-4, 4] (exact in bf16).
__device__ __forceinline__ u32 mix32(u64 z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (u32)(z >> 32);
}

extern "C" __global__ __launch_bounds__(256) void proj_fill_probe(u16* __restrict__ out, long n, u32 seed,
                                                                  int kind, float scale)
{
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
        const u32 h = mix32(((u64)seed << 40) ^ (u64)i);
        float v;
        if (kind == 0) v = ((float)(h >> 8) * (1.0f / 8388608.0f) - 1.0f) * scale;
        else v = (float)((int)(h % 9u) - 4);
        out[i] = dev::to_bf16(v);
    }
}

extern "C" __global__ __launch_bounds__(256) void proj_fill_u32(u32* __restrict__ out, long n, u32 value)
{
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
        out[i] = value;
}

// Gate statistics written by proj_check: counters and the max error / max |ref|
// over the listed rows (non-negative floats compare like their bit patterns).
struct CheckStats {
    u32 bad;          // listed-row elements outside the tolerance (or not bit-equal when exact)
    u32 unwritten;    // elements of rows < M still holding the sentinel
    u32 guard;        // elements of rows >= M that no longer hold the sentinel
    u32 max_err;      // f32 bits of max |y - ref| over listed rows
    u32 max_ref;      // f32 bits of max |ref| over listed rows
    u32 pad[3];
};

template <int OUT>
__device__ __forceinline__ float load_out(const void* Y, long i)
{
    if constexpr (OUT == OUT_F32) return reinterpret_cast<const float*>(Y)[i];
    else return __builtin_bit_cast(float, (u32)reinterpret_cast<const u16*>(Y)[i] << 16);
}

template <int OUT>
__device__ __forceinline__ bool is_sentinel(const void* Y, long i)
{
    if constexpr (OUT == OUT_F32) return reinterpret_cast<const u32*>(Y)[i] == SENTINEL_F32;
    else return reinterpret_cast<const u16*>(Y)[i] == SENTINEL_BF16;
}

// Scans rows [0, rows_alloc) of Y: sentinel bookkeeping on every element, and
// the comparison with ref on the listed rows.  Tolerance (exact == 0):
//   f32 out:  |y - r| <= 1e-3 (|r| + 1)
//   bf16 out: |y - R| <= ulp(R) with R = bf16(r), or the f32 rule.
// exact == 1: y must equal the reference rounded to the output type, bit for bit.
template <int OUT>
__device__ __forceinline__ void check_body(const void* __restrict__ Y, long rows_alloc, int M,
                                           const float* __restrict__ ref, const int* __restrict__ rows,
                                           int nrows, int exact, CheckStats* __restrict__ st)
{
    const long total = rows_alloc * N;
    u32 bad = 0, unw = 0, grd = 0;
    float merr = 0.f, mref = 0.f;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
        const long row = i / N, col = i % N;
        const bool sent = is_sentinel<OUT>(Y, i);
        if (row < M) unw += sent ? 1u : 0u;
        else grd += sent ? 0u : 1u;
        if (row >= M) continue;
        for (int j = 0; j < nrows; ++j) {
            if (rows[j] != row) continue;
            const float r = ref[(long)j * N + col];
            const float y = load_out<OUT>(Y, i);
            const float err = __builtin_fabsf(y - r);
            bool ok;
            if (exact) {
                if constexpr (OUT == OUT_F32) ok = __builtin_bit_cast(u32, y) == __builtin_bit_cast(u32, r);
                else ok = reinterpret_cast<const u16*>(Y)[i] == dev::to_bf16(r);
            } else {
                ok = err <= 1e-3f * (__builtin_fabsf(r) + 1.f);
                if constexpr (OUT == OUT_BF16) {
                    const float R = __builtin_bit_cast(float, (u32)dev::to_bf16(r) << 16);
                    const float aR = __builtin_fabsf(R);
                    int e = aR > 0.f ? (int)((__builtin_bit_cast(u32, aR) >> 23) & 0xFF) - 127 : -126;
                    e = e < -126 ? -126 : e;
                    const float ulp = __builtin_ldexpf(1.f, e - 7);
                    ok = ok || (__builtin_fabsf(y - R) <= ulp);
                }
            }
            bad += ok ? 0u : 1u;
            merr = (err > merr || err != err) ? (err != err ? __builtin_inff() : err) : merr;
            mref = __builtin_fabsf(r) > mref ? __builtin_fabsf(r) : mref;
        }
    }
    if (bad) atomicAdd(&st->bad, bad);
    if (unw) atomicAdd(&st->unwritten, unw);
    if (grd) atomicAdd(&st->guard, grd);
    atomicMax(&st->max_err, __builtin_bit_cast(u32, merr));
    atomicMax(&st->max_ref, __builtin_bit_cast(u32, mref));
}

extern "C" __global__ __launch_bounds__(256) void proj_check_f32(const void* Y, long rows_alloc, int M,
                                                                 const float* ref, const int* rows,
                                                                 int nrows, int exact, CheckStats* st)
{
    check_body<OUT_F32>(Y, rows_alloc, M, ref, rows, nrows, exact, st);
}

extern "C" __global__ __launch_bounds__(256) void proj_check_bf16(const void* Y, long rows_alloc, int M,
                                                                  const float* ref, const int* rows,
                                                                  int nrows, int exact, CheckStats* st)
{
    check_body<OUT_BF16>(Y, rows_alloc, M, ref, rows, nrows, exact, st);
}
