// gemm.hip -- prefill kernels (part of the shape module; see kernels_head.hip).

// ---------------------------------------------------------------------------
// Prefill GEMM on MFMA (any M; block tile BM x BN, k-tile BK).
//
// Both operands are K-contiguous ("TN").  Each k-tile of X (BM x BK) and W
// (BN x BK) goes straight from global memory into LDS with MUBUF
// buffer_load_dwordx4 ... lds (DMA = 1; no trip through VGPRs): the wave's 64
// lanes fill 64 consecutive 16-byte LDS slots, and each lane fetches from
// global memory the chunk that belongs in its slot.  With DMA = 0 the same
// chunks go through registers (loaded before the tile's MFMAs, written to LDS
// after them).  LDS rows are BK*2 bytes (CPR 16-byte chunks); chunk c of row r
// lives in slot c ^ ((r >> SWZ) & (CPR-1)) of the row, so that the 16 rows one
// operand read serves at a time hit distinct banks.
//
// STAGES buffers form a ring: while the waves run MFMAs on tile kt, the copies
// of tiles kt+1 .. kt+STAGES-1 are in flight.  Before the last 16-wide k step
// of tile kt, each wave waits only for its own copies of tile kt+1 (s_waitcnt
// vmcnt with the count of younger copies), then a barrier makes every wave's
// part visible and also tells that every wave has read all of tile kt (the
// last step's operands are in registers), so the copy of tile kt+STAGES goes
// into tile kt's buffer at once.  Each buffer is its own __shared__ array so
// the compiler can see which copy writes which buffer.
//
// WM x WN waves; each wave owns a (BM/WM) x (BN/WN) sub-tile of 32 x 32 MFMA
// blocks (v_mfma_f32_32x32x16_bf16, X as the A operand, W as the B operand),
// and double-buffers its operand fragments in registers across the 16-wide k
// steps of a tile.  Rows of X at or past M are clamped to M-1 on load and never
// stored.
//
// Work split, one of:
//  * SK > 1 (split-K): block (tile, z) sums k in [z*K/SK, (z+1)*K/SK) and
//    writes an f32 partial into ws[z][M][N]; splitk_reduce adds the SK partials
//    in ascending z.
//  * TAILS > 1 (data-parallel with a split tail): of the T tiles, the largest
//    multiple of ROUND (the workgroups the device runs at once) that leaves a
//    remainder runs as whole tiles; each of the rem remaining tiles is split
//    TAILS ways along K (piece z: k-tiles [z*KT/TAILS, (z+1)*KT/TAILS), so the
//    pieces differ by at most one k-tile), and the last round is filled with
//    rem*TAILS shorter pieces instead of rem long ones.  Pieces write f32 partials into
//    ws[piece][BM*BN]; tail_reduce adds them in ascending split order.
// Both reductions use a fixed order, so results do not depend on which block
// finishes first.
//
// K order (KP > 1): the k-tiles of each aligned block of KP are visited in an
// order rotated by the tile's phase (tile-row + tile-column) mod KP, so tiles
// that share a panel of W (same tile-column) or of X (same tile-row) and run
// together under one L2 ask for different k-tiles first: each k-tile of a
// block is fetched from beyond the L2 by one of them and found in the L2 by
// the others a step or more later, instead of every tile waiting on the same
// misses at once.  The order is fixed per tile, so results do not depend on
// timing; a trailing KT % KP k-tiles keep their order.
//
// Tile order: the hardware deals consecutive workgroup ids round-robin to the
// 8 XCDs, each with its own L2.  Whole-tile ids are first remapped so that
// each XCD gets a contiguous range, then tile ids walk the tile grid GROUP_M
// tile-rows at a time, so tiles sharing X rows and W rows run together under
// one L2.
// ---------------------------------------------------------------------------
namespace gemm_detail {

// s_waitcnt until at most N vector-memory operations of this wave are
// outstanding and none of its LDS operations (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt 6:4 left at its maximum, lgkmcnt 11:8 = 0).
template <int N>
__device__ __forceinline__ void wait_vm_lds()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that orders the surrounding LDS accesses in the compiler
// without draining the outstanding global->LDS copies (their waits are
// explicit, above).  Nothing is scheduled across it.
__device__ __forceinline__ void barrier_lds()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

typedef __attribute__((address_space(3))) void lds_void;

template <long V> struct ic { static constexpr long value = V; };

constexpr int gcd(int a, int b) { return b == 0 ? a : gcd(b, a % b); }

// f(ic<I>{}, kt0 + I) for I = FROM .. TO-1, unrolled at compile time.
template <long FROM, long TO, typename F>
__device__ __forceinline__ void unroll_steps(F&& f, long kt0)
{
    if constexpr (FROM < TO) {
        f(ic<FROM>{}, kt0 + FROM);
        unroll_steps<FROM + 1, TO>(f, kt0);
    }
}

// Whole tiles and split tail tiles of a launch: T tiles, ROUND workgroups at
// once.  With T >= ROUND the tail is T % ROUND tiles; below one round every
// tile is a tail tile.  (The host computes the same split for the launch.)
__device__ __forceinline__ void tail_split(long T, long round, long* n_full, long* rem)
{
    *rem = T >= round ? T % round : T;
    *n_full = T - *rem;
}

// Tile id -> (tile-row, tile-column): GROUP_M tile-rows at a time.
template <int GROUP_M>
__device__ __forceinline__ void group_order(long pid, long tiles_m, long tiles_n, long* tm, long* tn)
{
    const long in_group = (long)GROUP_M * tiles_n;
    const long group = pid / in_group;
    const long first_m = group * GROUP_M;
    const long gsz = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
    *tm = first_m + (pid % in_group) % gsz;
    *tn = (pid % in_group) / gsz;
}

// Workgroup id -> tile id such that each XCD (ids dealt round-robin over 8)
// gets a contiguous range of tile ids.  A bijection on [0, nblk).
__device__ __forceinline__ long xcd_remap(long pid0, long nblk)
{
    const long q = nblk / 8, rem = nblk % 8;
    const long xcd = pid0 % 8, local = pid0 / 8;
    return (xcd < rem) ? xcd * (q + 1) + local : rem * (q + 1) + (xcd - rem) * q + local;
}

// The k-tile read at step t (0 <= t < nkt) of a tile whose k order has phase
// ph: inside the whole blocks of KP k-tiles (t < kpb = nkt - nkt % KP) the
// block's k-tiles rotated by ph, so each block is permuted onto itself; the
// trailing k-tiles, and every k-tile with KP <= 1, in order.
template <int KP>
__device__ __forceinline__ long ktile_order(long t, long kpb, long ph)
{
    if constexpr (KP > 1) {
        if (t < kpb) t = (t & ~(long)(KP - 1)) | ((t + ph) & (KP - 1));
    }
    return t;
}

}  // namespace gemm_detail

template <int BM, int BN, int BK, int STAGES, int WM, int WN, int SK, int GROUP_M, int SWZ, int OUT, int DMA = 1,
          int TAILS = 1, int ROUND = 0, int E = 0, int BST = 0, int KP = 0>
__device__ __forceinline__ void gemm_mfma(const u16* __restrict__ X, const u16* __restrict__ W,
                                          void* __restrict__ Y, float* __restrict__ ws, int M)
{
    constexpr long NO = E ? N / 2 : N;                // columns of Y
    using namespace gemm_detail;
    constexpr int NTHR = WM * WN * 64;
    constexpr int CPR = BK / 8;                       // 16-byte chunks per LDS row
    static_assert(BK == 32 || BK == 64, "k-tile of 32 or 64");
    static_assert(STAGES >= 2 && STAGES <= 4, "2..4 buffers");
    static_assert(K % (SK * BK) == 0, "K splits are whole k-tiles");
    static_assert(TAILS == 1 || (SK == 1 && ROUND > 0 && K % BK == 0 && K / BK >= TAILS), "tail pieces are whole k-tiles");
    static_assert(KP == 0 || KP == 2 || KP == 4 || KP == 8, "k-tile blocks of a power of two");
    constexpr long KS = K / SK;
    constexpr long KT = KS / BK;                      // k-tiles of a whole (split-K) tile
    // tail piece z takes k-tiles [z*KT/TAILS, (z+1)*KT/TAILS): KT_TAIL of them, or
    // one more when TAILS does not divide KT
    constexpr long KT_TAIL = KT / TAILS;
    constexpr int WTM = BM / WM, WTN = BN / WN;       // wave sub-tile
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile is whole 32x32 blocks");
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(N % BN == 0, "tiles cover N exactly");
    static_assert(E == 0 || (SK == 1 && TAILS == 1 && (BN / WN) % 64 == 0),
                  "fused SwiGLU: whole tiles, gate and up halves of every wave's columns");
    constexpr int CA = BM * CPR, CB = BN * CPR;       // chunks per buffer
    static_assert(CA % NTHR == 0 && CB % NTHR == 0, "copies split evenly over threads");
    constexpr int IA = CA / NTHR, IB = CB / NTHR;     // copy instructions per thread per tile
    constexpr int PER_TILE = IA + IB;
    // EARLY: the copy of tile kt+STAGES is issued right after the barrier inside
    // step kt; otherwise that of tile kt+STAGES-1 at the start of step kt.
    constexpr bool EARLY = DMA && STAGES == 2;
    constexpr int LEAD = EARLY ? STAGES : STAGES - 1;   // tiles in flight after the prologue
    // BST > STAGES: X (A) keeps STAGES buffers and W (B) gets BST of its own, so
    // each W copy is issued BST - STAGES k-tiles further ahead of its use than
    // X's (the copies of W are the ones that miss the L2: at a few hundred rows
    // W streams from HBM and only the copies in flight hide its latency).
    // BST == 0: X and W of a k-tile share one buffer.
    constexpr bool SPLIT = BST != 0;
    static_assert(BST == 0 || (DMA && BST > STAGES && BST <= 7), "W buffers beyond X's on the global->LDS ring");
    constexpr int NB = SPLIT ? BST : STAGES;          // W buffers
    constexpr int LEAD_B = SPLIT ? LEAD + BST - STAGES : LEAD;   // k-tiles of W in flight after the prologue
    constexpr int PERIOD = SPLIT ? STAGES * BST / gcd(STAGES, BST) : STAGES;  // ring positions before the buffer pattern repeats
    // copies younger than the ones waited for: at the prologue (after tile 0),
    // and in each step (after tile kt+1: with SPLIT, W of tile kt+2 goes out
    // right after X of tile kt+1)
    constexpr int WAIT0 = (LEAD - 1) * IA + (LEAD_B - 1) * IB;
    constexpr int WAITK = (SPLIT ? IB : 0) + (DMA && !EARLY ? (STAGES - 2) * PER_TILE : 0);
    static_assert(WAIT0 <= 63 && WAITK <= 63, "younger copies fit the vmcnt counter");
    constexpr int STAGE = CA + CB;                    // 16-byte slots per buffer
    constexpr long TILES_N = N / BN;
    constexpr int KK = BK / 16;                       // MFMA k-steps per tile

    // X and W of ring position s: one array per buffer holding both (X first),
    // or with SPLIT STAGES arrays of X and BST of W (each buffer its own array in
    // either case; 5 x 32 KiB for 256x256x64 with two X and three W buffers,
    // 3 x 16 + 6 x 16 KiB for 128x128x64 with three X and six W buffers)
    constexpr int SZ = SPLIT ? CA : STAGE;
    __shared__ u32x4 lds0[SZ];
    __shared__ u32x4 lds1[SZ];
    __shared__ u32x4 lds2[STAGES > 2 ? SZ : 1];
    __shared__ u32x4 lds3[STAGES > 3 ? SZ : 1];
    __shared__ u32x4 ldsb0[SPLIT ? CB : 1];
    __shared__ u32x4 ldsb1[SPLIT ? CB : 1];
    __shared__ u32x4 ldsb2[SPLIT ? CB : 1];
    __shared__ u32x4 ldsb3[SPLIT && BST > 3 ? CB : 1];
    __shared__ u32x4 ldsb4[SPLIT && BST > 4 ? CB : 1];
    __shared__ u32x4 ldsb5[SPLIT && BST > 5 ? CB : 1];
    __shared__ u32x4 ldsb6[SPLIT && BST > 6 ? CB : 1];
    auto buf = [&](int s) -> u32x4* { return s == 0 ? lds0 : s == 1 ? lds1 : s == 2 ? lds2 : lds3; };
    auto bufA = [&](int s) -> u32x4* { return buf(s % STAGES); };
    auto bufB = [&](int s) -> u32x4* {
        if constexpr (SPLIT) {
            const int t = s % NB;
            return t == 0 ? ldsb0 : t == 1 ? ldsb1 : t == 2 ? ldsb2 : t == 3 ? ldsb3 : t == 4 ? ldsb4 : t == 5 ? ldsb5 : ldsb6;
        } else {
            return buf(s % STAGES) + CA;
        }
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // ---- which tile (and which K range) this workgroup computes
    const long tiles_m = (M + BM - 1) / BM;
    const long T = tiles_m * TILES_N;
    long n_full = T, rem_t = 0;
    if constexpr (TAILS > 1) tail_split(T, ROUND, &n_full, &rem_t);
    const bool tail = TAILS > 1 && (long)blockIdx.x >= n_full;
    long pid, piece = 0;
    int z;
    long kbeg;
    if (tail) {
        piece = (long)blockIdx.x - n_full;
        pid = n_full + piece / TAILS;
        z = (int)(piece % TAILS);
        kbeg = ((long)z * KT / TAILS) * BK;
    } else {
        pid = xcd_remap(blockIdx.x, n_full);
        z = blockIdx.y;
        kbeg = (long)z * KS;
    }
    long tm, tn;
    group_order<GROUP_M>(pid, tiles_m, TILES_N, &tm, &tn);
    const long m0 = tm * BM;
    // the tile's phase in its blocks of KP k-tiles (uniform across the workgroup)
    const long kph = KP > 1 ? ((tm + tn) & (KP - 1)) : 0;
    // first weight row of the tile (with the SwiGLU epilogue: its first gate row,
    // which is also its first output column; the tile reads BN/2 gate rows and
    // the BN/2 up rows NO below them)
    const long n0 = tn * (E ? BN / 2 : BN);

    // ---- global sources of the copy slots.  Copy instruction i of thread t fills
    //      slot i*NTHR + t, i.e. row i*RPI + t/CPR of the buffer; the chunk's column
    //      (t%CPR) ^ swizzle(row) does not depend on i because RPI >> SWZ is a
    //      multiple of CPR.  Offsets are 32-bit and relative to the tile's first
    //      row (at most BN*K*2 bytes), on a block-uniform 64-bit base.
    constexpr int RPI = NTHR / CPR;                   // buffer rows per copy instruction
    static_assert(NTHR % CPR == 0 && (RPI >> SWZ) % CPR == 0, "swizzle column is copy-invariant");
    const int r0 = tid / CPR;
    const int ccol = (tid % CPR) ^ ((r0 >> SWZ) & (CPR - 1));
    const u16* __restrict__ abase = X + m0 * K + kbeg;
    // B source: row-major, from the tile's first row at column kbeg; in the
    // panel layout, from the start of the panel holding that row (pb), with the
    // k position in the scalar offset (koffb)
    const long pb = WPACK ? n0 - (n0 & (dev::kPanelRows - 1)) : n0;
    const u16* __restrict__ bbase = WPACK ? W + pb * K : W + n0 * K + kbeg;
    const long mlast = (long)M - 1 - m0;              // last valid row relative to m0
    unsigned aoff[IA];
#pragma unroll
    for (int i = 0; i < IA; ++i) {
        long r = i * RPI + r0;
        r = r < mlast ? r : mlast;
        aoff[i] = (unsigned)(r * K + ccol * 8);
    }
    // weight row (relative to the tile's first) held in B-tile row rr: with the
    // SwiGLU epilogue each wave's WTN columns are WTN/2 gate rows followed by
    // the matching up rows, so both halves of a pair land in the same lane
    auto wrow = [&](int rr) -> long {
        if constexpr (E) {
            const int wv = rr / WTN, c = rr % WTN;
            return c < WTN / 2 ? (long)wv * (WTN / 2) + c : NO + (long)wv * (WTN / 2) + c - WTN / 2;
        } else {
            return rr;
        }
    };
    // The copies are MUBUF loads into LDS (buffer_load_dwordx4 ... lds) over a
    // raw buffer descriptor per operand (gfx9 layout: base, stride 0, size in
    // bytes, word 3 = 0x00020000) that starts at the tile's first row and
    // covers exactly the bytes the tile reads.  Each lane's byte offset is
    // fixed; the k-tile advances in the scalar offset.  (The global_ form of
    // the same copy is a FLAT instruction, and while one is outstanding the
    // compiler can only wait for all LDS reads at once.)
    constexpr long B_ROWS = E ? NO + BN / 2 : BN;   // weight rows spanned by the B descriptor
    static_assert((long)(BM > B_ROWS ? BM : B_ROWS) * K * 2 < (1L << 31), "tile rows fit a 32-bit buffer size");
    static_assert(!WPACK || (B_ROWS / dev::kPanelRows + 2) * dev::kPanelRows * K * 2 < (1L << 31),
                  "the panels a tile touches fit a 32-bit buffer size");
    const long rows_a = (long)M - m0 < BM ? (long)M - m0 : BM;
    // bytes of W the descriptor covers: the tile's rows from column kbeg on, or
    // the whole panels that hold the tile's rows
    const long bspan = WPACK ? ((n0 + B_ROWS - 1) / dev::kPanelRows - pb / dev::kPanelRows + 1) *
                                   dev::kPanelRows * K * 2
                             : (B_ROWS * K - kbeg) * 2;
    const __amdgpu_buffer_rsrc_t rsa =
        __builtin_amdgcn_make_buffer_rsrc((void*)abase, 0, (int)((rows_a * K - kbeg) * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void*)bbase, 0, (int)bspan, 0x00020000);
    unsigned abyte[IA], bbyte[IB];
#pragma unroll
    for (int i = 0; i < IA; ++i) abyte[i] = aoff[i] * 2;
    // (in the panel layout a k-tile's chunks of one row are contiguous: BK is at
    //  most one 64-value block and k-tiles start at multiples of BK)
    static_assert(!WPACK || dev::kPanelCols % BK == 0, "k-tiles inside one panel block");
#pragma unroll
    for (int i = 0; i < IB; ++i)
        bbyte[i] = WPACK ? (unsigned)((w_row(n0 + wrow(i * RPI + r0)) - w_row(pb) + ccol) * 16)
                         : (unsigned)((wrow(i * RPI + r0) * K + ccol * 8) * 2);
    // byte offset of k-tile kt of this tile's K range in the B source
    auto koffb = [&](long kt) -> unsigned {
        if constexpr (WPACK) return (unsigned)(w_col((kbeg + kt * BK) / 8) * 16);
        else return (unsigned)(kt * BK * 2);
    };
    auto issueA = [&](u32x4* dst, long kt) {
        const unsigned koff = (unsigned)(kt * BK * 2);
#pragma unroll
        for (int i = 0; i < IA; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(dst + i * NTHR + wave * 64), 16, abyte[i],
                                                     koff, 0, 0);
    };
    auto issueB = [&](u32x4* dst, long kt) {
        const unsigned kob = koffb(kt);
#pragma unroll
        for (int i = 0; i < IB; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(dst + i * NTHR + wave * 64), 16, bbyte[i],
                                                     kob, 0, 0);
    };
    u32x4 ra[DMA ? 1 : IA], rb[DMA ? 1 : IB];
    auto gload = [&](long kt) {
        const u16* a = abase + kt * BK;
        const char* b = reinterpret_cast<const char*>(bbase) + koffb(kt);
#pragma unroll
        for (int i = 0; i < IA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a + aoff[i]);
#pragma unroll
        for (int i = 0; i < IB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(b + bbyte[i]);
    };
    auto lstore = [&](u32x4* dA, u32x4* dB) {
#pragma unroll
        for (int i = 0; i < IA; ++i) dA[i * NTHR + tid] = ra[i];
#pragma unroll
        for (int i = 0; i < IB; ++i) dB[i * NTHR + tid] = rb[i];
    };
    static_assert(DMA || STAGES == 2, "register-staged copies use two buffers");

    // ---- operand fragment addressing (slot of lane's row/chunk within a buffer)
    const int lrow = lane & 31;
    const int lhalf = lane >> 5;
    // The swizzle of a row does not change in 32-row steps, so each lane's
    // chunk for k step kk is (2*kk) ^ q with a per-lane q, and the 32-row steps
    // of a fragment are constant offsets (immediates of the LDS read).
    static_assert((32 >> SWZ) % CPR == 0, "32-row steps keep the swizzle");
    const int rowa0 = wm * WTM + lrow, rowb0 = wn * WTN + lrow;
    const int qa = lhalf ^ ((rowa0 >> SWZ) & (CPR - 1));
    const int qb = lhalf ^ ((rowb0 >> SWZ) & (CPR - 1));
    auto frag_a = [&](const u32x4* b, int i, int kk) -> bf16x8 {
        const u32x4* p = b + rowa0 * CPR + ((kk * 2) ^ qa);
        return __builtin_bit_cast(bf16x8, p[i * 32 * CPR]);
    };
    auto frag_b = [&](const u32x4* b, int j, int kk) -> bf16x8 {
        const u32x4* p = b + rowb0 * CPR + ((kk * 2) ^ qb);
        return __builtin_bit_cast(bf16x8, p[j * 32 * CPR]);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // ---- the k loop over NKT k-tiles (a compile-time count: KT for a whole
    //      tile, KT_TAIL or KT_TAIL + 1 for a tail piece).  Tile t lives in buffer
    //      t % STAGES.
    //      The barrier that publishes tile kt+1 (and frees tile kt's buffer)
    //      sits before the last 16-wide k step of tile kt: after it, each wave
    //      reads the first operand fragments of tile kt+1 while the MFMAs of
    //      that last k step, whose operands are already in registers, keep the
    //      matrix pipe busy.  Neither the barrier nor the first operand reads of
    //      a tile then find the pipe empty.  Operand fragments alternate between
    //      two register slots: k step kk of a tile uses slot kk & 1.
    bf16x8 fa[2][TM], fb[2][TN];
    // W fragments first: the first MFMAs of a step then wait only for the reads
    // of their own operands, not for the whole set.
    auto read_frags = [&](const u32x4* bA, const u32x4* bB, int kk, int slot) {
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[slot][j] = frag_b(bB, j, kk);
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[slot][i] = frag_a(bA, i, kk);
    };
    auto mfmas = [&](int slot) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
    };
    // Instruction order for the scheduler, per k step: the next step's operand
    // reads first, then this step's MFMAs, so the reads have a whole step of
    // MFMAs to land.  (While copies into LDS are in flight the compiler can
    // only wait for all outstanding LDS reads at once, so reads slotted late
    // between the MFMAs would stall the next step's first MFMA.)
    auto interleave = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
    };

    auto kloop = [&](auto nkt) {
        constexpr long NKT = decltype(nkt)::value;
        auto clamp = [&](long t) -> long { return t < NKT ? t : NKT - 1; };
        // the k-tile the copy for step t reads: t past the end re-reads the
        // last one; inside the whole blocks of KP, the tile's rotated order (a
        // permutation of each block, so every index stays below NKT)
        constexpr long KPB = KP > 1 ? NKT - NKT % KP : 0;
        auto src = [&](long t) -> long { return ktile_order<KP>(clamp(t), KPB, kph); };
        // prologue: X of tiles 0 .. LEAD-1 and W of tiles 0 .. LEAD_B-1 in flight,
        // in tile order (DMA), or tile 0 through registers; then tile 0
        // published and its first fragments read.
        if constexpr (DMA) {
#pragma unroll
            for (int s = 0; s < LEAD_B; ++s) {
                if (s < LEAD) issueA(bufA(s), src(s));
                issueB(bufB(s), src(s));
            }
        } else {
            gload(src(0));
            lstore(bufA(0), bufB(0));
        }
        wait_vm_lds<DMA ? WAIT0 : 0>();
        barrier_lds();
        read_frags(bufA(0), bufB(0), 0, 0);
        // One k-tile kt at ring position R: the MFMAs of all but the last k step,
        // then wait for this wave's copies of tile kt+1, barrier -- every wave
        // has now read all of tile kt and written its part of tile kt+1 -- then
        // the last k step's MFMAs beside the reads of tile kt+1's first
        // fragments.  The copies of the next tiles to fetch go out right after
        // that barrier into tile kt's buffers (EARLY: X of tile kt+2, W of tile
        // kt+LEAD_B, so a copy gets at least a whole step between issue and wait)
        // or at the start of the step into tile kt-1's buffer (three or more
        // buffers: already STAGES-1.75 steps ahead).  Past the last tile a copy
        // re-reads tile NKT-1 into the free buffer, so every step issues the same
        // number of copies and the vmcnt bound stays exact without branches
        // (branches here hide from the compiler which buffer a copy writes, and
        // it then drains every copy before each LDS read).  With DMA == 0, tile
        // kt+1 is loaded into registers before the MFMAs and written to its
        // buffers after them.
        auto step = [&](auto r, long kt) {
            constexpr int R = decltype(r)::value;
            u32x4* bA = bufA(R);
            u32x4* bB = bufB(R);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!DMA) {
                gload(src(kt + 1));
            } else if constexpr (!EARLY) {
                issueA(bufA(R + STAGES - 1), src(kt + LEAD));
                issueB(bufB(R + NB - 1), src(kt + LEAD_B));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk + 1 < KK; ++kk) {
                read_frags(bA, bB, kk + 1, (kk + 1) & 1);
                mfmas(kk & 1);
            }
#pragma unroll
            for (int kk = 0; kk + 1 < KK; ++kk) interleave();
            if constexpr (!DMA) {
                __builtin_amdgcn_sched_barrier(0);
                lstore(bufA(R + 1), bufB(R + 1));
            }
            __builtin_amdgcn_sched_barrier(0);
            wait_vm_lds<WAITK>();
            barrier_lds();
            read_frags(bufA(R + 1), bufB(R + 1), 0, 0);
            if constexpr (EARLY) {
                issueA(bA, src(kt + LEAD));
                issueB(bB, src(kt + LEAD_B));
            }
            mfmas((KK - 1) & 1);
            // the reads first, then the MFMAs with any copies slotted between them
            __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
            if constexpr (EARLY) {
                constexpr int NMF = TM * TN;
                constexpr int PAIRS = NMF < PER_TILE ? NMF : PER_TILE;
#pragma unroll
                for (int q = 0; q < PAIRS; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
                if constexpr (NMF > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, NMF - PAIRS, 0);
                if constexpr (PER_TILE > PAIRS) __builtin_amdgcn_sched_group_barrier(0x020, PER_TILE - PAIRS, 0);
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
            }
        };
        // PERIOD positions per pass (tile t at position t % PERIOD), then the rest
        constexpr long KMAIN = NKT - NKT % PERIOD;
        for (long kt = 0; kt < KMAIN; kt += PERIOD) unroll_steps<0, PERIOD>(step, kt);
        unroll_steps<0, NKT % PERIOD>(step, KMAIN);
        wait_vm_lds<0>();   // no copy may still write LDS when the block ends
    };

    // ---- epilogue.  acc[i][j][e] of lane l is C[row][col] of its 32x32 block with
    //      row = 8*(e>>2) + 4*(l>>5) + (e&3), col = l & 31.  A tile whose rows all
    //      lie below M (every tile but those of the last tile-row of a ragged M)
    //      stores without per-element row checks, element e at the compile-time
    //      distance 8*(e>>2) + (e&3) rows from the lane's first row of the block
    //      (one 64-bit add of a constant per element, no branch); other tiles
    //      check each element's row against M.
    const bool full = m0 + BM <= (long)M;             // uniform across the workgroup
    // body(e, r0, dr): element e of block row i, whose row is r0 + dr (r0 counted
    // from row 0 of the destination, dr a constant once unrolled)
    auto rows = [&](int i, auto&& body) {
        const long r0 = m0 + wm * WTM + i * 32 + 4 * lhalf;
        if (full) {
#pragma unroll
            for (int e = 0; e < 16; ++e) body(e, r0, 8 * (e >> 2) + (e & 3));
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (r0 + 8 * (e >> 2) + (e & 3) < M) body(e, r0, 8 * (e >> 2) + (e & 3));
        }
    };
    if constexpr (TAILS > 1) {
        if (tail) {
            if constexpr (KT % TAILS == 0) {
                kloop(ic<KT_TAIL>{});
            } else {
                // uniform across the workgroup; each count its own unrolled loop
                if (((long)(z + 1) * KT / TAILS) - ((long)z * KT / TAILS) == KT_TAIL) kloop(ic<KT_TAIL>{});
                else kloop(ic<KT_TAIL + 1>{});
            }
            float* part = ws + piece * ((long)BM * BN);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = wn * WTN + j * 32 + (lane & 31);
                    rows(i, [&](int e, long r0, int dr) {
                        float* p = part + (r0 - m0) * BN + col;
                        p[(long)dr * BN] = acc[i][j][e];
                    });
                }
            return;
        }
    }
    kloop(ic<KT>{});
    if constexpr (E) {
        // block j < TN/2 holds gate rows, block j + TN/2 the matching up rows
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN / 2; ++j) {
                const long col = n0 + wn * (WTN / 2) + j * 32 + (lane & 31);
                rows(i, [&](int e, long r0, int dr) {
                    const long b = r0 * NO + col;
                    dev::store1<OUT>(Y, b + (long)dr * NO, dev::swiglu<OUT>(acc[i][j][e], acc[i][j + TN / 2][e]));
                });
            }
        return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const long col = n0 + wn * WTN + j * 32 + (lane & 31);
            rows(i, [&](int e, long r0, int dr) {
                if constexpr (SK == 1) {
                    const long b = r0 * N + col;
                    dev::store1<OUT>(Y, b + (long)dr * N, acc[i][j][e]);
                } else {
                    const long b = ((long)z * M + r0) * N + col;
                    ws[b + (long)dr * N] = acc[i][j][e];
                }
            });
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

// Sum of the TAILS partials of each tail tile (ascending split order), then the
// epilogue.  One thread per 4 consecutive outputs of a tail tile; the tile ids
// and their positions follow gemm_mfma's split and order exactly.
template <int BM, int BN, int TAILS, int ROUND, int GROUP_M, int OUT>
__device__ __forceinline__ void tail_reduce(const float* __restrict__ ws, void* __restrict__ Y, int M)
{
    using namespace gemm_detail;
    constexpr long TILES_N = N / BN;
    constexpr long PER_TILE4 = (long)BM * BN / 4;
    const long tiles_m = (M + BM - 1) / BM;
    long n_full, rem_t;
    tail_split(tiles_m * TILES_N, ROUND, &n_full, &rem_t);
    const long g = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= rem_t * PER_TILE4) return;
    const long t = g / PER_TILE4, e4 = g % PER_TILE4;
    long tm, tn;
    group_order<GROUP_M>(n_full + t, tiles_m, TILES_N, &tm, &tn);
    const long row = tm * BM + (e4 * 4) / BN, col = tn * BN + (e4 * 4) % BN;
    if (row >= M) return;
    const f32x4* p = reinterpret_cast<const f32x4*>(ws + t * TAILS * ((long)BM * BN)) + e4;
    f32x4 s = p[0];
#pragma unroll
    for (int z = 1; z < TAILS; ++z) s += p[z * PER_TILE4];
    dev::store4<OUT>(Y, row * N + col, s);
}

// ---------------------------------------------------------------------------
// Plain kernel for any shape: one thread per output, k ascending, f32 FMA.
// Serves shapes no tiled candidate divides.
// ---------------------------------------------------------------------------
template <int OUT, int E = 0>
__device__ __forceinline__ void gemm_plain(const u16* __restrict__ X, const u16* __restrict__ W,
                                           void* __restrict__ Y, int M)
{
    constexpr long NO = E ? N / 2 : N;                // columns of Y
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)M * NO) return;
    const long m = idx / NO, n = idx % NO;
    const u32x4* xp = reinterpret_cast<const u32x4*>(X + m * K);
    const u32x4* wp = reinterpret_cast<const u32x4*>(W) + w_row(n);
    float acc = 0.f;
    for (long c = 0; c < K / 8; ++c) acc = dev::dot8(wp[w_col(c)], xp[c], acc);
    if constexpr (E) {           // the up row of output column n is W row NO + n
        const u32x4* up = reinterpret_cast<const u32x4*>(W) + w_row(NO + n);
        float au = 0.f;
        for (long c = 0; c < K / 8; ++c) au = dev::dot8(up[w_col(c)], xp[c], au);
        acc = dev::swiglu<OUT>(acc, au);
    }
    dev::store1<OUT>(Y, idx, acc);
}
