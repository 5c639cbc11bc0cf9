/*
 * proj.h -- C ABI of libproj: shape-specialised bf16 weight projections
 *           Y[M,N] = X[M,K] . W[N,K]^T on one AMD Instinct MI355X (gfx950).
 *
 * The operation is the weight projection of a decoder layer and of its output
 * head, as in the blog series "On descend d'un cran": weights and activations
 * in bf16, accumulators in f32, nothing quantised ("On descend d'un cran"
 * (post 0), section "Ce qu'il y aura dans le depot"; "#002 le meme compilateur
 * sur un GPU", section "Le contrat numerique").  N and K are fixed when a plan
 * is created; the row count M is the only dimension chosen per call ("#001 un
 * compilateur pour moteur de LLM", section "Un compilateur, pas une
 * bibliotheque de kernels").
 *
 * Conventions for every entry point below:
 *   - X, W, Y and every other buffer argument are DEVICE pointers on the
 *     plan's device unless stated otherwise; the caller owns them.
 *   - X [M,K], W [N,K], Y [M,N] are dense row-major, except W for a plan
 *     created with PROJ_W_PACKED (the packed layout of proj_pack_weights).  X
 *     and W hold bf16 bit patterns; Y holds f32 (PROJ_OUT_F32) or bf16
 *     (PROJ_OUT_BF16).  All three must be 16-byte aligned; Y must not overlap
 *     X or W (both checked: PROJ_EINVAL).
 *   - Work is enqueued on `stream` (a HIP stream of the plan's device, or NULL
 *     for the null stream) and the call returns without synchronising and
 *     without allocating.
 *   - Return codes are PROJ_OK (0) or a negative PROJ_E* value; on failure
 *     nothing was enqueued and proj_last_error() describes the cause.
 *   - The library is thread-safe across plans.  One plan may be used from
 *     several host threads, but its launches that use the split-K workspace
 *     must not overlap on the device: use one plan per concurrently running
 *     stream.
 */
#ifndef PROJ_H
#define PROJ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef struct proj_plan proj_plan; /* opaque; owned by the library */

/* Storage type of Y.  X and W are always bf16. */
enum { PROJ_OUT_F32 = 0, PROJ_OUT_BF16 = 1 };

/* Flags of proj_plan_create_ex: work folded into a plan's kernels, and the
 * layout its kernels read W in. */
enum { PROJ_EPI_NONE = 0, PROJ_EPI_SWIGLU = 1, PROJ_PRO_RMSNORM = 2, PROJ_W_PACKED = 4 };

enum {
    PROJ_OK = 0,
    PROJ_EINVAL = -1,   /* bad argument: null or misaligned pointer, bad size or dtype, wrong device */
    PROJ_EDEVICE = -2,  /* a HIP call failed (message holds the HIP error string) */
    PROJ_ECOMPILE = -3, /* hipRTC could not compile the generated source */
    PROJ_ENOCAND = -4,  /* no candidate kernel passed validation for some row bucket */
    PROJ_ENOMEM = -5    /* device allocation failed */
};

/*
 * Build a plan for Y = X . W^T with fixed N (rows of W) and K (row length).
 *
 * Emits HIP source with N, K, tile sizes and trip counts as literals, compiles
 * it with hipRTC for the current device, then, for each row bucket
 * {1}, {2..16}, {17..128}, {129..512}, {513..1024}, {1025..2048}, {2049..8192},
 * validates every candidate kernel on synthetic probe inputs (full and partial
 * block, NaN-sentinel output, integer probe bit-exact) against a plain
 * reference kernel on sampled rows and, on the integer probe, against the
 * plain kernel's whole output (an order-independent hash of every element),
 * times the ones that pass and keeps the fastest: the
 * load-time tuner with its correctness gate of "#004 the same compiler on
 * Apple's chips", sections "Catching up on prefill" and "The night the engine
 * chose wrong".  Blocks for seconds.
 *
 * N >= 1, K >= 8 with K % 8 == 0, dtype in {PROJ_OUT_F32, PROJ_OUT_BF16}.
 * The plan is bound to the device current at the call.  Returns NULL on
 * failure (see proj_last_error()).
 *
 * Environment (read at creation): PROJ_LOG=1 prints the tuner log to stderr;
 * PROJ_TUNE=0 skips timing and takes the first candidate that validates;
 * PROJ_TUNE_REPS=<n> (default 10, at least 3) sets the timing rounds of each
 * candidate that a first screen of three rounds puts within 10 % of the best (a
 * round: launches back to back on rotating copies of the probe weights that
 * exceed the last-level cache); PROJ_FORCE=<name>
 * keeps only that candidate (plus the plain kernel) where it applies;
 * PROJ_DUMP_DIR=<dir> writes the generated source and code object there;
 * PROJ_CACHE_DIR=<dir> turns on the persistent tuning cache: the choices of a
 * tuned plan are written to <dir>/proj-<key>.txt, where the key hashes the
 * device (architecture name, CU count), the HIP runtime and driver versions
 * and the complete generated source; a later plan with the same key runs
 * every cached choice through the same validation gate instead of timing
 * candidates, and tunes afresh any bucket whose cached choice is unknown or
 * fails the gate (the cache the pages propose, and doubt because machine state
 * drifts: "#004 the same compiler on Apple's chips", section "So, does it start
 * up more slowly?").  The compiled modules are kept under the same key
 * (<dir>/proj-<key>.m<g>.co, the key also covering the compiler and its
 * options), so such a plan skips hipRTC as well; a file that does not load is
 * compiled afresh and replaced.
 * proj_plan_describe reports "cache" and "code_cache": off, miss, hit or stale.
 */
proj_plan* proj_plan_create(int64_t N, int64_t K, int dtype);

/*
 * Like proj_plan_create, with work folded into the plan's kernels or with
 * weights in the packed layout; `flags` is PROJ_EPI_NONE or an OR of the flags
 * below.  The pages fuse exactly these two: each RMSNorm into the projection
 * after it and the SwiGLU activation into the gate_up projection, with results
 * identical bit for bit to the unfused kernels ("#004 the same compiler on
 * Apple's chips", section "Decode").
 *
 * PROJ_EPI_SWIGLU: W is a fused gate_up matrix, rows [0, N/2) the gate
 * projection and rows [N/2, N) the up projection (N even), and the plan's Y is
 * [M, N/2] with
 *     Y[m, j] = silu(g) * u,   silu(g) = g / (1 + exp(-g)),
 *     g = (X . W^T)[m, j],  u = (X . W^T)[m, N/2 + j],
 * evaluated in f32 on the f32 sums; with PROJ_OUT_BF16, g and u are first
 * rounded to bf16 (the values a plain plan would store) and the product is
 * rounded to bf16 once.  The result is bit-identical to the unfused path -- a
 * plain plan running the same kernel variant, then proj_swiglu on its output --
 * while writing N/2 columns instead of N and skipping one launch and the round
 * trip of the N-column intermediate: the SwiGLU folded into the gate_up
 * projection of "#004 the same compiler on Apple's chips", section "Decode"
 * (a fusion there changes no output bit), and of "#002
 * le meme compilateur sur un GPU", section "Emettre pour un GPU" (the
 * activation fused with the projection that produces its input).  The fused
 * candidates come from the kernel families that have the epilogue (vector
 * GEMVs with an even row count per wave, whole-tile MFMA GEMMs, the plain
 * kernel); every other candidate of a plain plan is compiled as well and run
 * unfused -- its N-column projection into an intermediate of the plan (as
 * many rows of N values as fit 256 MiB, at most 8192), then the activation
 * kernel -- and the load-time tuner picks between fused and unfused per row
 * bucket, the fusion being an option measured at load (same page and section).
 * The tuner's gate holds a SwiGLU candidate to bit equality on the integer
 * probe and, on the random probe, to an allowance derived from the plain
 * projection's f32 rule on g and u carried through silu (Lipschitz constant
 * 1.1) plus the bf16 roundings of g, u and Y: candidates sum g and u in
 * different orders, and one bf16 step of g near a rounding boundary moves
 * silu(g) * u by more than one bf16 step of Y.
 *
 * PROJ_PRO_RMSNORM: X is normalised first, row by row, as by proj_rmsnorm with
 * epsilon `norm_eps` (a constant of the generated code) and the norm weights
 * `gamma` passed to proj_run_ex; Y is then the projection of the normalised
 * rows, bit-identical to proj_rmsnorm followed by a plain plan running the
 * same kernel variant.  Every candidate of the plan can run unfused (the norm
 * kernel into a workspace of the plan, 8192 x K bf16, then the candidate on
 * it); the vector GEMVs for M = 1 also come with the norm folded in (each
 * block normalises the row into LDS first), and the load-time tuner picks
 * between them by measurement -- the pages find the folded norm faster on
 * small models and slower from the 4B on, where every workgroup re-reads the
 * whole row.  proj_run on such a plan fails with PROJ_EINVAL: use proj_run_ex.
 *
 * PROJ_W_PACKED: every kernel of the plan reads W in the packed layout that
 * proj_pack_weights writes (N % 128 == 0 and K % 64 == 0), and the plan runs
 * through proj_run_packed (proj_run and proj_run_ex fail with PROJ_EINVAL).
 * Each candidate reads the same values in the same order as on row-major
 * weights, so a packed plan gives the same bits as a row-major plan running
 * the same kernel variant; only the memory addresses change.  Combines with
 * the two flags above.
 *
 * Unknown flags, an odd N with PROJ_EPI_SWIGLU, a negative or non-finite
 * norm_eps with PROJ_PRO_RMSNORM, or a shape without whole 128 x 64 blocks with
 * PROJ_W_PACKED return NULL with PROJ_EINVAL in proj_last_error.  norm_eps is
 * ignored without PROJ_PRO_RMSNORM; proj_plan_create_ex(N, K, dtype,
 * PROJ_EPI_NONE, 0) is proj_plan_create.
 */
proj_plan* proj_plan_create_ex(int64_t N, int64_t K, int dtype, int flags, float norm_eps);

/*
 * Enqueue Y[0:M, :] = X[0:M, :] . W^T on `stream`.  Rows of Y at or past M are
 * never written.  M == 0 returns PROJ_OK without launching; M < 0, an M for
 * which X or Y would exceed 2^48 bytes, null or misaligned pointers, or a
 * current device other than the plan's give PROJ_EINVAL; a failed launch
 * gives PROJ_EDEVICE.  M above 8192 is processed
 * as consecutive blocks of at most 8192 rows.
 *
 * Only kernel launches are enqueued (one, or two for split-K and split-tail
 * kernels whose second pass sums f32 partials kept in the plan's workspace):
 * no allocation, no synchronisation, no memset, so the call may be recorded
 * into a HIP graph by stream capture.  Calls on one plan share its workspace:
 * they must not run concurrently (different streams without ordering, or
 * overlapping graph replays).  A plan created with PROJ_W_PACKED gives
 * PROJ_EINVAL here: it runs through proj_run_packed.
 */
int proj_run(const proj_plan* plan, const void* X, const void* W, void* Y, int64_t M,
             hipStream_t stream);

/* proj_run with the norm weights of a PROJ_PRO_RMSNORM plan: gamma is a device
 * pointer to K f32 values, 16-byte aligned, owned by the caller (NULL for
 * plans without the prologue; missing or misaligned for one: PROJ_EINVAL). */
int proj_run_ex(const proj_plan* plan, const void* X, const void* W, void* Y, int64_t M, const float* gamma,
                hipStream_t stream);

/*
 * proj_run_ex for callers that cannot allocate device memory while they run:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same kernels, same results bit for bit, same arguments and
 * errors as proj_run_ex (row-major W; gamma for a PROJ_PRO_RMSNORM plan), but
 * the workspace of the tuned kernel for M -- split-K and split-tail partials,
 * the normalised rows of an unfused RMSNorm candidate, the N-column
 * intermediate of an unfused SwiGLU candidate -- comes from a static device
 * array of the library, 64 MiB per GPU, instead of from the plan; the call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * The array is looked up on a device once, when the first plan is created
 * there, and is held until the process ends.  A call whose kernel needs more
 * than 64 MiB at its M (e.g. split tails of the widest shapes at thousands of
 * rows) returns PROJ_EINVAL naming the bytes needed, with nothing enqueued:
 * use fewer rows per call.  Nothing in the array needs to start at zero: every
 * kernel writes the partials it reads.  All proj_run_noalloc calls on one GPU
 * share its array, so calls that overlap on the device (different streams
 * without ordering, overlapping graph replays) race; calls on one stream are
 * ordered.  They do not share the plan's own workspace, so they do not race
 * with proj_run / proj_run_ex calls of the plan.
 */
int proj_run_noalloc(const proj_plan* plan, const void* X, const void* W, void* Y, int64_t M, const float* gamma,
                     hipStream_t stream);

/*
 * Load-time weight repacking.  Enqueue the copy of the row-major weights W
 * [N, K] (bf16 bit patterns) into Wp, the same N * K values in the packed
 * layout: W is cut into panels of 128 consecutive rows, each panel is stored
 * as K/64 consecutive blocks of 128 rows x 64 values, each block row-major, so
 *     Wp[((n / 128) * (K / 64) + k / 64) * 8192 + (n % 128) * 64 + k % 64] = W[n][k].
 * A 64-value slice of 128 rows -- what one k-step of an MFMA tile reads -- is
 * then one contiguous 16 KiB block instead of 128 separate 128-byte pieces; a
 * decode GEMV still reads each row in 128-byte runs.  The pages pack their
 * weights in the order their kernels read them (16-column blocks at a fixed
 * distance: "#001 un compilateur pour moteur de LLM", section "Lire le meme
 * emetteur rempli deux fois"; aligned to cache lines: section "Les chiffres"),
 * and expect the layout to pay on GPUs too, to be measured kernel by kernel
 * ("#002 le meme compilateur sur un GPU", section "Les autres cartes").
 *
 * N % 128 == 0 and K % 64 == 0; W and Wp are caller-owned device buffers of
 * N * K * 2 bytes, 16-byte aligned and not overlapping (no in-place packing).
 * Independent of any plan: pack once at load, then run any PROJ_W_PACKED plan
 * of that shape on Wp with proj_run_packed.  N == 0 or K == 0 is a no-op;
 * other shapes, null, misaligned or overlapping buffers give PROJ_EINVAL.
 */
int proj_pack_weights(int64_t N, int64_t K, const void* W, void* Wp, hipStream_t stream);

/*
 * proj_run_ex for a plan created with PROJ_W_PACKED: Wp holds the weights in
 * the packed layout (proj_pack_weights); gamma as in proj_run_ex (required for
 * a PROJ_PRO_RMSNORM plan, NULL otherwise).  Same results, bit for bit, as a
 * plan without PROJ_W_PACKED running the same kernel variant on the row-major
 * W; same errors as proj_run_ex, and PROJ_EINVAL for a plan without
 * PROJ_W_PACKED.
 */
int proj_run_packed(const proj_plan* plan, const void* X, const void* Wp, void* Y, int64_t M, const float* gamma,
                    hipStream_t stream);

/* Free the plan's modules and workspace.  NULL-safe.  Waits first for all
 * work queued on the plan's device to finish (hipDeviceSynchronize), so a
 * launch of the plan still pending on any stream completes before its kernels
 * and workspace go away; so it must not be called during a stream capture on
 * that device. */
void proj_plan_destroy(proj_plan* plan);

/* Message of the last failure on the calling thread ("" if none).  The pointer
 * stays valid until the next library call on this thread. */
const char* proj_last_error(void);

/* ---- introspection and forced variants (tests, benchmarks, ablations) ---- */

/*
 * Write the HIP source a plan for (N, K, dtype) would compile for device
 * architecture `arch` (e.g. "gfx950"), NUL-terminated, into host buffer `buf`
 * of `cap` bytes; `*needed` (if not NULL) receives the size including the NUL.
 * Needs no GPU.  Returns PROJ_EINVAL for bad shapes or if cap is too small
 * (buf may be NULL to query the size).  The analogue of the pages' option that
 * dumps emitted code ("#001 un compilateur pour moteur de LLM", section "Lire
 * le meme emetteur rempli deux fois").
 */
int proj_emit_source(int64_t N, int64_t K, int dtype, const char* arch, char* buf, size_t cap,
                     size_t* needed);
/* The same for a plan with fused work or packed weights (proj_plan_create_ex's flags and epsilon). */
int proj_emit_source_ex(int64_t N, int64_t K, int dtype, int flags, float norm_eps, const char* arch, char* buf,
                        size_t cap, size_t* needed);

/*
 * Emit and compile, for device architecture `arch` (NULL: "gfx950"), every
 * module a plan for (N, K, dtype, flags, norm_eps) would load -- the same
 * sources and the same hipRTC options as proj_plan_create_ex -- without a GPU
 * and without keeping the code.  *seconds (if not NULL) receives the wall
 * time.  PROJ_OK, PROJ_EINVAL for arguments proj_plan_create_ex would reject,
 * or PROJ_ECOMPILE with hipRTC's log in proj_last_error().  The compilation
 * step alone: the pages report it separately from the tuning measurements
 * ("#004 the same compiler on Apple's chips", section "So, does it start up
 * more slowly?").
 *
 * Compilation (here and in proj_plan_create_ex) runs in up to PROJ_RTC_JOBS
 * (default: the CPUs the process may use, at most 16) child processes of the
 * helper proj_rtc installed beside the library, one per module, since hipRTC
 * compiles one program at a time per process.  Without the helper, or with
 * PROJ_RTC_JOBS=0, the modules are compiled one after another in the calling
 * process, by whichever hipRTC library it has loaded.
 */
int proj_compile_only(int64_t N, int64_t K, int dtype, int flags, float norm_eps, const char* arch,
                      double* seconds);

/* JSON text (host buffer) describing the plan: shape, candidates, per-bucket
 * choice and timings, the tuner log, compile and tuning seconds.  Same size
 * protocol as proj_emit_source. */
int proj_plan_describe(const proj_plan* plan, char* buf, size_t cap, size_t* needed);

/* Number of compiled candidates, and the name of candidate `idx` (host buffer). */
int proj_plan_num_candidates(const proj_plan* plan);
int proj_plan_candidate_name(const proj_plan* plan, int idx, char* buf, size_t cap);

/* Rows this candidate accepts per launch (16 for the GEMV families, 8192 for
 * the tiled GEMMs, fewer for a split-K GEMM whose partials would not fit the
 * plan's workspace), or a negative error code. */
int64_t proj_plan_candidate_max_m(const proj_plan* plan, int idx);

/*
 * Like proj_run but with candidate `idx` instead of the tuned choice; M must
 * be within the candidate's limit (proj_plan_candidate_max_m); W is in the
 * plan's layout (packed for a PROJ_W_PACKED plan).  The analogue of
 * the pages' command-line override of a tuned variant ("#004 the same compiler
 * on Apple's chips", section "Reproducing at home").
 */
int proj_run_candidate(const proj_plan* plan, int idx, const void* X, const void* W, void* Y,
                       int64_t M, hipStream_t stream);
/* ... with the norm weights of a PROJ_PRO_RMSNORM plan (as proj_run_ex). */
int proj_run_candidate_ex(const proj_plan* plan, int idx, const void* X, const void* W, void* Y, int64_t M,
                          const float* gamma, hipStream_t stream);

/* Index of the candidate proj_run uses for M rows (M >= 1), or a negative error. */
int proj_plan_choice(const proj_plan* plan, int64_t M);

/* ---- the unfused activation (shape-independent) ---- */

/*
 * Enqueue H[m, j] = silu(G[m, j]) * G[m, N/2 + j] for m < M, j < N/2: the
 * SwiGLU of a plain gate_up projection's output G [M, N] into H [M, N/2], both
 * of storage type dtype (f32, or bf16 read and written as bit patterns), dense
 * row-major device buffers owned by the caller, H not overlapping G.  The
 * same f32 operations and roundings as the PROJ_EPI_SWIGLU epilogue -- the
 * separate kernel that epilogue replaces ("#004 the same compiler on Apple's
 * chips", section "Decode").  N must be even; M == 0 or N == 0 is a no-op;
 * negative sizes, odd N, a bad dtype, null pointers, G or H not aligned to
 * the element size, or H overlapping G give PROJ_EINVAL.
 */
int proj_swiglu(const void* G, void* H, int64_t M, int64_t N, int dtype, hipStream_t stream);

/*
 * Enqueue the RMSNorm of each of the M rows of X [M, K] (bf16 bit patterns)
 * into Xn [M, K] (bf16): with ss = sum_k x_k^2 in f32 in one fixed order (a
 * 256-thread block per row: thread t adds k = t, t + 256, ... with FMA, then
 * pairwise halving of the 256 partials),
 *     r = 1 / sqrt(ss / K + eps),   Xn[m][k] = bf16((x_k * r) * gamma[k]),
 * the products in f32, IEEE division and square root, one rounding to bf16.
 * gamma is K f32 values (pass 1 + w for a norm whose weights are centred on
 * zero).  The separate kernel that the PROJ_PRO_RMSNORM prologue replaces
 * ("#004 the same compiler on Apple's chips", section "Decode").  Device
 * pointers owned by the caller; Xn must not overlap X.  M == 0 or K == 0 is a
 * no-op; negative sizes, a negative or non-finite eps, M >= 2^31 or null
 * pointers, X or Xn not 2-byte aligned, gamma not 4-byte aligned, or Xn
 * overlapping X or gamma give PROJ_EINVAL.
 */
int proj_rmsnorm(const void* X, const float* gamma, void* Xn, int64_t M, int64_t K, float eps, hipStream_t stream);

/* ---- measurement support (shape-independent) ---- */

/*
 * Enqueue one streaming read of `bytes` bytes at device pointer `buf`
 * (16-byte aligned, bytes % 16 == 0) with non-temporal 16-byte loads over the
 * whole device; `sink` is a device pointer to 4 writable bytes that is written
 * only in the practically impossible case that the XOR of all data equals
 * `never`.  Time it with events on `stream` to get the device's read bandwidth,
 * the denominator the pages measure instead of assuming ("#001 un compilateur
 * pour moteur de LLM", section "Mesurer la limite plutot que la supposer").
 */
int proj_probe_read(const void* buf, int64_t bytes, uint32_t never, void* sink, hipStream_t stream);

/*
 * Enqueue out[i] = bf16_rne(in[i]) for i < n with the exact device function
 * the projection epilogue uses (in: f32 device array, out: uint16 device
 * array).  Exposed so that the epilogue rounding can be checked on all 2^32
 * f32 patterns, as the pages check their GPU's f32 -> f16 conversion ("#004
 * the same compiler on Apple's chips", section "f16").  n == 0 is a no-op;
 * negative n, null pointers, `in` not 4-byte or `out` not 2-byte aligned, or
 * `out` overlapping `in` give PROJ_EINVAL.
 */
int proj_round_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PROJ_H */
