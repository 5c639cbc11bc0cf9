// gate.hip -- validation-gate kernels of the load-time tuner (part of the shape module)

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
    u32 pad;
    u64 hash;         // proj_hash_out: hash of every output element of rows < M
};

// SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom
// number generators", 2014): a bijective 64-bit mixer.
__device__ __forceinline__ u64 mix64(u64 z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Order-independent hash of the first n output elements: the sum mod 2^64 of
// mix64(index, bits) over the elements.  Equal outputs hash equally whatever
// the launch order; a differing element changes the sum unless mixes cancel,
// which the mixer makes vanishingly unlikely.  Used on the integer probe, where
// every candidate's output must equal the plain kernel's bit for bit.
extern "C" __global__ __launch_bounds__(256) void proj_hash_out(const void* __restrict__ Y, long n,
                                                                CheckStats* __restrict__ st)
{
    u64 h = 0;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
        const u64 v = OUT_SEL == OUT_BF16 ? (u64)reinterpret_cast<const u16*>(Y)[i]
                                          : (u64)reinterpret_cast<const u32*>(Y)[i];
        h += mix64(((u64)i << 32) ^ v ^ 0x9E3779B97F4A7C15ull);
    }
    if (h) atomicAdd(&st->hash, h);
}

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

// Spacing of bf16 numbers at |a|: 2^(max(exponent(a), -126) - 7).
__device__ __forceinline__ float bf16_spacing(float a)
{
    a = __builtin_fabsf(a);
    int e = a > 0.f ? (int)((__builtin_bit_cast(u32, a) >> 23) & 0xFF) - 127 : -126;
    e = e < -126 ? -126 : e;
    return __builtin_ldexpf(1.f, e - 7);
}

// Allowance for a SwiGLU output h = silu(g) u against the reference gate and
// up sums g, u ("#004 the same compiler on Apple's chips", section "Decode",
// the activation folded into the gate_up projection).  Each candidate sum g', u' meets the projection's f32 rule, |g' - g| <=
// 1e-3 (|g| + 1); with bf16 output both are rounded to bf16 before the
// activation (relative 2^-9, 2^-8 taken), and a rounding boundary can fall
// between g' and g, so the rounded operands may differ by a whole bf16 ulp.
// silu has Lipschitz constant 1.1, hence |silu(g')u' - silu(g)u| <=
// 1.1 eg (|u| + eu) + |silu(g)| eu, plus the f32 evaluation (2^-20 |h|) and,
// for bf16, the store's rounding (one bf16 spacing).  An ulp-of-output rule
// is too tight here: one ulp of g at |g| ~ 8 moves h by more than one ulp.
template <int OUT>
__device__ __forceinline__ float swiglu_allowance(float g, float u, float h)
{
    const float ag = __builtin_fabsf(g), au = __builtin_fabsf(u);
    float eg = 1e-3f * (ag + 1.f), eu = 1e-3f * (au + 1.f);
    if constexpr (OUT == OUT_BF16) {
        eg += 0x1p-8f * (ag + eg);
        eu += 0x1p-8f * (au + eu);
    }
    const float s = __builtin_fabsf(g / (1.0f + expf(-g)));
    float a = 1.1f * eg * (au + eu) + s * eu + 0x1p-20f * __builtin_fabsf(h);
    if constexpr (OUT == OUT_BF16) a += bf16_spacing(__builtin_fabsf(h) + a);
    return a;
}

// Scans rows [0, rows_alloc) of Y: sentinel bookkeeping on every element, and
// the comparison with ref on the listed rows.  ref holds the plain f32 sums of
// all N columns; with the SwiGLU epilogue, output column n pairs the gate sum
// ref[n] with the up sum ref[NOUT + n].  Tolerance (exact == 0):
//   plain, f32 out:   |y - r| <= 1e-3 (|r| + 1)
//   plain, bf16 out:  |y - R| <= ulp(R) with R = bf16(r), or the f32 rule
//   SwiGLU:           |y - h| <= swiglu_allowance, h = silu(g) u unrounded
// exact == 1: y must equal the reference (through dev::swiglu with the SwiGLU
// epilogue, which rounds as the candidates do) rounded to the output type.
template <int OUT>
__device__ __forceinline__ void check_body(const void* __restrict__ Y, long rows_alloc, int M,
                                           const float* __restrict__ ref, const int* __restrict__ rows,
                                           int nrows, int exact, CheckStats* __restrict__ st)
{
    const long total = rows_alloc * NOUT;
    u32 bad = 0, unw = 0, grd = 0;
    float merr = 0.f, mref = 0.f;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
        const long row = i / NOUT, col = i % NOUT;
        const bool sent = is_sentinel<OUT>(Y, i);
        if (row < M) unw += sent ? 1u : 0u;
        else grd += sent ? 0u : 1u;
        if (row >= M) continue;
        for (int j = 0; j < nrows; ++j) {
            if (rows[j] != row) continue;
            float r, tol = 0.f;
            if constexpr (EPI) {
                const float g = ref[(long)j * N + col], u = ref[(long)j * N + NOUT + col];
                r = exact ? dev::swiglu<OUT>(g, u) : dev::swiglu<OUT_F32>(g, u);
                tol = swiglu_allowance<OUT>(g, u, r);
            } else {
                r = ref[(long)j * N + col];
            }
            const float y = load_out<OUT>(Y, i);
            const float err = __builtin_fabsf(y - r);
            bool ok;
            if (exact) {
                if constexpr (OUT == OUT_F32) ok = __builtin_bit_cast(u32, y) == __builtin_bit_cast(u32, r);
                else ok = reinterpret_cast<const u16*>(Y)[i] == dev::to_bf16(r);
            } else if constexpr (EPI) {
                ok = err <= tol;
            } else {
                ok = err <= 1e-3f * (__builtin_fabsf(r) + 1.f);
                if constexpr (OUT == OUT_BF16) {
                    const float R = __builtin_bit_cast(float, (u32)dev::to_bf16(r) << 16);
                    ok = ok || (__builtin_fabsf(y - R) <= bf16_spacing(R));
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
