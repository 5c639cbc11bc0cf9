// support.hip -- shape-independent device code: the memory read probe, the
// exposed epilogue rounding, the unfused SwiGLU and RMSNorm kernels and the
// weight repacking.  Compiled once per process and device by hipRTC.

// (types and the dev:: helpers come from device_common.hip, prepended by the host)

// Streaming read of n16 16-byte chunks with non-temporal loads, four loads in
// flight per lane per iteration.  The XOR of everything read is stored only if
// it equals a value chosen by the caller, which keeps the loads alive without
// writing in practice.  The GPU analogue of the pages' bandwidth probe: a pure
// sequential read, best of several passes, taken as the denominator beside the
// vendor figure ("#001 un compilateur pour moteur de LLM", section "Mesurer la
// limite plutot que la supposer").
//
// Each block reads one contiguous 32 KiB span (8 loads in flight per lane, each
// wave instruction 1 KiB contiguous) and exits, so the device keeps many short
// waves in flight, the access pattern of a weight-streaming GEMV.
// Grid: ceil(n16 / 2048) blocks of 256 threads.
extern "C" __global__ __launch_bounds__(256) void proj_probe_read(const u32x4* __restrict__ p, long n16,
                                                                  u32 never, u32* __restrict__ sink)
{
    constexpr int LOADS = 8;
    const long base = (long)blockIdx.x * (256 * LOADS) + threadIdx.x;
    u32x4 v[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const long i = base + j * 256;
        v[j] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4{0u, 0u, 0u, 0u};
    }
    u32 acc = 0;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    if (acc == never) sink[0] = acc;
}

// The projection epilogue's f32 -> bf16 conversion, dev::to_bf16 (IEEE round
// to nearest even), applied element-wise so that it can be checked on every f32 pattern.
extern "C" __global__ __launch_bounds__(256) void proj_round_bf16(const float* __restrict__ in,
                                                                  u16* __restrict__ out, long n)
{
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
        out[i] = dev::to_bf16(in[i]);
}

// The SwiGLU activation as a kernel of its own -- the unfused path that the
// projection's fused epilogue must reproduce bit for bit: G [M, N] holds the
// gate_up projection (gate in columns [0, N/2), up in [N/2, N)), H [M, N/2]
// receives dev::swiglu(gate, up) stored with the same rounding.
template <int OUT>
__device__ __forceinline__ void swiglu_rows(const void* __restrict__ G, void* __restrict__ H, long M, long N)
{
    const long half = N / 2;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < M * half; i += (long)gridDim.x * blockDim.x) {
        const long m = i / half, j = i % half;
        float g, u;
        if constexpr (OUT == OUT_F32) {
            g = reinterpret_cast<const float*>(G)[m * N + j];
            u = reinterpret_cast<const float*>(G)[m * N + half + j];
        } else {
            g = dev::lo_bf16(reinterpret_cast<const u16*>(G)[m * N + j]);
            u = dev::lo_bf16(reinterpret_cast<const u16*>(G)[m * N + half + j]);
        }
        dev::store1<OUT>(H, i, dev::swiglu<OUT>(g, u));
    }
}

extern "C" __global__ __launch_bounds__(256) void proj_swiglu_f32(const void* G, void* H, long M, long N)
{
    swiglu_rows<OUT_F32>(G, H, M, N);
}

extern "C" __global__ __launch_bounds__(256) void proj_swiglu_bf16(const void* G, void* H, long M, long N)
{
    swiglu_rows<OUT_BF16>(G, H, M, N);
}

// The RMSNorm as a kernel of its own -- the unfused path that the fused
// prologue must reproduce bit for bit: one block of 256 threads per row of
// X [M, K] (bf16), Xn[m][k] = bf16((X[m][k] * r_m) * gamma[k]) with gamma f32
// [K] and r_m from dev::rms_scale_block.  Grid: M blocks.
extern "C" __global__ __launch_bounds__(256) void proj_rmsnorm_rows(const u16* __restrict__ X,
                                                                    const float* __restrict__ gamma,
                                                                    u16* __restrict__ Xn, long K, float eps)
{
    __shared__ float red[256];
    const u16* x = X + (long)blockIdx.x * K;
    const float r = dev::rms_scale_block(x, K, eps, red);
    u16* xn = Xn + (long)blockIdx.x * K;
    for (long k = threadIdx.x; k < K; k += 256) xn[k] = dev::rms_apply(x[k], r, gamma[k]);
}

// Weight repacking into the panel layout (dev::kPanelRows x dev::kPanelCols
// blocks, see device_common): Wp receives the row-major W [N, K] (bf16 bit
// patterns; N % 128 == 0, K % 64 == 0).  One thread per 16-byte chunk of Wp,
// taken in Wp order: the writes are contiguous and each group of 8 lanes reads
// one 128-byte run of a weight row.  Grid-stride over all N * K / 8 chunks.
extern "C" __global__ __launch_bounds__(256) void proj_pack_panels(const u32x4* __restrict__ W,
                                                                   u32x4* __restrict__ Wp, long N, long K)
{
    const long CH = K / 8;                              // chunks per weight row
    const long blocks = K / dev::kPanelCols;            // 64-value blocks per row
    const long total = N * CH;
    for (long j = (long)blockIdx.x * blockDim.x + threadIdx.x; j < total; j += (long)gridDim.x * blockDim.x) {
        const long q = j & 7;                           // chunk within the block row
        const long r = (j >> 3) & (dev::kPanelRows - 1);  // row within the panel
        const long b = (j >> 10) % blocks;              // 64-value block along K
        const long p = (j >> 10) / blocks;              // panel
        Wp[j] = W[(p * dev::kPanelRows + r) * CH + b * 8 + q];
    }
}
