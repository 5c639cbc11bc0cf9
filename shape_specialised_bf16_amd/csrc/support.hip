// support.hip -- shape-independent device code: the memory read probe and the
// exposed epilogue rounding.  Compiled once per process and device by hipRTC.

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
