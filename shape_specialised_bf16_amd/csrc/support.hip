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
extern "C" __global__ __launch_bounds__(256) void proj_probe_read(const u32x4* __restrict__ p, long n16,
                                                                  u32 never, u32* __restrict__ sink)
{
    const long stride = (long)gridDim.x * blockDim.x;
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    u32 acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        const u32x4 b = __builtin_nontemporal_load(p + i + stride);
        const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n16; i += stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
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
