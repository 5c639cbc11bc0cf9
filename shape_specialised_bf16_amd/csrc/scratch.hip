// scratch.hip -- the library's static device scratch, for proj_run_noalloc.
//
// Some callers cannot allocate device memory while they run projections (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  proj_run_noalloc gives them the tuned kernels with their
// workspace -- split-K and split-tail partials, the normalised rows of an
// unfused RMSNorm, the intermediate of an unfused SwiGLU -- taken from this
// array instead of from the plan.  Every GPU the library runs on holds its own
// copy, at its own address, until the process ends.  Compiled by hipcc into
// libproj.so (the projection kernels themselves come from the hipRTC modules
// of each plan and receive the array's device address as an argument).
//
// In host code the name `scratch` is only a host-side stand-in: its device
// address is obtained once per device with hipGetSymbolAddress, with that
// device current, and only that address is used afterwards.
#include <hip/hip_runtime.h>

#include <mutex>

#include "proj.h"
#include "proj_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;   // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

namespace proj {

int set_error(int code, const char* f, ...);

size_t scratch_capacity() { return kScratchBytes; }

int scratch_address(int device, void** ptr)
{
    if (device < 0 || device >= kMaxDevices)
        return set_error(PROJ_EINVAL, "device %d: the static scratch covers devices 0..%d", device, kMaxDevices - 1);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return set_error(PROJ_EDEVICE, "hipGetDevice: %s", hipGetErrorString(e));
        if (cur != device)
            return set_error(PROJ_EINVAL, "the static scratch of device %d is looked up with device %d current",
                             device, cur);
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return set_error(PROJ_EDEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", device,
                             hipGetErrorString(e));
        g_scratch_ptr[device] = p;
    }
    *ptr = g_scratch_ptr[device];
    return PROJ_OK;
}

}  // namespace proj
