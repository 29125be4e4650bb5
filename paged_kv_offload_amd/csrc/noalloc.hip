// noalloc.hip - the device scratch of kvx_restore_noalloc: per-layer
// completion counters and the unit queue of a publishing RESTORE, in a
// file-scope device array instead of memory the library allocates, for
// callers that cannot allocate (code under graph capture, serving loops,
// harnesses that forbid allocation).
//
// Each GPU holds its own copy of the array, at its own address, until the
// process ends. In host code the array's name is only a host-side stand-in:
// its device address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address is passed to
// kernels. Every call on a GPU shares that GPU's copy and finds it as the
// last call left it; the caller clears what must start at zero.
#include "kvx_internal.h"

namespace kvx {

namespace {

constexpr int kMaxDevices = 64;

// [0, kNoAllocMaxLayers): per-layer unit counters; [kNoAllocMaxLayers]: the
// unit queue; the rest pads to a multiple of 64 words.
static __device__ __align__(256) uint32_t scratch[kNoAllocScratchWords];

std::mutex g_scratch_mu;
uint32_t* g_scratch_dev[kMaxDevices] = {};

}  // namespace

int noalloc_scratch(int device, uint32_t** out)
{
    if (device < 0 || device >= kMaxDevices)
        return fail(KVX_E_INVAL, "restore_noalloc: GPU " + std::to_string(device) +
                                     " is beyond the devices the scratch table covers");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_dev[device]) {
        DeviceGuard dg(device);
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess || cur != device) {
            (void)hipGetLastError();
            return fail(KVX_E_HIP, "restore_noalloc: cannot make GPU " + std::to_string(device) +
                                       " current to look up its scratch");
        }
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(KVX_E_HIP, std::string("restore_noalloc: hipGetSymbolAddress of the device "
                                               "scratch failed: ") +
                                       hipGetErrorString(e));
        }
        g_scratch_dev[device] = static_cast<uint32_t*>(p);
    }
    *out = g_scratch_dev[device];
    return KVX_OK;
}

}  // namespace kvx
