// oz2_scratch.hip -- the fixed device scratch behind oz2_dgemm_noalloc, for
// callers that cannot allocate device memory during a call (HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// One file-scope device array of kScratchBytes per GPU, allocated with the
// code object when the library loads on that GPU and held until the process
// ends.  In host code the array's name is only a host-side stand-in, so its
// device address is taken once per device with hipGetSymbolAddress (with
// that device current) and cached; kernels receive that address as an
// ordinary argument, like the workspace of oz2_dgemm.  Every call on a GPU
// shares that GPU's array: calls that overlap on one GPU race.
#include <mutex>

#include "oz2.h"
#include "oz2_internal.h"

namespace oz2 {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

int scratch_address(int device, void** out) {
    *out = nullptr;
    if (device < 0 || device >= kMaxDevices) return OZ2_STATUS_NOT_SUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_addr[device]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess || cur != device) return OZ2_STATUS_HIP_ERROR;
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return OZ2_STATUS_HIP_ERROR;
        }
        g_addr[device] = p;
    }
    *out = g_addr[device];
    return OZ2_STATUS_SUCCESS;
}

}  // namespace oz2
