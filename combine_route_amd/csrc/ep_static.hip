// ep_plan_static (include/ep.h): plans whose workspace is the library's own
// static device array, for callers that cannot allocate device memory.
//
// The array lives in every device's copy of the library's code object. Its
// name in host code is only a host-side stand-in for the symbol, not a device
// address: the address is looked up once per device with hipGetSymbolAddress,
// with that device current, and only that address reaches kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ep.h"
#include "ep_kernels.h"
#include "ep_static.h"

namespace {

__device__ __align__(256) uint8_t scratch[EP_STATIC_SCRATCH_BYTES];

std::mutex g_mutex;                     // guards g_scratch_ptr
void* g_scratch_ptr[ep::kMaxDevices];   // scratch's device address, per device

}  // namespace

extern "C" int ep_plan_static(const ep_config_t* cfg, ep_plan_t** out)
{
    if (!cfg)
        return ep::set_error(EP_ERR_NULL, "cfg is NULL");
    if (!out)
        return ep::set_error(EP_ERR_NULL, "out is NULL");
    const int rc = ep::static_plan_check(cfg, EP_STATIC_SCRATCH_BYTES);
    if (rc != EP_OK)
        return rc;
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess)
        return ep::set_error(EP_ERR_HIP, "hipGetDevice failed");
    if (device < 0 || device >= ep::kMaxDevices)
        return ep::set_error(EP_ERR_ARG, "ep_plan_static serves devices 0..63");
    void* ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        if (!g_scratch_ptr[device]) {
            void* p = nullptr;
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return ep::set_error(EP_ERR_HIP, "hipGetSymbolAddress of the static scratch "
                                     "failed on the current device");
            g_scratch_ptr[device] = p;
        }
        ptr = g_scratch_ptr[device];
    }
    return ep::static_plan_reset(cfg, ptr, EP_STATIC_SCRATCH_BYTES, device, out);
}
