// noalloc.hip -- the MLP forward for callers that cannot allocate device memory: its workspace
// is a file-scope device array, one copy per GPU, held until the process ends.
//
// The array's name is a host-side stand-in in host code: kernels and HIP calls only ever get the
// device address that hipGetSymbolAddress returns, fetched once per device at set-up (from
// vqmlp_create, with that device current) and kept in a per-device table.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "internal.h"
#include "vqmlp.h"

namespace vqmlp {

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

struct Slot {
    bool tried = false;
    void* ptr = nullptr;   // device address of this device's copy of `scratch`
    std::string error;     // why the set-up failed (ptr == nullptr)
};
std::mutex g_mutex;
Slot g_slots[kMaxDevices];

}  // namespace

// Once per device, with that device current: the address of this device's copy of the array,
// then a zero fill of the whole array (the fused kernel's control block must start at zero and
// its hand-off words must carry no tag of a call yet to come).  Synchronous; never called inside
// a forward.
void noalloc_setup() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return;
    std::lock_guard<std::mutex> lock(g_mutex);
    Slot& s = g_slots[dev];
    if (s.tried) return;
    s.tried = true;
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
        s.error = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
        return;
    }
    e = hipMemset(ptr, 0, kScratchBytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        s.error = std::string("zero fill of the scratch array: ") + hipGetErrorString(e);
        return;
    }
    s.ptr = ptr;
}

}  // namespace vqmlp

#define noalloc_fail(st, ...) static_cast<vqmlp_status>(vqmlp::set_last_error(st, __VA_ARGS__))

extern "C" vqmlp_status vqmlp_forward_noalloc(const vqmlp_plan* plan, int T, const void* x,
                                              void* y, void* stream) {
    using namespace vqmlp;
    if (!plan) return noalloc_fail(VQMLP_ERR_INVALID_ARG, "vqmlp_forward_noalloc: null plan");
    size_t need = 0;
    vqmlp_status st = vqmlp_workspace_bytes(plan, T, &need);
    if (st) return st;
    if (need > kScratchBytes)
        return noalloc_fail(VQMLP_ERR_WORKSPACE,
                            "vqmlp_forward_noalloc: this forward needs %zu workspace bytes, the "
                            "fixed scratch array holds %zu (use vqmlp_forward with a workspace)",
                            need, kScratchBytes);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return noalloc_fail(VQMLP_ERR_HIP, "vqmlp_forward_noalloc: no current device");
    void* ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        const Slot& s = g_slots[dev];
        if (!s.tried)
            return noalloc_fail(VQMLP_ERR_UNSUPPORTED,
                                "vqmlp_forward_noalloc: no plan was created with device %d "
                                "current (vqmlp_create sets up that device's scratch array)",
                                dev);
        if (!s.ptr)
            return noalloc_fail(VQMLP_ERR_HIP, "vqmlp_forward_noalloc: device %d: %s", dev,
                                s.error.c_str());
        ptr = s.ptr;
    }
    return vqmlp_forward(plan, T, x, y, ptr, kScratchBytes, stream);
}
