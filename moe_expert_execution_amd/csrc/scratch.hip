// A static per-GPU scratch array for the call that allocates nothing
// (ft_moe_forward_noalloc).  The array lives in each GPU's memory from the
// first use of the library on that GPU until the process ends; its device
// address is looked up once per device with that device current, and host
// code passes that address to kernels (the array's name in host code is a
// host-side stand-in, not a device address).
#include <mutex>

#include "common.h"

namespace ftmoe {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch_setup(int device) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_scratch[device]) return hipSuccess;
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;   // the caller makes `device` current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[device] = p;
    return hipSuccess;
}

void* static_scratch(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_mu);
    return g_scratch[device];
}

}  // namespace ftmoe
