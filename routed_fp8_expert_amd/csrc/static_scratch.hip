// static_scratch.hip -- the workspace of moe_layer_forward_static: a fixed
// array in the library's static device memory, for callers that cannot
// allocate device memory.  Each GPU the library runs on holds its own copy
// until the process ends; every call on a GPU shares it.
//
// The array's name is a host-side stand-in, not a device address: the host
// asks the runtime for the array's address on each device once, with that
// device current (at ctx creation), keeps it, and passes only that address
// to kernels and copies.
#include "kernels.hpp"

#include <mutex>
#include <vector>

namespace moe {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
std::mutex g_mu;
std::vector<void *> g_ptr;   // device address of `scratch`, indexed by device
}  // namespace

hipError_t static_scratch_init(int device) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (device < 0) return hipErrorInvalidDevice;
    if ((int)g_ptr.size() <= device) g_ptr.resize(device + 1, nullptr);
    if (g_ptr[device]) return hipSuccess;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[device] = p;
    return hipSuccess;
}

void *static_scratch_ptr(int device) {
    std::lock_guard<std::mutex> lock(g_mu);
    return device >= 0 && device < (int)g_ptr.size() ? g_ptr[device] : nullptr;
}

}  // namespace moe
