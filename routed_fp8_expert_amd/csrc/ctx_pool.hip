// ctx_pool.hip -- the ctxs' synchronisation words in static device memory.
//
// Each ctx needs kCtxWords words of device memory that start at zero
// (tickets, flags, counters, the error word).  They come from a fixed pool
// compiled into the library's code object -- kMaxCtxPerDevice slots per
// device, each GPU holding its own copy of the array until the process ends
// -- so creating a ctx allocates no device memory.  The host never uses the
// array's name as an address: per device, with that device current, it asks
// the runtime for the array's address once and keeps it.
#include "kernels.hpp"

#include <mutex>
#include <vector>

namespace moe {

static __device__ __align__(256) uint32_t ctx_words[kMaxCtxPerDevice][kCtxWords];

namespace {

struct DevicePool {
    uint32_t *base = nullptr;           // device address of ctx_words on this device
    bool used[kMaxCtxPerDevice] = {};
};

std::mutex g_mu;
std::vector<DevicePool> g_pools;        // indexed by device

}  // namespace

// `device` must be the current device.
hipError_t ctx_slot_acquire(int device, int *slot, uint32_t **words) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (device < 0) return hipErrorInvalidDevice;
    if ((int)g_pools.size() <= device) g_pools.resize(device + 1);
    DevicePool &p = g_pools[device];
    if (!p.base) {
        void *addr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(ctx_words));
        if (e != hipSuccess) return e;
        p.base = static_cast<uint32_t *>(addr);
    }
    int s = 0;
    while (s < kMaxCtxPerDevice && p.used[s]) ++s;
    if (s == kMaxCtxPerDevice) return hipErrorOutOfMemory;
    uint32_t *w = p.base + (size_t)s * kCtxWords;
    hipError_t e = hipMemset(w, 0, sizeof(uint32_t) * kCtxWords);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return e;
    p.used[s] = true;
    *slot = s;
    *words = w;
    return hipSuccess;
}

hipError_t ctx_layer_words_reset(uint32_t *words) {
    hipError_t e = hipMemset(words + kWordLayerSync, 0, sizeof(uint32_t) * kLayerSyncWords);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    return e;
}

void ctx_slot_release(int device, int slot) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (device >= 0 && device < (int)g_pools.size() && slot >= 0 && slot < kMaxCtxPerDevice)
        g_pools[device].used[slot] = false;
}

}  // namespace moe
