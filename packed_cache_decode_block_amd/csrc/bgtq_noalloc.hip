// Decode attention for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc): the split-K partials of
// bgtq_decode_attention live in a fixed device array of this library instead of a caller
// workspace.  Every call on one GPU uses that GPU's copy of the array, so calls that overlap on
// one GPU (other streams, other threads) race; calls in order on one stream are safe.  Every
// partial record a call reads back was written earlier in the same call, so the array needs no
// clearing between calls.
#include <mutex>

#include "bgtq_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)BGTQ_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// One copy per GPU the library runs on, held until the process ends.  Its name is a host-side
// stand-in: only the address hipGetSymbolAddress returns for the current device is used.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up once per device.
int scratch_for_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return bgtq::set_error(BGTQ_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return bgtq::set_error(BGTQ_E_UNSUPPORTED, "device %d above %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return bgtq::set_error(BGTQ_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return BGTQ_OK;
}

}  // namespace

extern "C" int bgtq_decode_attention_noalloc(const bgtq_cache* c, int layer, const void* q, int dtype, float* out,
                                             int n_splits, void* stream) {
    void* ws = nullptr;
    if (int rc = scratch_for_current_device(&ws)) return rc;
    return bgtq::decode_capped(c, layer, q, dtype, out, ws, kScratchBytes, n_splits, stream);
}
