// qubo_search_noalloc: the int32 whole-space search of qubo_search without any
// device allocation, for callers that cannot allocate (code under graph capture,
// tight serving loops, harnesses that forbid it).  The workspace (U, E_s, M_int,
// the Gray-ordered prefix energies, their per-body and per-group minima, the
// per-workgroup partials and the control block) lives in one static device array per GPU.
#include "host.h"

#include <mutex>

using namespace qubo_host;

// One copy per GPU, held until the process ends.  In host code `scratch` is a
// host-side stand-in for the symbol, never a device address: the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[QUBO_NOALLOC_BYTES];

namespace {

constexpr uint64_t kScratchBytes = (uint64_t)QUBO_NOALLOC_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

// The current device's copy of the array (looked up on its first use there).
int scratch_ptr(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return QUBO_EDEVICE;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return QUBO_EDEVICE;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return QUBO_OK;
}

}  // namespace

extern "C" {

QUBO_API int qubo_search_noalloc(const int32_t *Q, int n, int prefix_bits, int cache_bits, void *stream,
                                 qubo_result *out)
{
    if (!Q || !out || n < 1 || n > QUBO_MAX_N)
        return QUBO_EINVAL;
    DeviceInfo dev;
    int rc = device_info(&dev);
    if (rc != QUBO_OK)
        return rc;
    void *ws = nullptr;
    rc = scratch_ptr(&ws);
    if (rc != QUBO_OK)
        return rc;
    Request rq;
    rq.Q = Q;
    rq.n = n;
    rq.prefix_bits = prefix_bits;
    rq.cache_bits = cache_bits;
    rq.stream = static_cast<hipStream_t>(stream);
    rq.scratch = ws;
    rq.scratch_bytes = kScratchBytes;
    return run(rq, out);
}

}  // extern "C"
