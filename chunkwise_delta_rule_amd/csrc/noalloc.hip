// deltanet_fwd_noalloc: deltanet_fwd with its context-parallel workspace in a
// fixed device array of this library, for callers that cannot allocate
// device memory (code under stream capture, tight serving loops, harnesses
// that forbid allocation).
//
// The array `scratch` below is one per device; its device address is taken
// with hipGetSymbolAddress on the first call on each device (with that device
// current) and kept per device. Only that address is ever handed to the
// kernels: in host code the array's name is a host-side stand-in, not device
// memory. The workspace of the context-parallel path needs no clearing (every
// byte a launch reads was written earlier in the same call), so the array
// starts and stays uninitialised. Calls that overlap on one device share the
// array and race; calls on different devices do not.
#include "../../include/deltanet.h"
#include "dn_internal.h"

#include <mutex>

namespace {

constexpr size_t kScratchBytes = DN_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size must keep 256-byte alignment");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, or nullptr on a HIP error.
void *scratch_address() {
    static std::mutex mu;
    static void *addr[kMaxDevices] = {nullptr};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

} // namespace

extern "C" int deltanet_fwd_noalloc(const void *q, const void *k, const void *v, const void *beta, const float *S0,
                                    void *o, float *S_final, int B, int H, int T, int dk, int dv, int chunk, int dtype,
                                    int cp_groups, hipStream_t stream) {
    // 0 for a serial plan (no workspace) and for invalid shapes, which the
    // dense forward then rejects with its own status
    const size_t need = deltanet_workspace_bytes(B, H, T, dk, dv, chunk, cp_groups);
    if (need > kScratchBytes) return DN_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        ws = scratch_address();
        if (!ws) return DN_ERR_HIP;
    }
    return dn::fwd_dense(q, k, v, beta, nullptr, S0, o, S_final, B, H, T, 1, dk, dv, chunk, dtype, cp_groups, ws,
                         need > 0 ? kScratchBytes : 0, stream, false);
}
