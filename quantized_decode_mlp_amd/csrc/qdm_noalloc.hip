// The decode MLP for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// qdm_mlp_decode with its workspace -- the fp32 hidden rows and the split-K
// partial sums -- in a fixed device array of this file instead of a caller's
// buffer.
//
// The array is a file-scope __device__ variable, so every GPU the library's
// code object is loaded on holds its own copy until the process ends.  Its
// host-side name is not a device address: the address of each device's copy
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is handed to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qdm.h"
#include "qdm_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[QDM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, set on first use

// The current device's copy of the array (looked up on the first call made
// with that device current).
int device_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QDM_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QDM_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return QDM_OK;
}

}  // namespace

extern "C" int qdm_mlp_decode_noalloc(const void* x, const void* r, int32_t m, qdm_dtype act,
                                      const qdm_weight* gate_up, const qdm_weight* down, void* out, void* stream) {
    // invalid arguments: the ordinary entry point's checks name them (nothing runs)
    const size_t need = qdm_mlp_workspace_bytes(m, act, gate_up, down);
    if (need == 0 || !x || !r || !out) return qdm_mlp_decode(x, r, m, act, gate_up, down, nullptr, 0, out, stream);
    if (need > QDM_NOALLOC_SCRATCH_BYTES) return QDM_ERR_TOO_LARGE;
    void* ws = nullptr;
    if (int e = device_scratch(&ws)) return e;
    // the kernels write h and the partials before reading them: nothing needs clearing
    return qdm_mlp_decode(x, r, m, act, gate_up, down, ws, QDM_NOALLOC_SCRATCH_BYTES, out, stream);
}
