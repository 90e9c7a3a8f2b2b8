// la_noalloc.hip -- la_fwd_causal_noalloc: the causal forward with its
// per-segment states in a device array the library owns, for callers that
// cannot allocate (code under graph capture, tight serving loops, harnesses
// that forbid allocation).
//
// The array is a file-scope __device__ object of LA_NOALLOC_SCRATCH_BYTES:
// every GPU the library runs on holds its own copy from code-object load until
// the process ends.  Host code never passes the array's name to a kernel (on
// the host it is only a stand-in for the symbol): the first call on a device
// looks up that device's address with hipGetSymbolAddress and keeps it, and
// the kernels receive that address as their workspace.  Nothing here
// allocates.  Every call on one GPU shares its array and leaves its contents
// behind; the forward writes every state it reads before reading it, so no
// clearing is needed.  Calls that overlap on one GPU (several streams, or
// several host threads) race on the array.
#include <hip/hip_runtime.h>

#include <atomic>

#include "la.h"
#include "la_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch`, per device ordinal (null until first looked up).
std::atomic<void *> g_scratch[la::kMaxDevices];

la_status scratch_address(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return LA_ERR_LAUNCH;
    if (dev < 0 || dev >= la::kMaxDevices) return LA_ERR_UNSUPPORTED;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return LA_ERR_LAUNCH;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return LA_OK;
}

}  // namespace

extern "C" la_status la_fwd_causal_noalloc(const void *q, const void *k, const void *v, void *o, float *den,
                                           int B, int H, int N, int d_k, int d_v, int C, la_dtype in,
                                           la_dtype out, hipStream_t stream) {
    la_status st = la::check_fwd_causal_args(q, k, v, o, den, nullptr, nullptr, nullptr, nullptr, B, H, N, d_k, d_v,
                                             C, in, out);
    if (st != LA_OK) return st;
    // The segment split is capped so that its states fit the array; with one
    // segment per (b, h) no state is stored, so every size fits.
    const long per_state = la::state_floats(d_k, d_v) * (long)sizeof(float);
    const long states = (long)(LA_NOALLOC_SCRATCH_BYTES / per_state);
    if (states < 1) return LA_ERR_WORKSPACE;
    void *ws = nullptr;
    if ((st = scratch_address(&ws)) != LA_OK) return st;
    la::FwdDesc d{q, k, v, o, den, nullptr, nullptr, nullptr, nullptr, B, H, N, d_k, d_v, C,
                  in == LA_BF16, out == LA_BF16, static_cast<float *>(ws), stream, nullptr, states};
    return la::run_fwd(d, true);
}
