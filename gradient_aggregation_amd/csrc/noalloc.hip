// The workspace of ga_chunk_norm_topk_static in a fixed device array, for
// callers that cannot allocate device memory.
//
// `scratch` holds the [W][n_c] binary64 keys that ga_chunk_norm_topk takes as
// a caller buffer and, for chunks longer than 2048 elements, right after them
// the [W][n_c][parts] partial sums that ga_chunk_norm_topk keeps in the plan's
// workspace.  Each device the library runs on holds one until the process
// ends.  In host code the array's name is not
// a device address: its address on a device is looked up once, with that
// device current, at plan creation, and only that looked-up pointer is ever
// passed to a kernel.
#include <mutex>

#include "plan.h"

namespace ga {

namespace {

static __device__ __align__(256) double scratch[GA_STATIC_KEYS];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
double* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_keys_setup(int device) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[device]) return hipSuccess;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
        (void)hipGetLastError();   // not to be reported by the next launch check
        return e;
    }
    g_ptr[device] = static_cast<double*>(p);
    return hipSuccess;
}

double* static_keys(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    return g_ptr[device];
}

}  // namespace ga
