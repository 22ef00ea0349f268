// The split workspace of qsdpa_decode_static (include/qkv.h): a file-scope
// device array, one copy per GPU that loads the library, held until the
// process ends, so that the call allocates nothing.  Host code never passes
// the array's name to a kernel or a copy (on the host it only stands for the
// symbol): it asks HIP for the array's device address once per device, with
// that device current, and hands that address to the kernels.
#include <mutex>

#include "../../include/qkv.h"
#include "qkv_internal.hpp"
#include "qkv_merge.hpp"

namespace qkv {

namespace {

static __device__ __align__(256) uint8_t scratch[QKV_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices];      // device address of 'scratch' per device (null until resolved)
bool g_cleared[kMaxDevices];    // its ticket header has been zeroed

}  // namespace

hipError_t static_scratch(hipStream_t stream, void** addr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    hipDevice_t sdev = cur;
    if (stream) {
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return e;
    }
    if (sdev != cur || cur < 0 || cur >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_addr[cur]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_addr[cur] = p;
    }
    if (!g_cleared[cur]) {
        // the tickets must start at zero; every completed call leaves them so
        e = launch_fill_zero(g_addr[cur], kTicketBytes, stream);
        if (e != hipSuccess) return e;
        g_cleared[cur] = true;
    }
    *addr = g_addr[cur];
    return hipSuccess;
}

}  // namespace qkv
