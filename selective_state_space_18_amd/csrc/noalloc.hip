// The scan entry point that allocates nothing: ssm_scan_fwd_ex's computation
// on scratch held in a file-scope device array instead of the library's
// per-stream buffer.  For callers that cannot allocate device memory.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "ssm_launch.h"
#include "ssmscan.h"

namespace {

// 64 MiB per GPU, resident from the library's load until the process ends.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;

// In host code `scratch` names the symbol only (a host-side stand-in, not a
// device address); kernels get the address hipGetSymbolAddress returns for the
// current device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_mu;
std::map<int, void *> g_ptr;  // device -> address of that device's copy of `scratch`

// Address of `scratch` on device `dev` (the current device), looked up on the
// first call on that device and kept.
int resolve(int dev, void **out) {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_ptr.find(dev);
    if (it != g_ptr.end()) {
        *out = it->second;
        return SSM_OK;
    }
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return ssm::set_error(SSM_ERR_HIP, "hipGetSymbolAddress(scratch) of the no-allocation entry point failed");
    }
    if (ptr == nullptr) return ssm::set_error(SSM_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_ptr[dev] = ptr;
    *out = ptr;
    return SSM_OK;
}

}  // namespace

extern "C" int ssm_scan_fwd_noalloc(const void *x, const void *delta, const float *A, const void *B, const void *C,
                                    const float *D, const float *h_init, void *y, float *h_final, int64_t Bsz,
                                    int64_t L, int64_t Dm, int64_t N, int dtype, void *stream) {
    return ssm::scan_fwd_fixed_scratch(x, delta, A, B, C, D, h_init, y, h_final, Bsz, L, Dm, N, dtype, stream,
                                       kNoAllocScratchBytes, resolve);
}
