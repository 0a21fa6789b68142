// Complex-A scan and decode step for bf16 storage.
#include "cplx_kernels.h"

namespace ssm {

hipError_t cplx_pass_bf16(ScanPass pass, const ScanParams &p, int N, hipStream_t s) {
    return cplx_pass<bf16>(pass, p, N, s);
}

hipError_t cplx_step_bf16(const StepParams &p, int N, hipStream_t s) { return cplx_step_launch<bf16, false>(p, N, s); }

}  // namespace ssm
