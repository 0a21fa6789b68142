// Complex-A scan and decode step for f32 storage.
#include "cplx_kernels.h"

namespace ssm {

hipError_t cplx_pass_f32(ScanPass pass, const ScanParams &p, int N, hipStream_t s) {
    return cplx_pass<float>(pass, p, N, s);
}

hipError_t cplx_step_f32(const StepParams &p, int N, hipStream_t s) { return cplx_step_launch<float, true>(p, N, s); }

}  // namespace ssm
