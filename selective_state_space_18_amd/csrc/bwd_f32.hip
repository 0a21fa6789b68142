// Backward kernels for f32 storage.
#include "bwd_kernels.h"

namespace ssm {

hipError_t bwd_pass_f32(BwdPass pass, const BwdParams &q, int N, hipStream_t s) {
    return bwd_pass<float, false>(pass, q, N, s);
}

}  // namespace ssm
