// Backward kernels for f32 storage, packed variable-length sequences.
#include "bwd_kernels.h"

namespace ssm {

hipError_t bwd_pass_f32_packed(BwdPass pass, const BwdParams &q, int N, hipStream_t s) {
    return bwd_pass<float, true>(pass, q, N, s);
}

}  // namespace ssm
