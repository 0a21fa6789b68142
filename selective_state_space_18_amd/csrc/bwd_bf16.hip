// Backward kernels for bf16 storage.
#include "bwd_kernels.h"

namespace ssm {

hipError_t bwd_pass_bf16(BwdPass pass, const BwdParams &q, int N, hipStream_t s) {
    return bwd_pass<bf16, false>(pass, q, N, s);
}

}  // namespace ssm
