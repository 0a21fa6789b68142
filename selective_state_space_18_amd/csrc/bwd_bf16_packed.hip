// Backward kernels for bf16 storage, packed variable-length sequences.
#include "bwd_kernels.h"

namespace ssm {

hipError_t bwd_pass_bf16_packed(BwdPass pass, const BwdParams &q, int N, hipStream_t s) {
    return bwd_pass<bf16, true>(pass, q, N, s);
}

}  // namespace ssm
