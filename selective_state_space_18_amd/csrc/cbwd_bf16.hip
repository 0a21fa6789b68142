// Backward of the complex-A scan for bf16 storage.
#include "cbwd_kernels.h"

namespace ssm {

hipError_t cbwd_pass_bf16(BwdPass pass, const BwdParams &q, int N, hipStream_t s) {
    return cbwd_pass<bf16>(pass, q, N, s);
}

}  // namespace ssm
