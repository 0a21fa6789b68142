// Scalar-decay (state-space duality) layer for bf16 storage.
#include "ssd_kernels.h"

namespace ssm {

hipError_t ssd_pass_bf16(SsdPass pass, const SsdParams &p, int N, hipStream_t s) {
    return ssd_pass<bf16>(pass, p, N, s);
}

}  // namespace ssm
