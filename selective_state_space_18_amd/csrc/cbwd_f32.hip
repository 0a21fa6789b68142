// Backward of the complex-A scan for f32 storage.
#include "cbwd_kernels.h"

namespace ssm {

int cbwd_segment_len() { return kCbwdT; }
int cbwd_waves(int dtype) { return dtype == 0 ? CbwdShape<double>::kWaves : CbwdShape<float>::kWaves; }

hipError_t cbwd_pass_f32(BwdPass pass, const BwdParams &q, int N, hipStream_t s) {
    return cbwd_pass<float>(pass, q, N, s);
}

}  // namespace ssm
