// Backward of the complex-A scan for f32 storage.
#include "cbwd_kernels.h"

namespace ssm {

int cbwd_segment_len() { return kCbwdT; }
int cbwd_tiles_per_block(int dtype, int N) {
    const int w = dtype == 0 ? CbwdShape<double>::kWaves : CbwdShape<float>::kWaves;
    return N >= 2 ? w / cbwd_split<2>() : w / cbwd_split<1>();
}
int cbwd_blocks_per_cu(int dtype) {
    return dtype == 0 ? CbwdShape<double>::kBlocksPerCU : CbwdShape<float>::kBlocksPerCU;
}

hipError_t cbwd_pass_f32(BwdPass pass, const BwdParams &q, int N, hipStream_t s) {
    return cbwd_pass<float>(pass, q, N, s);
}

}  // namespace ssm
