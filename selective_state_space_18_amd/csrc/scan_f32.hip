// Scan kernels for fp32 storage (fp64 arithmetic), a dense batch.
#include "scan_kernels.h"

namespace ssm {

hipError_t scan_pass_f32(ScanPass pass, const ScanParams &p, int N, hipStream_t s) {
    return scan_pass<float, false>(pass, p, N, s);
}

}  // namespace ssm
