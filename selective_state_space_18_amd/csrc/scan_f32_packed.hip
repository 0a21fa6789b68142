// Scan kernels for fp32 storage (fp64 arithmetic), packed variable-length sequences.
#include "scan_kernels.h"

namespace ssm {

hipError_t scan_pass_f32_packed(ScanPass pass, const ScanParams &p, int N, hipStream_t s) {
    return scan_pass<float, true>(pass, p, N, s);
}

}  // namespace ssm
