// Scan kernels for bf16 storage (fp32 arithmetic), a dense batch.
#include "scan_kernels.h"

namespace ssm {

hipError_t scan_pass_bf16(ScanPass pass, const ScanParams &p, int N, hipStream_t s) {
    return scan_pass<bf16, false>(pass, p, N, s);
}

}  // namespace ssm
