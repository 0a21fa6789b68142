// Scan kernels for bf16 storage (fp32 arithmetic), packed variable-length sequences.
#include "scan_kernels.h"

namespace ssm {

hipError_t scan_pass_bf16_packed(ScanPass pass, const ScanParams &p, int N, hipStream_t s) {
    return scan_pass<bf16, true>(pass, p, N, s);
}

}  // namespace ssm
