// Scan launchers by storage dtype, and the small kernels that set the final
// state of empty sequences.
#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {

namespace {

constexpr int kBlock = 256;

hipError_t by_dtype(ScanPass pass, const ScanParams &p, int N, int dtype, hipStream_t s) {
    const bool packed = p.cu != nullptr;
    if (dtype == 0) return packed ? scan_pass_f32_packed(pass, p, N, s) : scan_pass_f32(pass, p, N, s);
    if (dtype == 1) return packed ? scan_pass_bf16_packed(pass, p, N, s) : scan_pass_bf16(pass, p, N, s);
    return hipErrorInvalidValue;
}

// h_final of empty sequences in a packed variable-length call: their
// initial state.  One thread per (sequence, d, n).
__global__ __launch_bounds__(kBlock) void varlen_empty_kernel(const int64_t *__restrict__ cu, int64_t nseq,
                                                              const float *__restrict__ h_init,
                                                              float *__restrict__ h_final, int64_t dn) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= nseq * dn) return;
    const int64_t k = i / dn;
    if (cu[k] != cu[k + 1]) return;
    h_final[i] = h_init ? h_init[i] : 0.f;
}

// h_final for an empty sequence: the initial state.
__global__ __launch_bounds__(kBlock) void state_init_kernel(const float *__restrict__ h_init,
                                                            float *__restrict__ h_final, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < count) h_final[i] = h_init ? h_init[i] : 0.f;
}

__global__ __launch_bounds__(kBlock) void fill_kernel(float *__restrict__ dst, int64_t count, float v) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < count) dst[i] = v;
}

}  // namespace

hipError_t launch_fill(float *dst, int64_t count, float v, hipStream_t s) {
    if (count == 0 || dst == nullptr) return hipSuccess;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((count + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, dst, count, v);
    return hipGetLastError();
}

size_t scan_acc_bytes(int dtype) { return dtype == 0 ? sizeof(double) : sizeof(float); }

// Must match BwdShape<Acc>::kT in bwd_kernels.h.
int bwd_segment_len(int dtype) { return dtype == 0 ? 16 : 32; }

hipError_t launch_bc_prep(const ScanParams &p, int N, int dtype, hipStream_t s) {
    return by_dtype(ScanPass::kPrep, p, N, dtype, s);
}

hipError_t launch_scan_aggregate(const ScanParams &p, int N, int dtype, hipStream_t s) {
    return by_dtype(ScanPass::kAggregate, p, N, dtype, s);
}

hipError_t launch_scan_carry(const ScanParams &p, int N, int dtype, hipStream_t s) {
    return by_dtype(ScanPass::kCarry, p, N, dtype, s);
}

hipError_t launch_scan_output(const ScanParams &p, int N, int dtype, hipStream_t s) {
    return by_dtype(ScanPass::kOutput, p, N, dtype, s);
}

hipError_t launch_varlen_empty(const ScanParams &p, int N, hipStream_t s) {
    const int64_t dn = p.Dm * N;
    const int64_t count = p.nseq * dn;
    if (count == 0 || p.h_final == nullptr || p.cu == nullptr) return hipSuccess;
    const unsigned grid = (unsigned)((count + kBlock - 1) / kBlock);
    hipLaunchKernelGGL(varlen_empty_kernel, dim3(grid), dim3(kBlock), 0, s, p.cu, p.nseq, p.h_init, p.h_final, dn);
    return hipGetLastError();
}

hipError_t launch_state_init(const ScanParams &p, int N, hipStream_t s) {
    const int64_t count = p.Bsz * p.Dm * N;
    if (count == 0 || p.h_final == nullptr) return hipSuccess;
    const unsigned grid = (unsigned)((count + kBlock - 1) / kBlock);
    hipLaunchKernelGGL(state_init_kernel, dim3(grid), dim3(kBlock), 0, s, p.h_init, p.h_final, count);
    return hipGetLastError();
}

}  // namespace ssm
