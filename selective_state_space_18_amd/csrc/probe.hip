// Issue-rate probes: kernels with a known per-lane instruction mix, timed by
// the caller to measure what the VALU and the transcendental unit of the
// device actually sustain.  They calibrate the arithmetic roofline the scan
// kernels are reported against; they compute nothing of the scan.
#include <hip/hip_runtime.h>

#include "ssm_launch.h"
#include "ssmscan.h"

namespace {

constexpr int kProbeBlock = 256;
constexpr int kChains = 16;  // independent dependency chains per lane

// Every iteration issues, per lane and in independent chains:
//   kFma : kChains * kFmaRep v_fma_f32 (v = v * a + b)
//   kExp : kChains v_exp_f32 (v = exp2(-|v|), the modifiers are free)
//   kF64 : kChains * 2 v_fma_f64
// `sentinel` is never matched in practice; the store keeps the chains live.
template <int kFmaRep, bool kExp, bool kF64>
__global__ __launch_bounds__(kProbeBlock) void probe_kernel(float *sink, int iters, float a, float b,
                                                            float sentinel) {
    const int tid = blockIdx.x * kProbeBlock + threadIdx.x;
    float v[kChains], w[kChains];
    double dv[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
        v[k] = 0.001f * (float)(threadIdx.x + k);
        w[k] = 0.5f + 0.01f * (float)k;
        dv[k] = (double)v[k];
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < kFmaRep; ++r) {
#pragma unroll
            for (int k = 0; k < kChains; ++k) v[k] = __builtin_fmaf(v[k], a, b);
        }
        if constexpr (kExp) {
#pragma unroll
            for (int k = 0; k < kChains; ++k) w[k] = __builtin_amdgcn_exp2f(-__builtin_fabsf(w[k]));
        }
        if constexpr (kF64) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
#pragma unroll
                for (int k = 0; k < kChains; ++k) dv[k] = __builtin_fma(dv[k], (double)a, (double)b);
            }
        }
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kChains; ++k) s += v[k] + w[k] + (float)dv[k];
    if (s == sentinel) sink[tid] = s;
}

}  // namespace

extern "C" int ssm_probe_issue(int kind, int64_t blocks, int64_t iters, float *sink, void *stream,
                               int64_t *valu_per_iter, int64_t *trans_per_iter) {
    if (blocks <= 0 || blocks > (int64_t(1) << 24) || iters <= 0 || iters > (int64_t(1) << 24))
        return ssm::set_error(SSM_ERR_BAD_DIM, "probe: blocks and iterations must be in [1, 2^24]");
    if (sink == nullptr) return ssm::set_error(SSM_ERR_NULLPTR, "probe: sink is NULL");
    if (kind < SSM_PROBE_FMA_F32 || kind > SSM_PROBE_FMA_F64)
        return ssm::set_error(SSM_ERR_BAD_OPTION, "probe: unknown kind");
    static const int64_t valu[] = {4 * kChains, kChains, 4 * kChains + kChains, 2 * kChains};
    static const int64_t trans[] = {0, kChains, kChains, 0};
    if (valu_per_iter) *valu_per_iter = valu[kind];
    if (trans_per_iter) *trans_per_iter = trans[kind];
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)blocks), block(kProbeBlock);
    const int it = (int)iters;
    const float a = 0.999f, b = 1e-3f, sentinel = -12345.0f;
    switch (kind) {
        case SSM_PROBE_FMA_F32:
            hipLaunchKernelGGL((probe_kernel<4, false, false>), grid, block, 0, s, sink, it, a, b, sentinel);
            break;
        case SSM_PROBE_EXP_F32:
            hipLaunchKernelGGL((probe_kernel<0, true, false>), grid, block, 0, s, sink, it, a, b, sentinel);
            break;
        case SSM_PROBE_FMA_EXP_F32:
            hipLaunchKernelGGL((probe_kernel<4, true, false>), grid, block, 0, s, sink, it, a, b, sentinel);
            break;
        case SSM_PROBE_FMA_F64:
            hipLaunchKernelGGL((probe_kernel<0, false, true>), grid, block, 0, s, sink, it, a, b, sentinel);
            break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return ssm::set_error(SSM_ERR_HIP, hipGetErrorString(e));
    return SSM_OK;
}
