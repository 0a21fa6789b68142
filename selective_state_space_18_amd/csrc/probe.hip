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

// One instruction form per probe, 16 independent chains, kRep x 16 per iteration:
//   kOp 0: v_fmac_f32 (VOP2: v += w * u, all VGPRs)
//   kOp 1: v_mul_f32  (VOP2: v = v * w)
//   kOp 2: v_add_f32  (VOP2: v = v + w)
//   kOp 3: v_fma_f32 with two VGPR sources and the VGPR addend (VOP3: v = v * w + u)
template <int kOp>
__global__ __launch_bounds__(kProbeBlock) void form_kernel(float *sink, int iters, float a, float b, float sentinel) {
    const int tid = blockIdx.x * kProbeBlock + threadIdx.x;
    float v[kChains];
    float w = a + 1e-7f * (float)threadIdx.x, u = b;
#pragma unroll
    for (int k = 0; k < kChains; ++k) v[k] = 0.001f * (float)(threadIdx.x + k);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int k = 0; k < kChains; ++k) {
                if constexpr (kOp == 0) v[k] = __builtin_fmaf(w, u, v[k]);
                else if constexpr (kOp == 1) v[k] = v[k] * w;
                else if constexpr (kOp == 2) v[k] = v[k] + w;
                else v[k] = __builtin_fmaf(v[k], w, u);
            }
        }
        __asm__ volatile("" : "+v"(w), "+v"(u));  // keep w, u in VGPRs, opaque per iteration
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kChains; ++k) s += v[k];
    if (s == sentinel) sink[tid] = s;
}

// The arithmetic of one structured-A output step for N = 16 states, with no
// memory traffic: per step an exp, the E chain, and per state element the
// input, update and output FMAs, the B/C row entering as wave-uniform scalar
// operands (kernel arguments) as in the scan.  x and delta follow cheap
// per-lane recurrences, so nothing is loop-invariant.  One iteration is one
// wave-step of the scan's output pass without its loads and stores.
constexpr int kMixN = 16;
struct MixRow {
    float v[2 * kMixN];
};

__global__ __launch_bounds__(kProbeBlock) void step_mix_kernel(float *sink, int iters, MixRow row, float sentinel) {
    const int tid = blockIdx.x * kProbeBlock + threadIdx.x;
    float g[kMixN];
#pragma unroll
    for (int n = 0; n < kMixN; ++n) g[n] = 0.01f * (float)(threadIdx.x & 7) + 0.001f * (float)n;
    const float a0 = -0.5f - 1e-4f * (float)(threadIdx.x & 15), inva = 1.0f / a0;
    float xv = 0.3f + 1e-3f * (float)(threadIdx.x & 31), dv = 0.01f + 1e-5f * (float)(threadIdx.x & 63);
    float ysum = 0.f;
    for (int i = 0; i < iters; ++i) {
        const float r = __builtin_amdgcn_exp2f(dv * a0);
        const float E1 = r - 1.0f;
        const float xa = xv * inva;
        float E = E1, y = 0.f;
#pragma unroll
        for (int n = 0; n < kMixN; ++n) {
            const float tt = __builtin_fmaf(row.v[n], xa, g[n]);
            g[n] = __builtin_fmaf(E, tt, g[n]);
            y = __builtin_fmaf(row.v[kMixN + n], g[n], y);
            if (n + 1 < kMixN) E = __builtin_fmaf(E, r, E1);
        }
        ysum += y;
        xv = __builtin_fmaf(xv, 0.999f, 1e-4f);
        dv = __builtin_fmaf(dv, 1.0001f, 1e-7f);
    }
    float s = ysum;
#pragma unroll
    for (int n = 0; n < kMixN; ++n) s += g[n];
    if (s == sentinel) sink[tid] = s;
}

__global__ __launch_bounds__(kProbeBlock) void empty_kernel() {}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kNt = 2;  // buffer cache-policy bit: nontemporal

// Streaming probes over `words` 16-byte words, grid-stride, every access a
// range-checked buffer access (a chunk is below 1 GiB, so offsets fit 32 bits).
//   kMode 0 (read) : sum the words; the sum is stored only if it matches the sentinel
//   kMode 1 (rmw)  : add 1 to every 32-bit value in place
//   kMode 2 (write): store a constant
template <int kMode>
__global__ __launch_bounds__(kProbeBlock) void stream_kernel(unsigned *buf, int32_t words, unsigned sentinel) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(buf, (short)0, words * 16, 0x00020000);
    const int32_t stride = (int32_t)(gridDim.x * kProbeBlock);
    unsigned acc = 0;
    for (int32_t w = (int32_t)(blockIdx.x * kProbeBlock + threadIdx.x); w < words; w += stride) {
        if constexpr (kMode == 2) {
            const u32x4 v = {(unsigned)w, 1u, 2u, 3u};
            __builtin_amdgcn_raw_buffer_store_b128(v, r, w * 16, 0, kNt);
        } else {
            u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, w * 16, 0, kNt);
            if constexpr (kMode == 0) {
                acc += v.x ^ v.y ^ v.z ^ v.w;
            } else {
                v += 1u;
                __builtin_amdgcn_raw_buffer_store_b128(v, r, w * 16, 0, kNt);
            }
        }
    }
    if constexpr (kMode == 0)
        if (acc == sentinel) __builtin_amdgcn_raw_buffer_store_b32(acc, r, 0, 0, 0);
}

}  // namespace

extern "C" int ssm_probe_hbm(int kind, void *buf, int64_t bytes, void *stream) {
    if (kind < SSM_PROBE_HBM_READ || kind > SSM_PROBE_HBM_WRITE)
        return ssm::set_error(SSM_ERR_BAD_OPTION, "probe: unknown memory probe kind");
    if (buf == nullptr) return ssm::set_error(SSM_ERR_NULLPTR, "probe: buf is NULL");
    if (bytes < 16 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
        return ssm::set_error(SSM_ERR_ALIGN, "probe: buf must be 16-byte aligned and bytes a positive multiple of 16");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // chunks below 1 GiB, each its own launch of 256 x 8 blocks (8 per CU)
    const int64_t chunk = int64_t(1) << 29;
    for (int64_t off = 0; off < bytes; off += chunk) {
        const int64_t n = bytes - off < chunk ? bytes - off : chunk;
        unsigned *p = reinterpret_cast<unsigned *>(static_cast<char *>(buf) + off);
        const int32_t words = (int32_t)(n / 16);
        const dim3 grid(2048), block(kProbeBlock);
        switch (kind) {
            case SSM_PROBE_HBM_READ: hipLaunchKernelGGL((stream_kernel<0>), grid, block, 0, s, p, words, 0x9e3779b9u); break;
            case SSM_PROBE_HBM_RMW: hipLaunchKernelGGL((stream_kernel<1>), grid, block, 0, s, p, words, 0u); break;
            case SSM_PROBE_HBM_WRITE: hipLaunchKernelGGL((stream_kernel<2>), grid, block, 0, s, p, words, 0u); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return ssm::set_error(SSM_ERR_HIP, hipGetErrorString(e));
    }
    return SSM_OK;
}

extern "C" int ssm_probe_issue(int kind, int64_t blocks, int64_t iters, float *sink, void *stream,
                               int64_t *valu_per_iter, int64_t *trans_per_iter) {
    if (blocks <= 0 || blocks > (int64_t(1) << 24) || iters <= 0 || iters > (int64_t(1) << 24))
        return ssm::set_error(SSM_ERR_BAD_DIM, "probe: blocks and iterations must be in [1, 2^24]");
    if (sink == nullptr) return ssm::set_error(SSM_ERR_NULLPTR, "probe: sink is NULL");
    if (kind < SSM_PROBE_FMA_F32 || kind > SSM_PROBE_SCAN_STEP_MIX)
        return ssm::set_error(SSM_ERR_BAD_OPTION, "probe: unknown kind");
    // VALU instructions per iteration counted from the source (the step mix:
    // its 63 FMAs and the exp; the compiled loop adds a few more)
    static const int64_t valu[] = {4 * kChains, kChains, 4 * kChains + kChains, 2 * kChains, 0,
                                   4 * kChains, 4 * kChains, 4 * kChains, 4 * kChains, 4 * kMixN};
    static const int64_t trans[] = {0, kChains, kChains, 0, 0, 0, 0, 0, 0, 1};
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
        case SSM_PROBE_EMPTY:
            hipLaunchKernelGGL(empty_kernel, grid, block, 0, s);
            break;
        case SSM_PROBE_FMAC_F32:
            hipLaunchKernelGGL((form_kernel<0>), grid, block, 0, s, sink, it, a, b, sentinel);
            break;
        case SSM_PROBE_MUL_F32:
            hipLaunchKernelGGL((form_kernel<1>), grid, block, 0, s, sink, it, a, b, sentinel);
            break;
        case SSM_PROBE_ADD_F32:
            hipLaunchKernelGGL((form_kernel<2>), grid, block, 0, s, sink, it, a, b, sentinel);
            break;
        case SSM_PROBE_FMA_F32_VGPR:
            hipLaunchKernelGGL((form_kernel<3>), grid, block, 0, s, sink, it, a, b, sentinel);
            break;
        case SSM_PROBE_SCAN_STEP_MIX: {
            MixRow row;
            for (int k = 0; k < 2 * kMixN; ++k) row.v[k] = 0.1f + 0.01f * (float)k;
            hipLaunchKernelGGL(step_mix_kernel, grid, block, 0, s, sink, it, row, sentinel);
            break;
        }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return ssm::set_error(SSM_ERR_HIP, hipGetErrorString(e));
    return SSM_OK;
}
