// Recurrent decode step on a resident state, in place, for gfx950.
//
// One token per call ("Mamba SSM Nedir?" page, sections "Ayrik Zamana Gecis"
// and "Karmasiklik Karsilastirmasi": inference updates a fixed-size state):
//   h[n] <- exp(delta A[n]) h[n] + (exp(delta A[n]) - 1)/A[n] B[n] x
//   y     = sum_n C[n] h[n] + D x
// (the input coefficient takes its limit delta B[n] at A[n] = 0).
//
// The step reads and writes the whole fp32 state once, so it is bound by HBM
// bandwidth.  Q = N/4 lanes share one (b, d) channel and each owns 4
// consecutive states (16 bytes), so one wave-wide 16-byte load or store moves
// 1 KiB of contiguous state.  The partial sums of y are combined across the Q
// lanes with cross-lane shuffles.
#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {

namespace {

constexpr int kBlock = 256;

template <int N>
struct StepShape {
    static constexpr int Q = (N >= 4) ? N / 4 : 1;  // lanes per channel
    static constexpr int SPL = N / Q;               // states per lane
};

// kVec: h and A rows are read/written as 16-byte vectors (needs 16-byte
// aligned base pointers, checked on the host).
template <typename T, int N, bool kPrecise, bool kVec>
__global__ __launch_bounds__(kBlock) void step_kernel(StepParams p) {
    constexpr int Q = StepShape<N>::Q;
    constexpr int SPL = StepShape<N>::SPL;
    const int64_t BD = p.Bsz * p.Dm;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t ch = i / Q;
    const int j = (int)(i - ch * Q);
    // Q divides the wave size, so the Q lanes of a channel leave together.
    if (ch >= BD) return;
    const int64_t b = ch / p.Dm;
    const int64_t d = ch - b * p.Dm;

    const float xv = to_f32(static_cast<const T *>(p.x)[ch]);
    const float dv = to_f32(static_cast<const T *>(p.delta)[ch]);
    const T *Bp = static_cast<const T *>(p.B) + b * N + j * SPL;
    const T *Cp = static_cast<const T *>(p.C) + b * N + j * SPL;
    const float *Ap = p.A + d * N + j * SPL;
    float *hp = p.h + ch * N + j * SPL;

    float h[SPL], a[SPL];
    if constexpr (kVec && SPL == 4) {
        const float4 hv = *reinterpret_cast<const float4 *>(hp);
        h[0] = hv.x; h[1] = hv.y; h[2] = hv.z; h[3] = hv.w;
        const float4 av = *reinterpret_cast<const float4 *>(Ap);
        a[0] = av.x; a[1] = av.y; a[2] = av.z; a[3] = av.w;
    } else {
#pragma unroll
        for (int k = 0; k < SPL; ++k) {
            h[k] = hp[k];
            a[k] = Ap[k];
        }
    }

    float yv = 0.f;
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
        float abar;
        const float E = kPrecise ? expm1_and_exp_precise(dv * a[k], abar) : expm1_and_exp(dv * a[k], abar);
        float coef;
        if constexpr (kPrecise)
            coef = (a[k] != 0.f) ? E / a[k] : dv;
        else
            coef = (a[k] != 0.f) ? E * __builtin_amdgcn_rcpf(a[k]) : dv;
        const float bx = to_f32(Bp[k]) * xv;
        h[k] = __builtin_fmaf(abar, h[k], coef * bx);
        yv = __builtin_fmaf(to_f32(Cp[k]), h[k], yv);
    }

    if constexpr (kVec && SPL == 4) {
        *reinterpret_cast<float4 *>(hp) = make_float4(h[0], h[1], h[2], h[3]);
    } else {
#pragma unroll
        for (int k = 0; k < SPL; ++k) hp[k] = h[k];
    }
#pragma unroll
    for (int off = 1; off < Q; off <<= 1) yv += __shfl_xor(yv, off, Q);
    if (j == 0) static_cast<T *>(p.y)[ch] = from_acc<T>(__builtin_fmaf(p.D[d], xv, yv));
}

template <typename T, bool kPrecise, int N>
hipError_t launch_n(const StepParams &p, hipStream_t s) {
    const int64_t threads = p.Bsz * p.Dm * StepShape<N>::Q;
    if (threads == 0) return hipSuccess;
    const unsigned grid = (unsigned)((threads + kBlock - 1) / kBlock);
    const bool vec = ((reinterpret_cast<uintptr_t>(p.h) | reinterpret_cast<uintptr_t>(p.A)) & 15) == 0;
    if (vec)
        hipLaunchKernelGGL((step_kernel<T, N, kPrecise, true>), dim3(grid), dim3(kBlock), 0, s, p);
    else
        hipLaunchKernelGGL((step_kernel<T, N, kPrecise, false>), dim3(grid), dim3(kBlock), 0, s, p);
    return hipGetLastError();
}

template <typename T, bool kPrecise>
hipError_t launch_t(const StepParams &p, int N, hipStream_t s) {
    switch (N) {
        case 1: return launch_n<T, kPrecise, 1>(p, s);
        case 2: return launch_n<T, kPrecise, 2>(p, s);
        case 4: return launch_n<T, kPrecise, 4>(p, s);
        case 8: return launch_n<T, kPrecise, 8>(p, s);
        case 16: return launch_n<T, kPrecise, 16>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_step(const StepParams &p, int N, int dtype, hipStream_t s) {
    if (dtype == 0) return launch_t<float, true>(p, N, s);
    if (dtype == 1) return launch_t<bf16, false>(p, N, s);
    return hipErrorInvalidValue;
}

}  // namespace ssm
