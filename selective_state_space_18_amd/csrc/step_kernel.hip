// Recurrent decode step on a resident state, in place, for gfx950.
//
// One token per call ("Mamba SSM Nedir?" page, sections "Ayrik Zamana Gecis"
// and "Karmasiklik Karsilastirmasi": inference updates a fixed-size state):
//   h[n] <- exp(delta A[n]) h[n] + (exp(delta A[n]) - 1)/A[n] B[n] x
//   y     = sum_n C[n] h[n] + D x
// (the input coefficient takes its limit delta B[n] at A[n] = 0).  The
// options of the scan apply here too: delta = softplus(delta_in + bias[d])
// (or delta_in + bias[d]) and the Euler input term delta B[n] x.
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
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int N>
struct StepShape {
    static constexpr int Q = (N >= 4) ? N / 4 : 1;  // lanes per channel
    static constexpr int SPL = N / Q;               // states per lane
};

// kVec: h and A rows are read/written as 16-byte vectors (needs 16-byte
// aligned base pointers, checked on the host).
// kU: channels per thread.  A thread owns lane j of kU channels spaced one
// grid-width apart, so every wave-wide access stays contiguous, and it issues
// all kU state loads before using any of them: kU x 16 bytes in flight per
// lane hides HBM latency at a modest occupancy.
template <typename T, int N, bool kPrecise, bool kVec, int kU>
__global__ __launch_bounds__(kBlock) void step_kernel(StepParams p, int64_t chan_stride) {
    constexpr int Q = StepShape<N>::Q;
    constexpr int SPL = StepShape<N>::SPL;
    const int64_t BD = p.Bsz * p.Dm;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t ch0 = i / Q;
    const int j = (int)(i - ch0 * Q);
    // Q divides the wave size, so the Q lanes of a channel leave together.
    if (ch0 >= BD) return;

    float h[kU][SPL], a[kU][SPL], xv[kU], dv[kU];
    int64_t chs[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int64_t ch = ch0 + u * chan_stride;
        chs[u] = ch < BD ? ch : ch0;  // channels past the end redo ch0 and store nothing
        const int64_t d = chs[u] % p.Dm;
        float *hp = p.h + chs[u] * N + j * SPL;
        const float *Ap = p.A + d * N + j * SPL;
        if constexpr (kVec && SPL == 4) {
            const f32x4 hv = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(hp));
            h[u][0] = hv.x; h[u][1] = hv.y; h[u][2] = hv.z; h[u][3] = hv.w;
            const float4 av = *reinterpret_cast<const float4 *>(Ap);
            a[u][0] = av.x; a[u][1] = av.y; a[u][2] = av.z; a[u][3] = av.w;
        } else {
#pragma unroll
            for (int k = 0; k < SPL; ++k) {
                h[u][k] = hp[k];
                a[u][k] = Ap[k];
            }
        }
        xv[u] = to_f32(static_cast<const T *>(p.x)[chs[u]]);
        dv[u] = to_f32(static_cast<const T *>(p.delta)[chs[u]]);
    }

#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int64_t ch = chs[u];
        const int64_t b = ch / p.Dm;
        const int64_t d = ch - b * p.Dm;
        const T *Bp = static_cast<const T *>(p.B) + b * N + j * SPL;
        const T *Cp = static_cast<const T *>(p.C) + b * N + j * SPL;
        if (p.delta_bias != nullptr || p.delta_softplus) {  // uniform over the launch
            const float v = dv[u] + (p.delta_bias != nullptr ? p.delta_bias[d] : 0.f);
            dv[u] = p.delta_softplus ? (kPrecise ? softplus_precise(v) : softplus_(v)) : v;
        }
        float yv = 0.f;
#pragma unroll
        for (int k = 0; k < SPL; ++k) {
            float abar;
            const float E = kPrecise ? expm1_and_exp_precise(dv[u] * a[u][k], abar)
                                     : expm1_and_exp(dv[u] * a[u][k], abar);
            float coef;
            if (p.euler_b)
                coef = dv[u];
            else if constexpr (kPrecise)
                coef = (a[u][k] != 0.f) ? E / a[u][k] : dv[u];
            else
                coef = (a[u][k] != 0.f) ? E * __builtin_amdgcn_rcpf(a[u][k]) : dv[u];
            const float bx = to_f32(Bp[k]) * xv[u];
            h[u][k] = __builtin_fmaf(abar, h[u][k], coef * bx);
            yv = __builtin_fmaf(to_f32(Cp[k]), h[u][k], yv);
        }
        const bool live = ch0 + u * chan_stride < BD;
        float *hp = p.h + ch * N + j * SPL;
        if (live) {
            if constexpr (kVec && SPL == 4) {
                const f32x4 hv = {h[u][0], h[u][1], h[u][2], h[u][3]};
                __builtin_nontemporal_store(hv, reinterpret_cast<f32x4 *>(hp));
            } else {
#pragma unroll
                for (int k = 0; k < SPL; ++k) hp[k] = h[u][k];
            }
        }
#pragma unroll
        for (int off = 1; off < Q; off <<= 1) yv += __shfl_xor(yv, off, Q);
        if (live && j == 0) static_cast<T *>(p.y)[ch] = from_acc<T>(__builtin_fmaf(p.D[d], xv[u], yv));
    }
}

int g_step_unroll = 1;  // channels per thread (1, 2 or 4)

template <typename T, bool kPrecise, int N, bool kVec, int kU>
hipError_t launch_u(const StepParams &p, hipStream_t s) {
    const int64_t BD = p.Bsz * p.Dm;
    const int64_t chan_stride = (BD + kU - 1) / kU;  // channels per "row" of the grid
    const int64_t threads = chan_stride * StepShape<N>::Q;
    const unsigned grid = (unsigned)((threads + kBlock - 1) / kBlock);
    hipLaunchKernelGGL((step_kernel<T, N, kPrecise, kVec, kU>), dim3(grid), dim3(kBlock), 0, s, p, chan_stride);
    return hipGetLastError();
}

template <typename T, bool kPrecise, int N>
hipError_t launch_n(const StepParams &p, hipStream_t s) {
    if (p.Bsz * p.Dm == 0) return hipSuccess;
    const bool vec = ((reinterpret_cast<uintptr_t>(p.h) | reinterpret_cast<uintptr_t>(p.A)) & 15) == 0;
    const int u = g_step_unroll;
    if (vec) {
        if (u >= 4) return launch_u<T, kPrecise, N, true, 4>(p, s);
        if (u == 2) return launch_u<T, kPrecise, N, true, 2>(p, s);
        return launch_u<T, kPrecise, N, true, 1>(p, s);
    }
    return launch_u<T, kPrecise, N, false, 1>(p, s);
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

void set_step_unroll(int u) { g_step_unroll = u; }

hipError_t launch_step(const StepParams &p, int N, int dtype, hipStream_t s) {
    if (dtype == 0) return launch_t<float, true>(p, N, s);
    if (dtype == 1) return launch_t<bf16, false>(p, N, s);
    return hipErrorInvalidValue;
}

}  // namespace ssm
