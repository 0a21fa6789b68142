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
// Grid: x runs over (channel d, lane j) of one batch row -- d = i / Q and
// j = i % Q with Q a power of two, no division -- and y over groups of kU
// batch rows.  The grid is kept to a few blocks per compute unit and each
// thread walks the row groups y, y + gridDim.y, ... with the next group's
// loads issued before the current group is computed: the state stream keeps
// loads in flight instead of paying a block launch and a full memory latency
// per row group.  A thread handles lane j of channel d; A's row, the bias and
// D are loaded once.  The state moves with non-temporal loads and stores: it
// is streamed once per step and should not displace the rows every channel
// shares.
template <typename T, int N, bool kPrecise, bool kVec, int kU>
__global__ __launch_bounds__(kBlock) void step_kernel(StepParams p) {
    constexpr int Q = StepShape<N>::Q;
    constexpr int SPL = StepShape<N>::SPL;
    static_assert((Q & (Q - 1)) == 0 && 64 % Q == 0, "Q lanes of a channel within one wave");
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t d = i / Q;
    const int j = (int)(i % Q);
    // Q divides the wave size, so the Q lanes of a channel leave together.
    if (d >= p.Dm) return;
    float a[SPL], a2[SPL];  // A and A log2(e) (exponent in base-2 units)
    {
        const float *Ap = p.A + d * N + j * SPL;
        if constexpr (kVec && SPL == 4) {
            const float4 av = *reinterpret_cast<const float4 *>(Ap);
            a[0] = av.x; a[1] = av.y; a[2] = av.z; a[3] = av.w;
        } else {
#pragma unroll
            for (int k = 0; k < SPL; ++k) a[k] = Ap[k];
        }
#pragma unroll
        for (int k = 0; k < SPL; ++k) a2[k] = a[k] * kLog2e;
    }
    const float bias = p.delta_bias != nullptr ? p.delta_bias[d] : 0.f;
    const float Dd = p.D[d];

    // one row group's inputs: state, x and delta of kU rows
    struct In {
        float h[kU][SPL], xv[kU], dv[kU];
    };
    auto load = [&](int64_t b0, In &in) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t b = b0 + u < p.Bsz ? b0 + u : b0;  // rows past the end redo b0 and store nothing
            const int64_t ch = b * p.Dm + d;
            const float *hp = p.h + ch * N + j * SPL;
            if constexpr (kVec && SPL == 4) {
                const f32x4 hv = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(hp));
                in.h[u][0] = hv.x; in.h[u][1] = hv.y; in.h[u][2] = hv.z; in.h[u][3] = hv.w;
            } else {
#pragma unroll
                for (int k = 0; k < SPL; ++k) in.h[u][k] = __builtin_nontemporal_load(hp + k);
            }
            in.xv[u] = to_f32(static_cast<const T *>(p.x)[ch]);
            in.dv[u] = to_f32(static_cast<const T *>(p.delta)[ch]);
        }
    };
    const int64_t gstep = (int64_t)gridDim.y * kU;
    int64_t b0 = (int64_t)blockIdx.y * kU;
    In cur;
    if (b0 < p.Bsz) load(b0, cur);
    for (; b0 < p.Bsz; b0 += gstep) {
        In nxt;
        if (b0 + gstep < p.Bsz) load(b0 + gstep, nxt);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t b = b0 + u < p.Bsz ? b0 + u : b0;
            const int64_t ch = b * p.Dm + d;
            const T *Bp = static_cast<const T *>(p.B) + b * N + j * SPL;
            const T *Cp = static_cast<const T *>(p.C) + b * N + j * SPL;
            float dv = cur.dv[u];
            if (p.delta_bias != nullptr || p.delta_softplus) {  // uniform over the launch
                const float v = dv + bias;
                dv = p.delta_softplus ? (kPrecise ? softplus_precise(v) : softplus_(v)) : v;
            }
            float h[SPL];
            float yv = 0.f;
#pragma unroll
            for (int k = 0; k < SPL; ++k) {
                float abar;
                const float E = kPrecise ? expm1_and_exp_precise(dv * a[k], abar) : expm1_and_exp2(dv * a2[k], abar);
                float coef;
                if (p.euler_b)
                    coef = dv;
                else if constexpr (kPrecise)
                    coef = (a[k] != 0.f) ? E / a[k] : dv;
                else
                    coef = (a[k] != 0.f) ? E * __builtin_amdgcn_rcpf(a[k]) : dv;
                const float bx = to_f32(Bp[k]) * cur.xv[u];
                h[k] = __builtin_fmaf(abar, cur.h[u][k], coef * bx);
                yv = __builtin_fmaf(to_f32(Cp[k]), h[k], yv);
            }
            const bool live = b0 + u < p.Bsz;
            float *hp = p.h + ch * N + j * SPL;
            if (live) {
                if constexpr (kVec && SPL == 4) {
                    const f32x4 hv = {h[0], h[1], h[2], h[3]};
                    __builtin_nontemporal_store(hv, reinterpret_cast<f32x4 *>(hp));
                } else {
#pragma unroll
                    for (int k = 0; k < SPL; ++k) __builtin_nontemporal_store(h[k], hp + k);
                }
            }
#pragma unroll
            for (int off = 1; off < Q; off <<= 1) yv += __shfl_xor(yv, off, Q);
            if (live && j == 0) static_cast<T *>(p.y)[ch] = from_acc<T>(__builtin_fmaf(Dd, cur.xv[u], yv));
        }
        cur = nxt;
    }
}

int g_step_unroll = 1;  // batch rows per thread (1, 2 or 4)

template <typename T, bool kPrecise, int N, bool kVec, int kU>
hipError_t launch_u(const StepParams &p, hipStream_t s) {
    const int64_t lanes = p.Dm * StepShape<N>::Q;
    const unsigned gx = (unsigned)((lanes + kBlock - 1) / kBlock);
    // about 2048 blocks in all (8 per compute unit), at least one row group each
    const int64_t groups = (p.Bsz + kU - 1) / kU;
    int64_t want = (2048 + (int64_t)gx - 1) / (int64_t)gx;
    if (want < 1) want = 1;
    const unsigned gy = (unsigned)(groups < want ? groups : want);
    hipLaunchKernelGGL((step_kernel<T, N, kPrecise, kVec, kU>), dim3(gx, gy), dim3(kBlock), 0, s, p);
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
