// Scalar-decay (state-space duality) layer for fp32 storage: the recurrence
// in fp64.  The chunked matrix form (ssd_kernels.h) accumulates in fp32 on the
// matrix cores, which does not keep the fp32 storage path's error bound.
#include "ssd_kernels.h"

namespace ssm {

namespace {

// fp32 storage: h_t = exp(dt a) h_{t-1} + k_t B_t x_t, y_t = C_t h_t + D x_t in
// fp64, one thread per (b, d, 8 states); the N/8 threads of a channel are
// adjacent lanes and sum y with shuffles.  One pass over all of time (the
// plan keeps a single segment), so h_init may equal h_final.
template <int N>
__global__ __launch_bounds__(256) void ssd_recurrence_f64_kernel(SsdParams p) {
    constexpr int kG = 8;        // states per thread
    constexpr int kT = N / kG;   // threads per channel (divides 64)
    const int64_t total = p.Bsz * p.Dm * kT;
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool ok = tid < total;  // a channel's lanes are all in or all out
    const int64_t q = ok ? tid : total - 1;
    const int grp = (int)(q % kT);
    const int64_t bd = q / kT;
    const int64_t b = bd / p.Dm, d = bd - b * p.Dm;
    const int64_t h = d / kSsdP;
    const double a = p.A[h];
    const double bias = p.delta_bias ? (double)p.delta_bias[h] : 0.0;
    const double Dd = p.D[d];
    double hs[kG];
#pragma unroll
    for (int e = 0; e < kG; ++e) hs[e] = p.h_init ? (double)p.h_init[bd * N + kG * grp + e] : 0.0;
    const float *x = static_cast<const float *>(p.x);
    const float *dl = static_cast<const float *>(p.delta);
    const float *Bm = static_cast<const float *>(p.B);
    const float *Cm = static_cast<const float *>(p.C);
    float *y = static_cast<float *>(p.y);
    for (int64_t t = 0; t < p.L; ++t) {
        const int64_t bt = b * p.L + t;
        double dt = (double)dl[bt * p.H + h] + bias;
        if (p.delta_softplus) dt = softplus_(dt);
        const double la = dt * a;
        const double abar = exp(la);
        const double k = (p.euler_b || __builtin_fabs(a) < 1e-20) ? dt : expm1(la) / a;
        const double xv = x[bt * p.Dm + d];
        const double u = k * xv;
        const float *Bt = Bm + bt * N + kG * grp;
        const float *Ct = Cm + bt * N + kG * grp;
        double yv = 0.0;
#pragma unroll
        for (int e = 0; e < kG; ++e) {
            hs[e] = fma_(abar, hs[e], u * (double)Bt[e]);
            yv = fma_((double)Ct[e], hs[e], yv);
        }
#pragma unroll
        for (int off = 1; off < kT; off <<= 1) yv += __shfl_xor(yv, off);
        if (ok && grp == 0) y[bt * p.Dm + d] = (float)fma_(Dd, xv, yv);
    }
    if (ok && p.h_final != nullptr)
#pragma unroll
        for (int e = 0; e < kG; ++e) p.h_final[bd * N + kG * grp + e] = (float)hs[e];
}

template <int N>
hipError_t ssd_pass_f64_n(SsdPass pass, const SsdParams &p, hipStream_t s) {
    if (pass != SsdPass::kOutput) return hipSuccess;
    const int64_t n = p.Bsz * p.Dm * (N / 8);
    hipLaunchKernelGGL(ssd_recurrence_f64_kernel<N>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t ssd_pass_f64(SsdPass pass, const SsdParams &p, int N, hipStream_t s) {
    switch (N) {
        case 32: return ssd_pass_f64_n<32>(pass, p, s);
        case 64: return ssd_pass_f64_n<64>(pass, p, s);
        case 128: return ssd_pass_f64_n<128>(pass, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t ssd_pass_f32(SsdPass pass, const SsdParams &p, int N, hipStream_t s) {
    return ssd_pass_f64(pass, p, N, s);
}

}  // namespace ssm
