// Selective scan with complex diagonal A for gfx950: templates shared by
// cplx_bf16.hip and cplx_f32.hip.
//
// The bitig.info page on Mamba-3 (section "Karmasik Degerli Durum
// Guncellemesi") describes a state update with complex eigenvalues, which
// rotate as well as decay.  Per batch row b, channel d, state n, with
// A[d,n] = a + i w, a complex state h and real x, delta, B_t, C_t, D, y:
//   Abar = exp(delta A),  Bbar = (Abar - 1)/A * B_t[n]  (or delta B_t[n], Euler),
//   h_t = Abar h_{t-1} + Bbar x_t,   y_t = sum_n C_t[n] Re(h_t[n]) + D x_t.
//
// The work is laid out as in the real scan (scan_kernels.h): one lane per
// channel with the N complex states in registers, B_t/C_t rows as scalar
// operands, time cut into segments joined by an aggregate pass, a carry pass
// (the decay of a segment is exp(A * sum(delta))) and an output pass.  There
// is no structured fast path: every element takes one exp and one sin/cos pair.
#pragma once

#include "scan_kernels.h"

namespace ssm {

namespace {

// cos and sin of an angle, and exp of a real part.
//  fp32: the angle is reduced to revolutions in [0, 1) and fed to v_sin/v_cos
//        (which take revolutions); exp2 on the transcendental unit.
//  fp64: ocml sin, cos, exp.
__device__ __forceinline__ void cplx_exp(float zr, float zi, float &mag, float &c, float &s, float &em1) {
    constexpr float kInv2Pi = 0.15915494309189535f;
    const float rev = __builtin_amdgcn_fractf(zi * kInv2Pi);
    c = __builtin_amdgcn_cosf(rev);
    s = __builtin_amdgcn_sinf(rev);
    em1 = expm1_and_exp(zr, mag);
}
__device__ __forceinline__ void cplx_exp(double zr, double zi, double &mag, double &c, double &s, double &em1) {
    c = cos(zi);
    s = sin(zi);
    em1 = expm1(zr);
    mag = em1 + 1.0;
}

// Abar - 1 = (e^a cos w - 1) + i e^a sin w, with the real part as
// expm1(a) cos w + (cos w - 1); fp64 writes cos w - 1 as -2 sin^2(w/2).
__device__ __forceinline__ float cplx_cos_m1(float zi, float c) {
    (void)zi;
    return c - 1.0f;
}
__device__ __forceinline__ double cplx_cos_m1(double zi, double c) {
    (void)c;
    const double h = sin(0.5 * zi);
    return -2.0 * h * h;
}

// The same from an exponent already in the units of the transcendental unit:
// fp32 takes the real part in base-2 units (a log2 e) and the angle in
// revolutions (w / 2 pi), which saves two multiplies per element; fp64 takes
// natural units.
__device__ __forceinline__ void cplx_exp_units(float zr2, float zrev, float &mag, float &c, float &s, float &em1) {
    const float rev = __builtin_amdgcn_fractf(zrev);
    c = __builtin_amdgcn_cosf(rev);
    s = __builtin_amdgcn_sinf(rev);
    em1 = expm1_and_exp2(zr2, mag);
}
__device__ __forceinline__ void cplx_exp_units(double zr, double zi, double &mag, double &c, double &s, double &em1) {
    cplx_exp(zr, zi, mag, c, s, em1);
}

template <int N, typename Acc>
struct CplxConst {
    Acc ar[N], ai[N];  // A (a tiny real stand-in for |A| ~ 0)
    Acc wr[N], wi[N];  // 1 / A
    Acc aru[N], aiu[N];  // A in the units of cplx_exp_units
    __device__ __forceinline__ explicit CplxConst(const float *A2) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            Acc a = (Acc)A2[2 * n], w = (Acc)A2[2 * n + 1];
            if (abs_(a) < (Acc)(-kTinyA) && abs_(w) < (Acc)(-kTinyA)) {
                a = (Acc)kTinyA;
                w = 0;
            }
            ar[n] = a;
            ai[n] = w;
            const Acc den = a * a + w * w;
            wr[n] = a / den;
            wi[n] = -w / den;
            aru[n] = sizeof(Acc) == 4 ? a * (Acc)kLog2e : a;
            aiu[n] = sizeof(Acc) == 4 ? w * (Acc)0.15915494309189535 : w;
        }
    }
};

// One step of one channel; returns sum_n C_n Re(h_n) (kOut).
template <int N, bool kOut, bool kEuler, typename Acc>
__device__ __forceinline__ Acc cplx_step(const CplxConst<N, Acc> &cc, const Acc (&row)[2 * N], Acc xv, Acc dv,
                                         Acc (&hr)[N], Acc (&hi)[N]) {
    Acc yv = 0;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const Acc zr = dv * cc.aru[n], zi = dv * cc.aiu[n];
        Acc mag, c, s, em1;
        cplx_exp_units(zr, zi, mag, c, s, em1);
        const Acc abr = mag * c, abi = mag * s;
        const Acc u = row[n] * xv;
        Acc br, bi;
        if constexpr (kEuler) {
            br = dv * u;
            bi = 0;
        } else {
            const Acc er = fma_(em1, c, cplx_cos_m1(zi, c));
            const Acc ei = abi;
            br = (er * cc.wr[n] - ei * cc.wi[n]) * u;
            bi = (er * cc.wi[n] + ei * cc.wr[n]) * u;
        }
        const Acc r = hr[n], m = hi[n];
        hr[n] = fma_(abr, r, fma_(-abi, m, br));
        hi[n] = fma_(abr, m, fma_(abi, r, bi));
        if constexpr (kOut) yv = fma_(row[N + n], hr[n], yv);
    }
    return yv;
}

// B/C rows in the arithmetic type (unscaled).
template <typename T, int N>
__global__ __launch_bounds__(kBlock) void cplx_bc_prep_kernel(const T *__restrict__ B, const T *__restrict__ C,
                                                              typename AccOf<T>::type *__restrict__ bc, int64_t rows) {
    typedef typename AccOf<T>::type Acc;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= rows * N) return;
    const int64_t r = i / N;
    const int n = (int)(i - r * N);
    bc[r * (2 * N) + n] = (Acc)to_f32(B[i]);
    bc[r * (2 * N) + N + n] = (Acc)to_f32(C[i]);
}

// kOut = false: aggregate over segments 0..S-2 (from zero; stores the end
// state and the sum of delta).  kOut = true: output over all segments.
// Scratch: agg [S-1][2N+1][B*D], gin [S][2N][B*D] (re of state n at 2n,
// im at 2n+1, the delta sum at 2N).
template <typename T, int N, bool kOut, bool kEuler, bool kPre>
__global__ __launch_bounds__(kBlock) void cplx_segment_kernel(ScanParams p) {
    typedef typename AccOf<T>::type Acc;
    const int blocks_per_seg = (p.n_tiles + p.waves_per_block - 1) / p.waves_per_block;
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int s = lb / blocks_per_seg;
    const int wave = uniform((int)threadIdx.x / kWave);
    const int tile = (lb - s * blocks_per_seg) * p.waves_per_block + wave;
    if (wave >= p.waves_per_block || tile >= p.n_tiles) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t b = tile / p.tiles_per_b;
    const int64_t d0 = (int64_t)(tile - b * p.tiles_per_b) * kWave;
    const bool active = d0 + lane < p.Dm;
    const int64_t d = active ? d0 + lane : d0;
    const int64_t ch = b * p.Dm + d;
    const int64_t BD = p.Bsz * p.Dm;
    const int64_t t0 = (int64_t)s * p.seg_len;
    const int nsteps = uniform((int)((t0 + p.seg_len < p.L ? t0 + p.seg_len : p.L) - t0));

    const CplxConst<N, Acc> cc(p.A + d * 2 * N);
    const Acc Dd = (Acc)p.D[d];
    const Acc bias = (kPre && p.delta_bias != nullptr) ? (Acc)p.delta_bias[d] : (Acc)0;
    const bool soft = p.delta_softplus != 0;

    Acc hr[N], hi[N];
    if (kOut && p.S > 1) {
        const Acc *gin = static_cast<const Acc *>(p.gin);
#pragma unroll
        for (int n = 0; n < N; ++n) {
            hr[n] = gin[((int64_t)s * 2 * N + 2 * n) * BD + ch];
            hi[n] = gin[((int64_t)s * 2 * N + 2 * n + 1) * BD + ch];
        }
    } else if (kOut && p.h_init != nullptr) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            hr[n] = (Acc)p.h_init[(ch * N + n) * 2];
            hi[n] = (Acc)p.h_init[(ch * N + n) * 2 + 1];
        }
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) hr[n] = hi[n] = 0;
    }

    const int64_t off = (b * p.L + t0) * p.Dm + d0;
    const int32_t row = (int32_t)(p.Dm * (int64_t)sizeof(T));
    const int32_t span = nsteps * row;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(static_cast<const T *>(p.x) + off, span);
    const __amdgpu_buffer_rsrc_t rdl = make_rsrc(static_cast<const T *>(p.delta) + off, span);
    const __amdgpu_buffer_rsrc_t ry =
        make_rsrc(kOut ? static_cast<const T *>(p.y) + off : static_cast<const T *>(p.x) + off, kOut ? span : 0);
    const int32_t voff = (int32_t)((d - d0) * (int64_t)sizeof(T));
    const_row_ptr<Acc> bcp = (const_row_ptr<Acc>)(static_cast<const Acc *>(p.bc) + (b * p.L + t0) * (2 * N));

    constexpr int G = kPrefetch;
    uint32_t xc[G], dc[G], xn[G], dn[G];  // raw bits, one value per register (buf_load_raw)
    auto load = [&](int tb, uint32_t(&xs)[G], uint32_t(&ds)[G]) {
#pragma unroll
        for (int k = 0; k < G; ++k) {
            const int t = tb + k;
            const int so = (t < nsteps - 1 ? t : nsteps - 1) * row;
            xs[k] = buf_load_raw<T, kBufNt>(rx, voff, so);
            ds[k] = buf_load_raw<T, kBufNt>(rdl, voff, so);
        }
    };
    static_assert(G % 2 == 0, "the B/C row buffers alternate within a group");
    Acc lam = 0;
    Acc rowa[2 * N], rowb[2 * N];  // this step's B/C row and the next one's
    load_row<N>(rowa, bcp);
    load(0, xc, dc);
    for (int tb = 0; tb < nsteps; tb += G) {
        load(tb + G, xn, dn);
#pragma unroll
        for (int k = 0; k < G; ++k) {
            const int t = tb + k;
            if (t < nsteps) {
                // as in the real-A scan: wait for this row, then fetch the next
                Acc(&rw)[2 * N] = (k & 1) ? rowb : rowa;
                Acc(&nxt)[2 * N] = (k & 1) ? rowa : rowb;
                row_ready(rw);
                load_row<N>(nxt, bcp + (int64_t)(t + 1 < nsteps ? t + 1 : t) * (2 * N));
                __builtin_amdgcn_sched_barrier(0);
                const Acc xv = (Acc)raw_to_f32<T>(xc[k]);
                Acc dv = (Acc)raw_to_f32<T>(dc[k]);
                if constexpr (kPre) dv = soft ? softplus_(dv + bias) : dv + bias;
                const Acc yv = cplx_step<N, kOut, kEuler>(cc, rw, xv, dv, hr, hi);
                if constexpr (kOut)
                    buf_store<kBufNt>(from_acc<T>(fma_(Dd, xv, yv)), ry, voff, t * row);
                else
                    lam += dv;
            }
        }
#pragma unroll
        for (int k = 0; k < G; ++k) {
            xc[k] = xn[k];
            dc[k] = dn[k];
        }
    }
    if (!active) return;
    if constexpr (!kOut) {
        Acc *a = static_cast<Acc *>(p.agg) + (int64_t)s * (2 * N + 1) * BD + ch;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            a[(int64_t)(2 * n) * BD] = hr[n];
            a[(int64_t)(2 * n + 1) * BD] = hi[n];
        }
        a[(int64_t)(2 * N) * BD] = lam;
    } else if (s == p.S - 1 && p.h_final != nullptr) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            p.h_final[(ch * N + n) * 2] = (float)hr[n];
            p.h_final[(ch * N + n) * 2 + 1] = (float)hi[n];
        }
    }
}

// Carry: one thread per (state n, channel): entering state of s+1 =
// exp(A * sum(delta over s)) * entering state of s + end state of s.
template <typename Acc, int N>
__global__ __launch_bounds__(kBlock) void cplx_carry_kernel(ScanParams p) {
    const int64_t BD = p.Bsz * p.Dm;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= BD * N) return;
    const int n = (int)(i / BD);
    const int64_t ch = i - (int64_t)n * BD;
    const int64_t d = ch % p.Dm;
    const Acc a = (Acc)p.A[(d * N + n) * 2], w = (Acc)p.A[(d * N + n) * 2 + 1];
    Acc cr = 0, ci = 0;
    if (p.h_init) {
        cr = (Acc)p.h_init[(ch * N + n) * 2];
        ci = (Acc)p.h_init[(ch * N + n) * 2 + 1];
    }
    const Acc *agg = static_cast<const Acc *>(p.agg);
    Acc *gin = static_cast<Acc *>(p.gin);
    const int64_t sa = (int64_t)(2 * N + 1) * BD, sg = (int64_t)(2 * N) * BD;
    gin[(int64_t)(2 * n) * BD + ch] = cr;
    gin[(int64_t)(2 * n + 1) * BD + ch] = ci;
    for (int s = 0; s + 1 < p.S; ++s) {
        const Acc lam = agg[(int64_t)s * sa + (int64_t)(2 * N) * BD + ch];
        const Acc gr = agg[(int64_t)s * sa + (int64_t)(2 * n) * BD + ch];
        const Acc gi = agg[(int64_t)s * sa + (int64_t)(2 * n + 1) * BD + ch];
        Acc mag, c, sn, em1;
        cplx_exp(a * lam, w * lam, mag, c, sn, em1);
        const Acc er = mag * c, ei = mag * sn;
        const Acc nr = fma_(er, cr, fma_(-ei, ci, gr));
        const Acc ni = fma_(er, ci, fma_(ei, cr, gi));
        cr = nr;
        ci = ni;
        gin[(int64_t)(s + 1) * sg + (int64_t)(2 * n) * BD + ch] = cr;
        gin[(int64_t)(s + 1) * sg + (int64_t)(2 * n + 1) * BD + ch] = ci;
    }
}

// Decode step: Q lanes per channel, each owning 2 complex states (16 bytes)
// of the state row, so a wave-wide access is 1 KiB contiguous; y is summed
// across the Q lanes with DPP.  Grid: x over (channel d, lane j) of one batch
// row (d = i / Q, j = i % Q, Q a power of two), y over groups of kStepRows
// consecutive batch rows; each thread walks its row groups with the next
// group's loads issued before the current group is computed (two register
// sets used in turn).  The rows go through buffer descriptors whose range
// ends at the last batch row, so the fetch past the end reads zeros without a
// memory access and stores there are dropped: no branch around the loads.
// The per-(d, n) constants of A are formed once per thread.  kVec: state and
// B/C rows as vectors (16-byte aligned pointers, checked on the host); kPre:
// delta goes through the bias / softplus of the fused options.
constexpr int kStepRows = 4;
template <typename T, int N, bool kPrecise, bool kVec, bool kPre>
__global__ __launch_bounds__(kBlock) void cplx_step_kernel(StepParams p) {
    constexpr int SPL = N >= 2 ? 2 : 1;  // complex states per lane
    constexpr int Q = N / SPL;
    constexpr int kU = kStepRows;
    static_assert((Q & (Q - 1)) == 0 && Q <= 8, "Q lanes of a channel within one half-row");
    const int i = blockIdx.x * kBlock + threadIdx.x;
    const int d = i / Q;
    const int j = i % Q;
    if (d >= p.Dm) return;  // the Q lanes of a channel leave together
    float a[SPL], w[SPL], wr[SPL], wi[SPL];
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
        const int n = j * SPL + k;
        a[k] = p.A[((int64_t)d * N + n) * 2];
        w[k] = p.A[((int64_t)d * N + n) * 2 + 1];
        if (__builtin_fabsf(a[k]) < -kTinyA && __builtin_fabsf(w[k]) < -kTinyA) {
            a[k] = kTinyA;
            w[k] = 0.f;
        }
        const float den = a[k] * a[k] + w[k] * w[k];
        wr[k] = a[k] / den;
        wi[k] = -w[k] / den;
    }
    const float bias = p.delta_bias != nullptr ? p.delta_bias[d] : 0.f;
    const float Dd = p.D[d];

    const int Dm = (int)p.Dm;
    const int Bsz = (int)p.Bsz;
    const auto rh = make_rsrc(p.h, (int32_t)((int64_t)Bsz * Dm * N * 8));
    const auto rx = make_rsrc(p.x, (int32_t)((int64_t)Bsz * Dm * sizeof(T)));
    const auto rd = make_rsrc(p.delta, (int32_t)((int64_t)Bsz * Dm * sizeof(T)));
    const auto rb = make_rsrc(p.B, (int32_t)(Bsz * N * (int)sizeof(T)));
    const auto rc = make_rsrc(p.C, (int32_t)(Bsz * N * (int)sizeof(T)));
    const auto ry = make_rsrc(p.y, (int32_t)((int64_t)Bsz * Dm * sizeof(T)));
    const int vh = (d * N + j * SPL) * 8;
    const int vx = d * (int)sizeof(T);
    const int vbc = j * SPL * (int)sizeof(T);
    const int rowh = Dm * N * 8, rowx = Dm * (int)sizeof(T), rowbc = N * (int)sizeof(T);

    struct In {
        float h[kU][2 * SPL];  // (re, im) pairs
        T xv[kU], dv[kU], bv[kU][SPL], cv[kU][SPL];
    };
    auto load = [&](int b0, In &in) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int b = b0 + u;  // rows past the end read zeros
            load_run<float, 2 * SPL, kVec, kBufNt>(rh, vh, b * rowh, in.h[u]);
            T tmp[1];
            load_run<T, 1, false, 0>(rx, vx, b * rowx, tmp);
            in.xv[u] = tmp[0];
            load_run<T, 1, false, 0>(rd, vx, b * rowx, tmp);
            in.dv[u] = tmp[0];
            load_run<T, SPL, kVec, 0>(rb, vbc, b * rowbc, in.bv[u]);
            load_run<T, SPL, kVec, 0>(rc, vbc, b * rowbc, in.cv[u]);
        }
    };
    auto compute = [&](int b0, const In &cur) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int b = b0 + u;  // rows past the end compute on zeros and store nothing
            const float xv = to_f32(cur.xv[u]);
            float dv = to_f32(cur.dv[u]);
            if constexpr (kPre) {
                const float v = dv + bias;
                dv = p.delta_softplus ? (kPrecise ? softplus_precise(v) : softplus_(v)) : v;
            }
            float hn[2 * SPL];
            float yv = 0.f;
#pragma unroll
            for (int k = 0; k < SPL; ++k) {
                const float zr = dv * a[k], zi = dv * w[k];
                float mag, c, s, em1;
                if constexpr (kPrecise) {
                    c = cosf(zi);
                    s = sinf(zi);
                    em1 = expm1f(zr);
                    mag = em1 + 1.f;
                } else {
                    cplx_exp(zr, zi, mag, c, s, em1);
                }
                const float abr = mag * c, abi = mag * s;
                const float uu = to_f32(cur.bv[u][k]) * xv;
                float br, bi;
                if (p.euler_b) {
                    br = dv * uu;
                    bi = 0.f;
                } else {
                    const float hs = kPrecise ? sinf(0.5f * zi) : 0.f;
                    const float cm1 = kPrecise ? -2.f * hs * hs : c - 1.f;
                    const float er = __builtin_fmaf(em1, c, cm1), ei = abi;
                    br = (er * wr[k] - ei * wi[k]) * uu;
                    bi = (er * wi[k] + ei * wr[k]) * uu;
                }
                const float r = cur.h[u][2 * k], m = cur.h[u][2 * k + 1];
                hn[2 * k] = __builtin_fmaf(abr, r, __builtin_fmaf(-abi, m, br));
                hn[2 * k + 1] = __builtin_fmaf(abr, m, __builtin_fmaf(abi, r, bi));
                yv = __builtin_fmaf(to_f32(cur.cv[u][k]), hn[2 * k], yv);
            }
            store_run<2 * SPL, kVec, kBufNt>(hn, rh, vh, b * rowh);
            yv = lane_group_sum<Q>(yv);
            if (j == 0) buf_store(from_acc<T>(__builtin_fmaf(Dd, xv, yv)), ry, vx, b * rowx);
        }
    };
    const int gstep = gridDim.y * kU;
    int b0 = blockIdx.y * kU;
    In ra, rb2;
    load(b0, ra);
    for (;;) {
        load(b0 + gstep, rb2);
        compute(b0, ra);
        b0 += gstep;
        if (b0 >= Bsz) break;
        load(b0 + gstep, ra);
        compute(b0, rb2);
        b0 += gstep;
        if (b0 >= Bsz) break;
    }
}

template <typename T, int N, bool kOut>
void cplx_launch_segments(const ScanParams &p, unsigned grid, hipStream_t s) {
    const bool pre = p.delta_bias != nullptr || p.delta_softplus != 0;
    if (p.euler_b) {
        if (pre)
            hipLaunchKernelGGL((cplx_segment_kernel<T, N, kOut, true, true>), dim3(grid), dim3(kBlock), 0, s, p);
        else
            hipLaunchKernelGGL((cplx_segment_kernel<T, N, kOut, true, false>), dim3(grid), dim3(kBlock), 0, s, p);
    } else {
        if (pre)
            hipLaunchKernelGGL((cplx_segment_kernel<T, N, kOut, false, true>), dim3(grid), dim3(kBlock), 0, s, p);
        else
            hipLaunchKernelGGL((cplx_segment_kernel<T, N, kOut, false, false>), dim3(grid), dim3(kBlock), 0, s, p);
    }
}

template <typename T, int N>
hipError_t cplx_pass_n(ScanPass pass, const ScanParams &p, hipStream_t s) {
    typedef typename AccOf<T>::type Acc;
    switch (pass) {
        case ScanPass::kPrep: {
            const int64_t work = p.Bsz * p.L * N;
            if (work == 0) return hipSuccess;
            hipLaunchKernelGGL((cplx_bc_prep_kernel<T, N>), dim3((unsigned)((work + kBlock - 1) / kBlock)),
                               dim3(kBlock), 0, s, static_cast<const T *>(p.B), static_cast<const T *>(p.C),
                               static_cast<Acc *>(p.bc), p.Bsz * p.L);
            break;
        }
        case ScanPass::kAggregate:
        case ScanPass::kOutput: {
            const bool out = pass == ScanPass::kOutput;
            const int bps = (p.n_tiles + p.waves_per_block - 1) / p.waves_per_block;
            const int nseg = out ? p.S : p.S - 1;
            if (nseg <= 0 || bps == 0) return hipSuccess;
            const unsigned grid = (unsigned)bps * (unsigned)nseg;
            if (out)
                cplx_launch_segments<T, N, true>(p, grid, s);
            else
                cplx_launch_segments<T, N, false>(p, grid, s);
            break;
        }
        case ScanPass::kCarry: {
            const int64_t work = p.Bsz * p.Dm * N;
            if (work == 0 || p.S <= 1) return hipSuccess;
            hipLaunchKernelGGL((cplx_carry_kernel<Acc, N>), dim3((unsigned)((work + kBlock - 1) / kBlock)),
                               dim3(kBlock), 0, s, p);
            break;
        }
    }
    return hipGetLastError();
}

template <typename T>
hipError_t cplx_pass(ScanPass pass, const ScanParams &p, int N, hipStream_t s) {
    switch (N) {
        case 1: return cplx_pass_n<T, 1>(pass, p, s);
        case 2: return cplx_pass_n<T, 2>(pass, p, s);
        case 4: return cplx_pass_n<T, 4>(pass, p, s);
        case 8: return cplx_pass_n<T, 8>(pass, p, s);
        case 16: return cplx_pass_n<T, 16>(pass, p, s);
        default: return hipErrorInvalidValue;
    }
}

// Offsets of one launch, the fetch past the last row included, stay below
// 2^31: the batch is stepped in slices of at most kCplxSliceBytes of state,
// the row stride of a thread is capped so that the overrun is at most as much
// again, and a batch row holds at most kCplxMaxRowBytes (the host rejects
// larger Dm * N).
constexpr int64_t kCplxSliceBytes = int64_t(1) << 30;
constexpr int64_t kCplxMaxRowBytes = int64_t(1) << 26;
constexpr int64_t kCplxTargetBlocks = 256;  // blocks per launch: about one per compute unit

template <typename T, bool kPrecise, int N, bool kVec, bool kPre>
hipError_t cplx_step_n(const StepParams &p, hipStream_t s) {
    constexpr int Q = N >= 2 ? N / 2 : 1;
    constexpr int kU = kStepRows;
    const int64_t row_bytes = p.Dm * N * 8;
    const int64_t rows = kCplxSliceBytes / row_bytes;  // >= 16
    const unsigned gx = (unsigned)((p.Dm * Q + kBlock - 1) / kBlock);
    int64_t want = (kCplxTargetBlocks + (int64_t)gx - 1) / (int64_t)gx;
    if (want > rows / kU - 1) want = rows / kU - 1;
    if (want < 1) want = 1;
    for (int64_t r0 = 0; r0 < p.Bsz; r0 += rows) {
        StepParams q = p;
        q.Bsz = p.Bsz - r0 < rows ? p.Bsz - r0 : rows;
        q.x = static_cast<const T *>(p.x) + r0 * p.Dm;
        q.delta = static_cast<const T *>(p.delta) + r0 * p.Dm;
        q.y = static_cast<T *>(p.y) + r0 * p.Dm;
        q.B = static_cast<const T *>(p.B) + r0 * N;
        q.C = static_cast<const T *>(p.C) + r0 * N;
        q.h = p.h + r0 * p.Dm * N * 2;
        const int64_t groups = (q.Bsz + kU - 1) / kU;
        const dim3 grid(gx, (unsigned)(groups < want ? groups : want));
        hipLaunchKernelGGL((cplx_step_kernel<T, N, kPrecise, kVec, kPre>), grid, dim3(kBlock), 0, s, q);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T, bool kPrecise, int N>
hipError_t cplx_step_v(const StepParams &p, hipStream_t s) {
    if (p.Dm * N * 8 > kCplxMaxRowBytes) return hipErrorInvalidValue;
    const bool vec = ((reinterpret_cast<uintptr_t>(p.h) | reinterpret_cast<uintptr_t>(p.B) |
                       reinterpret_cast<uintptr_t>(p.C)) & 15) == 0;
    const bool pre = p.delta_bias != nullptr || p.delta_softplus;
    if (vec) return pre ? cplx_step_n<T, kPrecise, N, true, true>(p, s) : cplx_step_n<T, kPrecise, N, true, false>(p, s);
    return pre ? cplx_step_n<T, kPrecise, N, false, true>(p, s) : cplx_step_n<T, kPrecise, N, false, false>(p, s);
}

template <typename T, bool kPrecise>
hipError_t cplx_step_launch(const StepParams &p, int N, hipStream_t s) {
    if (p.Bsz * p.Dm == 0) return hipSuccess;
    switch (N) {
        case 1: return cplx_step_v<T, kPrecise, 1>(p, s);
        case 2: return cplx_step_v<T, kPrecise, 2>(p, s);
        case 4: return cplx_step_v<T, kPrecise, 4>(p, s);
        case 8: return cplx_step_v<T, kPrecise, 8>(p, s);
        case 16: return cplx_step_v<T, kPrecise, 16>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

}  // namespace ssm
