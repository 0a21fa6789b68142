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
// lanes of a channel with DPP quad permutations.
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

// Grid: x runs over (channel d, lane j) of one batch row -- d = i / Q and
// j = i % Q with Q a power of two -- and y over groups of kU consecutive batch
// rows.  About one block runs per compute unit, and each thread walks the row
// groups y, y + gridDim.y, ... with the next group's loads issued before the
// current group is computed (two register sets used in turn, no copies).
// Measured on the 256 x 8192 x 16 state, one wave per SIMD with four rows in
// flight per thread moved the state faster than more waves with fewer rows.
// A's row, the bias and D are loaded once per thread.
//
// Rows are addressed through buffer descriptors whose range ends at the last
// batch row: a load of a row past the end returns zeros without a memory
// access and a store there is dropped.  So the next row group is fetched
// unconditionally (a branch around the loads would make the compiler wait for
// them before the current group is computed) and stores need no row test.
// The state moves with non-temporal accesses: it is streamed once per step
// and should not displace the rows every channel shares.
//
// kVec: h, A, B and C are read/written as 8- or 16-byte vectors (needs
// 16-byte aligned base pointers, checked on the host).  kPre: delta goes
// through the bias / softplus of the fused options.
template <typename T, int N, bool kPrecise, bool kVec, int kU, bool kPre>
__global__ __launch_bounds__(kBlock) void step_kernel(StepParams p) {
    constexpr int Q = StepShape<N>::Q;
    constexpr int SPL = StepShape<N>::SPL;
    static_assert((Q & (Q - 1)) == 0 && Q <= 4, "Q lanes of a channel within one quad");
    const int i = blockIdx.x * kBlock + threadIdx.x;
    const int d = i / Q;
    const int j = i % Q;
    // Q divides the wave size, so the Q lanes of a channel leave together.
    if (d >= p.Dm) return;
    float a[SPL], a2[SPL];  // A and A log2(e) (exponent in base-2 units)
    {
        const float *Ap = p.A + (int64_t)d * N + j * SPL;
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
    // The input coefficient is delta (Euler term, or the limit at A = 0) or
    // (exp(delta A) - 1)/A: a per-lane choice fixed for the whole call.
    bool lin[SPL];
    float ainv[SPL];
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
        lin[k] = p.euler_b || a[k] == 0.f;
        ainv[k] = __builtin_amdgcn_rcpf(a[k]);
    }
    const float bias = p.delta_bias != nullptr ? p.delta_bias[d] : 0.f;
    const float Dd = p.D[d];

    const int Dm = (int)p.Dm;
    const int Bsz = (int)p.Bsz;
    const auto rh = make_rsrc(p.h, (int32_t)((int64_t)Bsz * Dm * N * 4));
    const auto rx = make_rsrc(p.x, (int32_t)((int64_t)Bsz * Dm * sizeof(T)));
    const auto rd = make_rsrc(p.delta, (int32_t)((int64_t)Bsz * Dm * sizeof(T)));
    const auto rb = make_rsrc(p.B, (int32_t)(Bsz * N * (int)sizeof(T)));
    const auto rc = make_rsrc(p.C, (int32_t)(Bsz * N * (int)sizeof(T)));
    const auto ry = make_rsrc(p.y, (int32_t)((int64_t)Bsz * Dm * sizeof(T)));
    // per-lane byte offsets within a row; the row goes into the scalar offset
    const int vh = (d * N + j * SPL) * 4;
    const int vx = d * (int)sizeof(T);
    const int vbc = j * SPL * (int)sizeof(T);
    const int rowh = Dm * N * 4, rowx = Dm * (int)sizeof(T), rowbc = N * (int)sizeof(T);

    // One row group's inputs, as stored; converted at use.
    struct In {
        float h[kU][SPL];
        T xv[kU], dv[kU], bv[kU][SPL], cv[kU][SPL];
    };
    auto load = [&](int b0, In &in) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int b = b0 + u;  // rows past the end read zeros
            load_run<float, SPL, kVec, kBufNt>(rh, vh, b * rowh, in.h[u]);
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
            float h[SPL];
            float yv = 0.f;
#pragma unroll
            for (int k = 0; k < SPL; ++k) {
                float abar;
                const float E = kPrecise ? expm1_and_exp_precise(dv * a[k], abar) : expm1_and_exp2(dv * a2[k], abar);
                const float coef = lin[k] ? dv : (kPrecise ? E / a[k] : E * ainv[k]);
                const float bx = to_f32(cur.bv[u][k]) * xv;
                h[k] = __builtin_fmaf(abar, cur.h[u][k], coef * bx);
                yv = __builtin_fmaf(to_f32(cur.cv[u][k]), h[k], yv);
            }
            store_run<SPL, kVec && SPL == 4, kBufNt>(h, rh, vh, b * rowh);
            yv = lane_group_sum<Q>(yv);
            if (j == 0) buf_store(from_acc<T>(__builtin_fmaf(Dd, xv, yv)), ry, vx, b * rowx);
        }
    };
    const int gstep = gridDim.y * kU;
    int b0 = blockIdx.y * kU;
    In ra, rb2;
    load(b0, ra);
    // two copies of the body with the buffers' roles swapped: no register copies
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

int g_step_unroll = 4;  // batch rows per thread and row group (1, 2 or 4)

// Every buffer offset of one launch, including the row group fetched past the
// last row, stays below 2^31: the batch is stepped in slices of at most
// kSliceBytes of state and the row stride of a thread is capped so that the
// overrun is at most another kSliceBytes.  A batch row of state is at most
// kMaxRowBytes (the host rejects larger Dm * N).
constexpr int64_t kSliceBytes = int64_t(1) << 30;
constexpr int64_t kMaxRowBytes = int64_t(1) << 26;
constexpr int64_t kTargetBlocks = 256;  // blocks per launch at four rows per group

template <typename T, bool kPrecise, int N, bool kVec, int kU, bool kPre>
hipError_t launch_p(const StepParams &p, hipStream_t s) {
    const int64_t row_bytes = p.Dm * N * 4;
    const int64_t rows = kSliceBytes / row_bytes;  // >= 16
    const int64_t lanes = p.Dm * StepShape<N>::Q;
    const unsigned gx = (unsigned)((lanes + kBlock - 1) / kBlock);
    // about one block per compute unit at four rows per group (more blocks
    // for fewer rows), at least one row group each
    const int64_t target = kTargetBlocks * 4 / kU;
    int64_t want = (target + (int64_t)gx - 1) / (int64_t)gx;
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
        q.h = p.h + r0 * p.Dm * N;
        const int64_t groups = (q.Bsz + kU - 1) / kU;
        const unsigned gy = (unsigned)(groups < want ? groups : want);
        hipLaunchKernelGGL((step_kernel<T, N, kPrecise, kVec, kU, kPre>), dim3(gx, gy), dim3(kBlock), 0, s, q);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T, bool kPrecise, int N, bool kVec, int kU>
hipError_t launch_u(const StepParams &p, hipStream_t s) {
    if (p.Dm * N * 4 > kMaxRowBytes) return hipErrorInvalidValue;
    if (p.delta_bias != nullptr || p.delta_softplus) return launch_p<T, kPrecise, N, kVec, kU, true>(p, s);
    return launch_p<T, kPrecise, N, kVec, kU, false>(p, s);
}

template <typename T, bool kPrecise, int N>
hipError_t launch_n(const StepParams &p, hipStream_t s) {
    if (p.Bsz * p.Dm == 0) return hipSuccess;
    const bool vec = ((reinterpret_cast<uintptr_t>(p.h) | reinterpret_cast<uintptr_t>(p.A) |
                       reinterpret_cast<uintptr_t>(p.B) | reinterpret_cast<uintptr_t>(p.C)) & 15) == 0;
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
