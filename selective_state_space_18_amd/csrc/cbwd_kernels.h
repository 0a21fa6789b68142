// Backward of the selective scan with complex diagonal A for gfx950:
// templates shared by cbwd_bf16.hip and cbwd_f32.hip.
//
// The recurrence is the complex-A forward's (cplx_kernels.h; the bitig.info
// page on Mamba-3, section "Karmasik Degerli Durum Guncellemesi"), and the
// gradients its chain rule ("Mamba SSM Nedir?", section "Paralel Tarama
// Algoritmasi": training runs the same scan).  Every complex quantity is a
// pair of reals; for a real loss and w = p q the gradient pair of p is G_w
// conj(q) as a complex number.  With lambda = dL/dh_t (complex), u = B_t[n] x_t
// and k the input coefficient ((Abar - 1)/A, or delta for the Euler rule):
//   lambda   += C_t[n] dy_t                (y reads Re h)
//   dL/du     = Re(lambda conj(k))         -> dx, dB
//   ddelta   += Re(lambda conj(h_{t-1}) conj(A Abar)) + Re(lambda u conj(dk/ddelta))
//   dA       += lambda conj(h_{t-1}) conj(delta Abar)  + lambda u conj(dk/dA)
//   lambda    = lambda conj(Abar)          (into step t-1)
// with dk/ddelta = Abar, dk/dA = (delta A Abar - (Abar - 1)) / A^2 (ZOH), and
// dk/ddelta = 1, dk/dA = 0 (Euler).
//
// Work layout, as the real backward (bwd_kernels.h), one lane per channel:
//   1. cbwd_aggregate_kernel: per 16-step segment, in one pass forward in
//      time, the end state from a zero start (the complex forward's carry,
//      cplx_carry_kernel, then gives the state entering every segment) and
//      the adjoint a zero adjoint at the segment end leaves at its start;
//   2. cbwd_carry_kernel composes the adjoint summaries from the right and
//      keeps the adjoint entering the last segment of each group;
//   3. cbwd_main_kernel: a block per group of segments and two 64-channel
//      tiles, last segment first.  A tile is shared by two waves, each holding
//      half of its N complex states, so that two blocks fit on a compute unit
//      (two waves per SIMD).  Per segment, the states before steps 4, 8 and 12
//      go to LDS; each 4-step sub-chunk's states are recomputed from its
//      checkpoint, then the adjoint runs back over them, and the two waves of
//      a tile add their dx and d(delta) shares through LDS.  dB and dC (sums
//      over channels) go through the real backward's reduce-scatter and
//      per-block LDS sums, then cbwd_reduce_kernel.
#pragma once

#include "bwd_kernels.h"
#include "cplx_kernels.h"

namespace ssm {

namespace {

// Main-kernel blocks: kWaves waves; kBlocksPerCU of them share a compute
// unit (their LDS fits), one wave per SIMD each.  fp64 arithmetic doubles the
// checkpoints, so that block takes a compute unit alone.
template <typename Acc>
struct CbwdShape;
template <>
struct CbwdShape<float> {
    static constexpr int kWaves = 4;
    static constexpr int kBlocksPerCU = 2;
};
template <>
struct CbwdShape<double> {
    static constexpr int kWaves = 4;
    static constexpr int kBlocksPerCU = 1;
};
constexpr int kCbwdT = 16;  // segment length
constexpr int kCbwdK = 4;   // checkpoint interval = sub-chunk length
// Waves that share one 64-channel tile in the main kernel, each holding
// N / split of its states.
template <int N>
constexpr int cbwd_split() {
    return N >= 2 ? 2 : 1;
}

// A and 1/A of one channel.  The exponent is formed as (delta * unit) * A with
// the unit taken per step (log2 e and 1/(2 pi) in fp32 arithmetic, where the
// transcendental unit takes base-2 exponents and angles in revolutions), so
// no scaled copy of A is kept.
template <int N, typename Acc>
struct CbwdConst {
    Acc ar[N], ai[N];  // A (the forward's tiny real stand-in for |A| ~ 0)
    Acc wr[N], wi[N];  // 1 / A
    __device__ __forceinline__ explicit CbwdConst(const float *A2) {
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
        }
    }
};

// delta in the exponent units of cplx_exp_units: (real part, angle).
template <typename Acc>
__device__ __forceinline__ void delta_units(Acc dv, Acc &ur, Acc &ui) {
    ur = sizeof(Acc) == 4 ? dv * (Acc)kLog2e : dv;
    ui = sizeof(Acc) == 4 ? dv * (Acc)0.15915494309189535 : dv;
}

// Abar = exp(delta A) of state n, Re(Abar - 1) (er; Im(Abar - 1) = abi) and
// the input coefficient k ((Abar - 1)/A, or delta for the Euler rule).
template <int N, bool kEuler, typename Acc>
__device__ __forceinline__ void cplx_coef(const CbwdConst<N, Acc> &cc, int n, Acc dv, Acc ur, Acc ui, Acc &abr,
                                          Acc &abi, Acc &kr, Acc &ki, Acc &er) {
    const Acc zi = ui * cc.ai[n];
    Acc mag, c, s, em1;
    cplx_exp_units(ur * cc.ar[n], zi, mag, c, s, em1);
    abr = mag * c;
    abi = mag * s;
    er = fma_(em1, c, cplx_cos_m1(zi, c));
    if constexpr (kEuler) {
        kr = dv;
        ki = 0;
    } else {
        kr = er * cc.wr[n] - abi * cc.wi[n];
        ki = er * cc.wi[n] + abi * cc.wr[n];
    }
}

// One forward step of one channel (states advanced in place).
template <int N, bool kEuler, typename Acc>
__device__ __forceinline__ void cbwd_fwd_step(const CbwdConst<N, Acc> &cc, const Acc (&row)[2 * N], Acc xv, Acc dv,
                                              Acc (&hr)[N], Acc (&hi)[N]) {
    Acc ur, ui;
    delta_units(dv, ur, ui);
#pragma unroll
    for (int n = 0; n < N; ++n) {
        Acc abr, abi, kr, ki, er;
        cplx_coef<N, kEuler>(cc, n, dv, ur, ui, abr, abi, kr, ki, er);
        const Acc u = row[n] * xv;
        const Acc r = hr[n], m = hi[n];
        hr[n] = fma_(abr, r, fma_(-abi, m, kr * u));
        hi[n] = fma_(abr, m, fma_(abi, r, ki * u));
    }
}

// dk/dA of state n for ZOH: (delta A Abar - (Abar - 1)) / A^2 = (delta Abar -
// k) / A = delta^2 phi'(delta A), phi'(z) = (z e^z - (e^z - 1)) / z^2.  Near
// z = 0 the closed forms cancel: they lose about log2(2/|z|) bits.
//  fp64: the Taylor polynomial to z^4 where |z| < 1/1000 (truncation below
//        |z|^5 / 840), the closed form elsewhere.
//  fp32: (delta Abar - k) / A, with no branch (a per-lane branch here costs
//        the registers that keep the kernel at two waves per SIMD).  Its
//        absolute error is about 6 eps |delta| / |A| against a value near
//        delta^2 / 2: a few eps of the dA sum for |A| above about 1e-3.  The
//        tiny real stand-in that replaces A = 0 takes the limit delta^2 / 2
//        instead (exact in fp32 at that |z|).
template <int N, typename Acc>
__device__ __forceinline__ void cplx_dk_da(const CbwdConst<N, Acc> &cc, int n, Acc dv, Acc abr, Acc abi, Acc er,
                                           Acc kr, Acc ki, Acc &gr, Acc &gi) {
    if constexpr (sizeof(Acc) == 4) {
        (void)er;
        const Acc nr = fma_(dv, abr, -kr), ni = fma_(dv, abi, -ki);
        const Acc cr = nr * cc.wr[n] - ni * cc.wi[n];
        const Acc ci = nr * cc.wi[n] + ni * cc.wr[n];
        const bool zero = cc.ar[n] == (Acc)kTinyA && cc.ai[n] == (Acc)0;
        gr = zero ? (Acc)0.5 * dv * dv : cr;
        gi = zero ? (Acc)0 : ci;
        return;
    }
    (void)kr;
    (void)ki;
    const Acc zr = dv * cc.ar[n], zi = dv * cc.ai[n];
    if (zr * zr + zi * zi < (Acc)1e-6) {
        // 1/2 + z/3 + z^2/8 + z^3/30 + z^4/144 (Horner, complex)
        Acc pr = (Acc)(1.0 / 144.0), pi = 0;
        const Acc cs[4] = {(Acc)(1.0 / 30.0), (Acc)(1.0 / 8.0), (Acc)(1.0 / 3.0), (Acc)0.5};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const Acc r = fma_(pr, zr, fma_(-pi, zi, cs[k]));
            const Acc m = fma_(pr, zi, pi * zr);
            pr = r;
            pi = m;
        }
        const Acc d2 = dv * dv;
        gr = pr * d2;
        gi = pi * d2;
    } else {
        // (z Abar - E) W^2, W = 1/A
        const Acc nr = (zr * abr - zi * abi) - er;
        const Acc ni = (zr * abi + zi * abr) - abi;
        const Acc w2r = cc.wr[n] * cc.wr[n] - cc.wi[n] * cc.wi[n];
        const Acc w2i = 2 * cc.wr[n] * cc.wi[n];
        gr = nr * w2r - ni * w2i;
        gi = nr * w2i + ni * w2r;
    }
}

// ---------------------------------------------------------------------------
// Segment summaries of both directions in one pass over each segment, which
// forms every Abar once for both:
//  * forward (segments 0..S-2, for the complex forward's carry): the end
//    state from a zero start, agg [S-1][2N+1][B*D];
//  * reverse (segments 1..S-1): the adjoint that a zero adjoint at the
//    segment end leaves at its start, after the first step's decay,
//    ragg [S][2N+1][B*D].  Run back step by step it is
//    sum_i c_i conj(P_i) with c_i = C_i[n] dy_i and P_i = Abar_0 ... Abar_i,
//    so forward in time it takes the running product P and one complex
//    multiply-add per step.
// Both store the segment's sum of delta in slot 2N.
template <typename T, int N, bool kEuler, bool kPre>
__global__ __launch_bounds__(kBlock) void cbwd_aggregate_kernel(BwdParams q) {
    typedef typename AccOf<T>::type Acc;
    const ScanParams &p = q.f;
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
    const bool fwd = s + 1 < p.S, rev = s > 0;

    const CbwdConst<N, Acc> cc(p.A + d * 2 * N);
    const Acc bias = (kPre && p.delta_bias != nullptr) ? (Acc)p.delta_bias[d] : (Acc)0;
    const bool soft = p.delta_softplus != 0;
    const int64_t off = (b * p.L + t0) * p.Dm + d0;
    const int32_t row = (int32_t)(p.Dm * (int64_t)sizeof(T));
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(static_cast<const T *>(p.x) + off, nsteps * row);
    const __amdgpu_buffer_rsrc_t rdl = make_rsrc(static_cast<const T *>(p.delta) + off, nsteps * row);
    const __amdgpu_buffer_rsrc_t rdy = make_rsrc(static_cast<const T *>(q.dy) + off, nsteps * row);
    const int32_t voff = (int32_t)((d - d0) * (int64_t)sizeof(T));
    const_row_ptr<Acc> bcp = (const_row_ptr<Acc>)(static_cast<const Acc *>(p.bc) + (b * p.L + t0) * (2 * N));

    Acc hr[N], hi[N], pr[N], pi[N], rr[N], ri[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        hr[n] = hi[n] = rr[n] = ri[n] = pi[n] = 0;
        pr[n] = 1;
    }
    Acc lam = 0;
    // the step's inputs, and the next step's fetched meanwhile
    uint32_t xc = buf_load_raw<T>(rx, voff, 0), dlc = buf_load_raw<T>(rdl, voff, 0);
    uint32_t dyc = buf_load_raw<T>(rdy, voff, 0);
    for (int i = 0; i < nsteps; ++i) {
        const int j = i + 1 < nsteps ? i + 1 : i;
        const uint32_t xn = buf_load_raw<T>(rx, voff, j * row), dln = buf_load_raw<T>(rdl, voff, j * row);
        const uint32_t dyn = buf_load_raw<T>(rdy, voff, j * row);
        Acc rw[2 * N];
        load_row<N>(rw, bcp + (int64_t)i * (2 * N));
        Acc dv = (Acc)raw_to_f32<T>(dlc);
        if constexpr (kPre) dv = soft ? softplus_(dv + bias) : dv + bias;
        const Acc xv = (Acc)raw_to_f32<T>(xc), gy = (Acc)raw_to_f32<T>(dyc);
        lam += dv;
        Acc ur, ui;
        delta_units(dv, ur, ui);
#pragma unroll
        for (int n = 0; n < N; ++n) {
            Acc abr, abi, kr, ki, er;
            cplx_coef<N, kEuler>(cc, n, dv, ur, ui, abr, abi, kr, ki, er);
            if (fwd) {
                const Acc u = rw[n] * xv;
                const Acc r = hr[n], m = hi[n];
                hr[n] = fma_(abr, r, fma_(-abi, m, kr * u));
                hi[n] = fma_(abr, m, fma_(abi, r, ki * u));
            }
            if (rev) {
                // P = P Abar;  R += c conj(P)
                const Acc r = pr[n], m = pi[n];
                pr[n] = fma_(r, abr, -m * abi);
                pi[n] = fma_(r, abi, m * abr);
                const Acc c = rw[N + n] * gy;
                rr[n] = fma_(c, pr[n], rr[n]);
                ri[n] = fma_(-c, pi[n], ri[n]);
            }
        }
        xc = xn;
        dlc = dln;
        dyc = dyn;
    }
    if (!active) return;
    if (fwd) {
        Acc *a = static_cast<Acc *>(p.agg) + (int64_t)s * (2 * N + 1) * BD + ch;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            a[(int64_t)(2 * n) * BD] = hr[n];
            a[(int64_t)(2 * n + 1) * BD] = hi[n];
        }
        a[(int64_t)(2 * N) * BD] = lam;
    }
    if (rev) {
        Acc *a = static_cast<Acc *>(q.ragg) + (int64_t)s * (2 * N + 1) * BD + ch;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            a[(int64_t)(2 * n) * BD] = rr[n];
            a[(int64_t)(2 * n + 1) * BD] = ri[n];
        }
        a[(int64_t)(2 * N) * BD] = lam;
    }
}

// Reverse carry: one thread per (state n, channel).  The adjoint entering the
// last segment is dL/dh_final; segment s-1 receives conj(exp(A sum(delta over
// s))) times what enters s, plus s's summary.  Only the adjoint entering each
// group's last segment is kept (gout [groups][2N][B*D]).
template <typename Acc, int N>
__global__ __launch_bounds__(kBlock) void cbwd_carry_kernel(BwdParams q) {
    const ScanParams &p = q.f;
    const int64_t BD = p.Bsz * p.Dm;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= BD * N) return;
    const int n = (int)(i / BD);
    const int64_t ch = i - (int64_t)n * BD;
    const int64_t d = ch % p.Dm;
    const Acc a = (Acc)p.A[(d * N + n) * 2], w = (Acc)p.A[(d * N + n) * 2 + 1];
    Acc lr = 0, li = 0;
    if (q.dh_final) {
        lr = (Acc)q.dh_final[(ch * N + n) * 2];
        li = (Acc)q.dh_final[(ch * N + n) * 2 + 1];
    }
    const Acc *ragg = static_cast<const Acc *>(q.ragg);
    Acc *out = static_cast<Acc *>(q.gout);
    const int64_t sa = (int64_t)(2 * N + 1) * BD, sg = (int64_t)(2 * N) * BD;
    const int spg = q.seg_per_group;
    auto put = [&](int grp) {
        out[(int64_t)grp * sg + (int64_t)(2 * n) * BD + ch] = lr;
        out[(int64_t)grp * sg + (int64_t)(2 * n + 1) * BD + ch] = li;
    };
    put((p.S - 1) / spg);
    for (int s = p.S - 1; s >= 1; --s) {
        const Acc lam = ragg[(int64_t)s * sa + (int64_t)(2 * N) * BD + ch];
        const Acc gr = ragg[(int64_t)s * sa + (int64_t)(2 * n) * BD + ch];
        const Acc gi = ragg[(int64_t)s * sa + (int64_t)(2 * n + 1) * BD + ch];
        Acc mag, c, sn, em1;
        cplx_exp(a * lam, w * lam, mag, c, sn, em1);
        const Acc er = mag * c, ei = mag * sn;  // exp(A sum); the adjoint takes its conjugate
        const Acc nr = fma_(er, lr, fma_(ei, li, gr));
        const Acc ni = fma_(er, li, fma_(-ei, lr, gi));
        lr = nr;
        li = ni;
        if ((s - 1) % spg == spg - 1) put((s - 1) / spg);
    }
}

// ---------------------------------------------------------------------------
// Main pass.  A 64-channel tile is shared by cbwd_split<N>() waves, wave h
// holding states n0 = h NH .. n0 + NH - 1 (NH = N / split): their registers
// and checkpoints are halved, so two blocks fit on a compute unit.  The
// waves of a tile add their shares of dx and d(delta) through LDS once per
// sub-chunk (the first wave stores them).
// part_bc [blocks per row][2][B*L*N] (block sums of the dB and dC lane
// values), part_a [groups][B*D][2N] (dA), part_d [groups][B*D][2] (dD,
// d(delta_bias)).
template <int NH, int N, typename Acc>
__device__ __forceinline__ void load_half_row(Acc (&dst)[2 * NH], const_row_ptr<Acc> row, int n0) {
#pragma unroll
    for (int i = 0; i < NH; ++i) {
        dst[i] = row[n0 + i];
        dst[NH + i] = row[N + n0 + i];
    }
}

template <typename T, int N, bool kEuler, bool kPre>
__global__ __launch_bounds__(CbwdShape<typename AccOf<T>::type>::kWaves *kWave,
                             CbwdShape<typename AccOf<T>::type>::kBlocksPerCU) void cbwd_main_kernel(BwdParams q) {
    typedef typename AccOf<T>::type Acc;
    constexpr int kWaves = CbwdShape<Acc>::kWaves;
    constexpr int P = cbwd_split<N>();
    constexpr int NH = N / P;
    constexpr int kTiles = kWaves / P;
    constexpr int kT = kCbwdT, kK = kCbwdK, kNck = kT / kK;
    __shared__ Acc ck[kWaves][kNck - 1][2 * NH][kWave];  // state before steps 4, 8, 12, per wave
    __shared__ Acc bacc[kTiles][kT][2][N];               // per-tile dB, dC sums of one segment
    __shared__ Acc xb[2][kTiles][kK][2][kWave];          // shares of dx, d(delta) from waves h > 0
    static_assert(sizeof(ck) + sizeof(bacc) + (P > 1 ? sizeof(xb) : 0) <= 163840 / CbwdShape<Acc>::kBlocksPerCU,
                  "the blocks of one compute unit must fit its 160 KB of LDS");
    static_assert(P <= 2 && kWaves % P == 0, "xb holds the share of one other wave per tile");
    const ScanParams &p = q.f;

    const int wave = uniform((int)threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    const int tb = wave / P;  // tile within the block
    const int half = wave - tb * P;
    const int n0 = uniform(half * NH);
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int per_grp = (int)p.Bsz * q.blocks_per_row;
    const int grp = lb / per_grp;
    const int rem = lb - grp * per_grp;
    const int64_t b = rem / q.blocks_per_row;
    const int br = rem - (int)b * q.blocks_per_row;
    const int tir = br * kTiles + tb;
    const bool tile_ok = tir < p.tiles_per_b;
    const int64_t d0 = (int64_t)(tile_ok ? tir : p.tiles_per_b - 1) * kWave;
    const bool in_range = d0 + lane < p.Dm;
    const int64_t d = in_range ? d0 + lane : d0;  // idle lanes shadow a valid channel
    const int64_t ch = b * p.Dm + d;
    const int64_t BD = p.Bsz * p.Dm;
    const int64_t BLN = p.Bsz * p.L * N;
    // tiles past the row and lanes past it run on x = dy = 0: every dB, dC,
    // dx and d(delta) share is a multiple of x or dy, and they store nothing
    const bool live = tile_ok && in_range;

    const CbwdConst<NH, Acc> cc(p.A + (d * N + n0) * 2);
    const Acc Dd = (Acc)p.D[d];
    const Acc bias = (kPre && p.delta_bias != nullptr) ? (Acc)p.delta_bias[d] : (Acc)0;
    const bool soft = p.delta_softplus != 0;
    const int32_t row = (int32_t)(p.Dm * (int64_t)sizeof(T));
    const int32_t voff = (int32_t)((d - d0) * (int64_t)sizeof(T));

    Acc dAr[NH], dAi[NH];
#pragma unroll
    for (int k = 0; k < NH; ++k) dAr[k] = dAi[k] = 0;
    Acc dDacc = 0, dbacc = 0;

    // the block's dB/dC sums of the segment's steps, each over the tiles in
    // order (between two barriers)
    auto write_segment_sums = [&](int64_t t0, int nseg) {
        Acc *dst = static_cast<Acc *>(q.part_bc) + ((int64_t)br * 2) * BLN + (b * p.L + t0) * N;
        constexpr int kE = kT * 2 * N;
        for (int e = threadIdx.x; e < kE; e += kWaves * kWave) {
            const int i = e / (2 * N);
            const int v = (e / N) & 1;
            const int n = e % N;
            Acc sum = 0;
#pragma unroll
            for (int w = 0; w < kTiles; ++w) sum += bacc[w][i][v][n];
            if (i < nseg) dst[(int64_t)v * BLN + (int64_t)i * N + n] = sum;
        }
    };
    // the state entering segment s (this wave's states)
    auto load_entry = [&](int s, Acc(&er)[NH], Acc(&ei)[NH]) {
        if (s == 0) {
#pragma unroll
            for (int k = 0; k < NH; ++k) {
                er[k] = p.h_init ? (Acc)p.h_init[(ch * N + n0 + k) * 2] : (Acc)0;
                ei[k] = p.h_init ? (Acc)p.h_init[(ch * N + n0 + k) * 2 + 1] : (Acc)0;
            }
        } else {
            const Acc *gin = static_cast<const Acc *>(p.gin);
#pragma unroll
            for (int k = 0; k < NH; ++k) {
                er[k] = gin[((int64_t)s * 2 * N + 2 * (n0 + k)) * BD + ch];
                ei[k] = gin[((int64_t)s * 2 * N + 2 * (n0 + k) + 1) * BD + ch];
            }
        }
    };

    // the adjoint entering the group's last segment from the right
    Acc lr[NH], li[NH];
    {
        const Acc *gout = static_cast<const Acc *>(q.gout);
#pragma unroll
        for (int k = 0; k < NH; ++k) {
            lr[k] = gout[((int64_t)grp * 2 * N + 2 * (n0 + k)) * BD + ch];
            li[k] = gout[((int64_t)grp * 2 * N + 2 * (n0 + k) + 1) * BD + ch];
        }
    }
    for (int si = q.seg_per_group - 1; si >= 0; --si) {
        const int s = grp * q.seg_per_group + si;
        if (s >= p.S) continue;
        const int64_t t0 = (int64_t)s * kT;
        const int nseg = uniform((int)((t0 + kT < p.L ? t0 + kT : p.L) - t0));
        const int64_t off = (b * p.L + t0) * p.Dm + d0;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(static_cast<const T *>(p.x) + off, nseg * row);
        const __amdgpu_buffer_rsrc_t rdl = make_rsrc(static_cast<const T *>(p.delta) + off, nseg * row);
        const __amdgpu_buffer_rsrc_t rdy = make_rsrc(static_cast<const T *>(q.dy) + off, nseg * row);
        const __amdgpu_buffer_rsrc_t rdx = make_rsrc(static_cast<const T *>(q.dx) + off, nseg * row);
        const __amdgpu_buffer_rsrc_t rdd = make_rsrc(static_cast<const T *>(q.ddelta) + off, nseg * row);
        const_row_ptr<Acc> bcp = (const_row_ptr<Acc>)(static_cast<const Acc *>(p.bc) + (b * p.L + t0) * (2 * N));
        // raw x and delta of steps t0 + i, clamped into the segment
        auto load_xd = [&](int i, uint32_t &xv, uint32_t &dv) {
            const int so = (i < nseg ? i : nseg - 1) * row;
            xv = buf_load_raw<T>(rx, voff, so);
            dv = buf_load_raw<T>(rdl, voff, so);
        };
        auto dval = [&](uint32_t raw) {
            Acc v = (Acc)raw_to_f32<T>(raw);
            if constexpr (kPre) v = soft ? softplus_(v + bias) : v + bias;
            return v;
        };
        // d(delta) as passed from d(delta) as used, and the running sums
        auto finish_step = [&](int t, Acc gy, Acc xv, Acc dv, Acc gx, Acc gdt) {
            Acc gdl = gdt;
            if constexpr (kPre) {
                if (soft) gdl *= softplus_grad_from_value(dv);
            }
            dDacc = fma_(gy, xv, dDacc);
            dbacc += gdl;
            if (live) {
                buf_store(from_acc<T>(gx), rdx, voff, t * row);
                buf_store(from_acc<T>(gdl), rdd, voff, t * row);
            }
        };

        // checkpoints: the state before steps 4, 8, 12 of the segment (x and
        // delta of steps 0..11 are loaded for this pass only; each sub-chunk
        // loads its own again, from the cache)
        Acc hr[NH], hi[NH];
        uint32_t xr[kT - kK], dr[kT - kK];
#pragma unroll
        for (int i = 0; i < kT - kK; ++i) load_xd(i, xr[i], dr[i]);
        load_entry(s, hr, hi);
#pragma unroll
        for (int j = 1; j < kNck; ++j) {
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                const int t = (j - 1) * kK + i;
                if (t < nseg) {
                    Acc rw[2 * NH];
                    load_half_row<NH, N>(rw, bcp + (int64_t)t * (2 * N), n0);
                    cbwd_fwd_step<NH, kEuler>(cc, rw, (Acc)raw_to_f32<T>(xr[t]), dval(dr[t]), hr, hi);
                }
            }
#pragma unroll
            for (int k = 0; k < NH; ++k) {
                ck[wave][j - 1][2 * k][lane] = hr[k];
                ck[wave][j - 1][2 * k + 1][lane] = hi[k];
            }
        }

        // sub-chunks from the last to the first
#pragma unroll
        for (int u = kNck - 1; u >= 0; --u) {
            if (u * kK >= nseg) continue;
            // the sub-chunk's x, delta and dy
            uint32_t xs[kK], ds[kK], ys[kK];
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                const int t = u * kK + i;
                load_xd(t, xs[i], ds[i]);
                ys[i] = buf_load_raw<T>(rdy, voff, (t < nseg ? t : nseg - 1) * row);
            }
            auto xval = [&](int i) { return live ? (Acc)raw_to_f32<T>(xs[i]) : (Acc)0; };
            auto gval = [&](int i) { return live ? (Acc)raw_to_f32<T>(ys[i]) : (Acc)0; };
            // the entering state: its checkpoint, or for the first sub-chunk
            // the segment's entry state, read again and kept in the slot of
            // the state before step 4 (whose sub-chunk is done); each lane
            // reads back only what it wrote.  Then the states after each
            // step: complex but for the last step's (its real part only).
            const int ks = u > 0 ? u - 1 : 0;
            if (u > 0) {
#pragma unroll
                for (int k = 0; k < NH; ++k) {
                    hr[k] = ck[wave][ks][2 * k][lane];
                    hi[k] = ck[wave][ks][2 * k + 1][lane];
                }
            } else {
                load_entry(s, hr, hi);
#pragma unroll
                for (int k = 0; k < NH; ++k) {
                    ck[wave][ks][2 * k][lane] = hr[k];
                    ck[wave][ks][2 * k + 1][lane] = hi[k];
                }
            }
            Acc gsr[kK][NH], gsi[kK - 1][NH];
#pragma unroll
            for (int i = 0; i < kK; ++i) {
                const int t = u * kK + i;
                if (t < nseg) {
                    Acc rw[2 * NH];
                    load_half_row<NH, N>(rw, bcp + (int64_t)t * (2 * N), n0);
                    cbwd_fwd_step<NH, kEuler>(cc, rw, (Acc)raw_to_f32<T>(xs[i]), dval(ds[i]), hr, hi);
                }
#pragma unroll
                for (int k = 0; k < NH; ++k) {
                    gsr[i][k] = hr[k];
                    if (i + 1 < kK) gsi[i < kK - 1 ? i : 0][k] = hi[k];
                }
            }
            // back over the sub-chunk; this wave's shares of dx and d(delta)
            Acc px[kK], pg[kK];
#pragma unroll
            for (int i = kK - 1; i >= 0; --i) {
                px[i] = pg[i] = 0;
                const int t = u * kK + i;
                if (t < nseg) {
                    Acc rw[2 * NH];
                    load_half_row<NH, N>(rw, bcp + (int64_t)t * (2 * N), n0);
                    const Acc xv = xval(i), gy = gval(i);
                    // delta through an empty asm: the coefficients are formed
                    // again rather than kept in registers from the recompute
                    Acc dv = dval(ds[i]);
                    __asm__ volatile("" : "+v"(dv));
                    Acc ur, ui;
                    delta_units(dv, ur, ui);
                    Acc vB[NH], vC[NH];
                    Acc acc_x = 0, gdt = 0;
#pragma unroll
                    for (int n = 0; n < NH; ++n) {
                        const Acc hpr = i > 0 ? gsr[i > 0 ? i - 1 : 0][n] : ck[wave][ks][2 * n][lane];
                        const Acc hpi = i > 0 ? gsi[i > 0 ? i - 1 : 0][n] : ck[wave][ks][2 * n + 1][lane];
                        Acc abr, abi, kr, ki, er;
                        cplx_coef<NH, kEuler>(cc, n, dv, ur, ui, abr, abi, kr, ki, er);
                        // lambda: the adjoint of h_t (y reads its real part)
                        const Acc mr = fma_(rw[NH + n], gy, lr[n]), mi = li[n];
                        const Acc u_ = rw[n] * xv;
                        // G_Abar = lambda conj(h_{t-1}),  G_k = lambda u
                        const Acc gar = fma_(mr, hpr, mi * hpi), gai = fma_(mi, hpr, -mr * hpi);
                        const Acc gkr = mr * u_, gki = mi * u_;
                        // dL/du = Re(lambda conj(k))
                        const Acc gu = fma_(mr, kr, mi * ki);
                        acc_x = fma_(gu, rw[n], acc_x);
                        vB[n] = gu * xv;
                        vC[n] = gy * gsr[i][n];
                        // d(delta): Re(G_Abar conj(A Abar)) + Re(G_k conj(dk/ddelta))
                        const Acc par = cc.ar[n] * abr - cc.ai[n] * abi, pai = cc.ar[n] * abi + cc.ai[n] * abr;
                        gdt = fma_(gar, par, fma_(gai, pai, gdt));
                        if constexpr (kEuler)
                            gdt += gkr;
                        else
                            gdt = fma_(gkr, abr, fma_(gki, abi, gdt));
                        // dA: G_Abar conj(delta Abar) + G_k conj(dk/dA)
                        const Acc dar = dv * abr, dai = dv * abi;
                        dAr[n] = fma_(gar, dar, fma_(gai, dai, dAr[n]));
                        dAi[n] = fma_(gai, dar, fma_(-gar, dai, dAi[n]));
                        if constexpr (!kEuler) {
                            Acc qr, qi;
                            cplx_dk_da<NH>(cc, n, dv, abr, abi, er, kr, ki, qr, qi);
                            dAr[n] = fma_(gkr, qr, fma_(gki, qi, dAr[n]));
                            dAi[n] = fma_(gki, qr, fma_(-gkr, qi, dAi[n]));
                        }
                        // into step t-1: lambda conj(Abar)
                        lr[n] = fma_(mr, abr, mi * abi);
                        li[n] = fma_(mi, abr, -mr * abi);
                    }
                    if constexpr (P == 1) {
                        finish_step(t, gy, xv, dv, fma_(Dd, gy, acc_x), gdt);
                    } else {
                        px[i] = acc_x;
                        pg[i] = gdt;
                        if (half != 0) {
                            xb[u & 1][tb][i][0][lane] = acc_x;
                            xb[u & 1][tb][i][1][lane] = gdt;
                        }
                    }
                    const int idx = wave_reduce_scatter<NH>(vB, lane);
                    (void)wave_reduce_scatter<NH>(vC, lane);
                    if ((lane & (kWave / NH - 1)) == 0) {
                        bacc[tb][t][0][n0 + idx] = vB[0];
                        bacc[tb][t][1][n0 + idx] = vC[0];
                    }
                }
            }
            if constexpr (P > 1) {
                // the other waves' shares of the sub-chunk are in (the buffer
                // alternates, so it is not written again before the next barrier)
                __syncthreads();
                if (half == 0) {
#pragma unroll
                    for (int i = 0; i < kK; ++i) {
                        const int t = u * kK + i;
                        if (t < nseg) {
                            const Acc gy = gval(i);
                            const Acc gx = fma_(Dd, gy, px[i]) + xb[u & 1][tb][i][0][lane];
                            finish_step(t, gy, xval(i), dval(ds[i]), gx, pg[i] + xb[u & 1][tb][i][1][lane]);
                        }
                    }
                }
            }
        }
        __syncthreads();  // every tile's partials of the segment are in
        write_segment_sums(t0, nseg);
        __syncthreads();  // ... and summed before the next segment's are written
        if (s == 0 && live && q.dh_init != nullptr) {
#pragma unroll
            for (int k = 0; k < NH; ++k) {
                q.dh_init[(ch * N + n0 + k) * 2] = (float)lr[k];
                q.dh_init[(ch * N + n0 + k) * 2 + 1] = (float)li[k];
            }
        }
    }

    if (!live) return;
    Acc *pa = static_cast<Acc *>(q.part_a) + ((int64_t)grp * BD + ch) * 2 * N + 2 * n0;
#pragma unroll
    for (int k = 0; k < NH; ++k) {
        pa[2 * k] = dAr[k];
        pa[2 * k + 1] = dAi[k];
    }
    if (half == 0) {
        Acc *pd = static_cast<Acc *>(q.part_d) + ((int64_t)grp * BD + ch) * 2;
        pd[0] = dDacc;
        pd[1] = dbacc;
    }
}

// dB, dC: the block partials summed (one thread per (b, t, n)); dA, dD,
// d(delta_bias): sums over batch rows and groups (one thread per value).
template <typename Acc, int N>
__global__ __launch_bounds__(kBlock) void cbwd_reduce_kernel(BwdParams q) {
    const ScanParams &p = q.f;
    const int64_t BLN = p.Bsz * p.L * N;
    const int64_t DN2 = p.Dm * N * 2;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < BLN) {
        const Acc *src = static_cast<const Acc *>(q.part_bc);
        Acc sb = 0, sc = 0;
        for (int k = 0; k < q.blocks_per_row; ++k) {
            sb += src[((int64_t)k * 2) * BLN + i];
            sc += src[((int64_t)k * 2 + 1) * BLN + i];
        }
        q.dB[i] = (float)sb;
        q.dC[i] = (float)sc;
        return;
    }
    const int64_t j = i - BLN;
    // The partial rows are (group, batch row) pairs, row r = g * Bsz + b, summed
    // in that order with kBatch loads in flight before their adds.
    constexpr int kBatch = 16;
    const int64_t rows = (int64_t)q.n_groups * p.Bsz;
    auto sum_rows = [&](const Acc *src, int64_t stride, int64_t off) -> Acc {
        Acc sacc = 0;
        for (int64_t r0 = 0; r0 < rows; r0 += kBatch) {
            Acc v[kBatch];
#pragma unroll
            for (int k = 0; k < kBatch; ++k) v[k] = r0 + k < rows ? src[(r0 + k) * stride + off] : (Acc)0;
#pragma unroll
            for (int k = 0; k < kBatch; ++k) sacc += v[k];
        }
        return sacc;
    };
    if (j < DN2) {
        // part_a: [groups][Bsz * Dm][2N]
        q.dA[j] = (float)sum_rows(static_cast<const Acc *>(q.part_a), p.Dm * 2 * N, j);
        return;
    }
    const int64_t k = j - DN2;
    if (k >= 2 * p.Dm) return;
    const int64_t d = k % p.Dm;
    const int which = (int)(k / p.Dm);  // 0: dD, 1: d(delta_bias)
    float *dst = which == 0 ? q.dD : q.ddelta_bias;
    if (dst == nullptr) return;
    // part_d: [groups][Bsz * Dm][2]
    dst[d] = (float)sum_rows(static_cast<const Acc *>(q.part_d), p.Dm * 2, d * 2 + which);
}

template <typename T, int N, bool kEuler, bool kPre>
void cbwd_launch_variant(BwdPass pass, const BwdParams &q, hipStream_t s) {
    typedef typename AccOf<T>::type Acc;
    const ScanParams &p = q.f;
    if (pass == BwdPass::kAggregate) {
        const int bps = (p.n_tiles + p.waves_per_block - 1) / p.waves_per_block;
        if (p.S <= 1 || bps == 0) return;
        hipLaunchKernelGGL((cbwd_aggregate_kernel<T, N, kEuler, kPre>), dim3((unsigned)bps * p.S), dim3(kBlock), 0,
                           s, q);
    } else {
        const unsigned grid = (unsigned)(q.n_groups * p.Bsz * q.blocks_per_row);
        if (grid == 0) return;
        hipLaunchKernelGGL((cbwd_main_kernel<T, N, kEuler, kPre>), dim3(grid), dim3(CbwdShape<Acc>::kWaves * kWave),
                           0, s, q);
    }
}

template <typename T, int N>
hipError_t cbwd_pass_n(BwdPass pass, const BwdParams &q, hipStream_t s) {
    typedef typename AccOf<T>::type Acc;
    const ScanParams &p = q.f;
    const bool pre = p.delta_bias != nullptr || p.delta_softplus != 0;
    switch (pass) {
        case BwdPass::kStarts:
            break;
        case BwdPass::kAggregate:
        case BwdPass::kMain:
            if (p.euler_b) {
                if (pre)
                    cbwd_launch_variant<T, N, true, true>(pass, q, s);
                else
                    cbwd_launch_variant<T, N, true, false>(pass, q, s);
            } else {
                if (pre)
                    cbwd_launch_variant<T, N, false, true>(pass, q, s);
                else
                    cbwd_launch_variant<T, N, false, false>(pass, q, s);
            }
            break;
        case BwdPass::kCarry: {
            const int64_t work = p.Bsz * p.Dm * N;
            if (work == 0) return hipSuccess;
            hipLaunchKernelGGL((cbwd_carry_kernel<Acc, N>), dim3((unsigned)((work + kBlock - 1) / kBlock)),
                               dim3(kBlock), 0, s, q);
            break;
        }
        case BwdPass::kReduce: {
            const int64_t work = p.Bsz * p.L * N + p.Dm * N * 2 + 2 * p.Dm;
            if (work == 0) return hipSuccess;
            hipLaunchKernelGGL((cbwd_reduce_kernel<Acc, N>), dim3((unsigned)((work + kBlock - 1) / kBlock)),
                               dim3(kBlock), 0, s, q);
            break;
        }
    }
    return hipGetLastError();
}

template <typename T>
hipError_t cbwd_pass(BwdPass pass, const BwdParams &q, int N, hipStream_t s) {
    switch (N) {
        case 1: return cbwd_pass_n<T, 1>(pass, q, s);
        case 2: return cbwd_pass_n<T, 2>(pass, q, s);
        case 4: return cbwd_pass_n<T, 4>(pass, q, s);
        case 8: return cbwd_pass_n<T, 8>(pass, q, s);
        case 16: return cbwd_pass_n<T, 16>(pass, q, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

}  // namespace ssm
