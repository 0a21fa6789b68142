// Selective-scan kernels for gfx950 (CDNA4, wave64): templates shared by the
// per-(dtype, layout) translation units (scan_{bf16,f32}{,_packed}.hip).
//
// What is computed ("Mamba SSM Nedir?" page, sections "Ayrik Zamana Gecis"
// and "State Space Model Temelleri"): per batch row b, channel d, state n,
//   Abar = exp(delta_t A),  Bbar = (Abar - 1)/A * B_t[n],
//   h_t = Abar h_{t-1} + Bbar x_t,   y_t = sum_n C_t[n] h_t + D x_t.
// Options of the same recurrence:
//   * Euler input term (kEuler): Bbar = delta_t B_t[n], Abar unchanged (the
//     rule the bitig.info Mamba-3 page, section "Gelistirilmis Ayriklastirma
//     Semasi", attributes to Mamba-1 and -2).
//   * delta pre-processing (kPre): delta_t = softplus(raw_t + bias[d]) or
//     raw_t + bias[d], the activation of delta's projection ("Mamba SSM
//     Nedir?", section "Mamba'nin Yeniligi: Selective SSM"), applied as delta
//     is read, so the activated delta never goes through HBM.
//   * packed sequences (kVarlen, with ScanParams::cu): several sequences
//     along time in one row, the state restarting at each start.
//
// Layout of the work
//   * One lane owns one (b, d) channel and keeps all N states in VGPRs for the
//     whole time segment; the expanded [B, L, D, N] state never leaves the
//     register file (the pages' kernel keeps it in on-chip memory too).
//   * A wave covers 64 consecutive channels of one batch row, so B_t and C_t
//     are wave-uniform: they are read with scalar loads into SGPRs and enter
//     every FMA as the SGPR operand, costing no vector instructions.
//   * x_t, delta_t are read per lane (64 lanes = 128 contiguous bytes in bf16)
//     a few steps ahead, and y_t is written the same way.
//   * Time is cut into S segments so that the chip has enough waves.  The
//     segments are tied together with the composition of affine maps
//     (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2) -- the parallel prefix scan of
//     section "Paralel Tarama Algoritmasi" -- in three passes:
//       1. aggregate: every segment but the last runs from a zero state and
//          stores its end state and the sum of its delta;
//       2. carry: per (channel, state), a short sequential scan over segments
//          gives the state entering each segment;
//       3. output: every segment reruns from its true entering state and
//          writes y (and h_final for the last one).
//
// State representation.  Lanes carry g_n = (n+1) h_n.  Then (ZOH)
//   g_n <- g_n + E_n (g_n + B_t[n] x_t (n+1)/A_n),   E_n = exp(delta A_n) - 1,
//   y_t  = sum_n (C_t[n]/(n+1)) g_n + D x_t,
// which is the recurrence above rewritten (Abar h + (Abar-1)/A B x
// = h + (Abar-1)(h + B x / A)).  When A[d, n] == (n+1) A[d, 0] for every n
// (the S4D-real structure) the factor (n+1)/A_n is the per-channel constant
// 1/A[d,0] and E_{n+1} = (1 + E_n)(1 + E_1) - 1: one transcendental per
// (t, d) and four FMAs per state element.  Any other A takes the general path
// with one exp per state element.  With the Euler input term the update is
//   g_n <- g_n + E_n g_n + ((n+1) B_t[n]) (delta x_t),
// also four FMAs per element.
//
// Arithmetic: fp32 for bf16 storage; fp64 for fp32 storage (see AccOf).
#pragma once

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {

namespace {

constexpr int kBlock = 256;
constexpr int kPrefetch = 4;  // time steps of x/delta loaded ahead of use

// ---------------------------------------------------------------------------
// B/C rows -> arithmetic type, C pre-divided by (n+1) for the scaled state;
// with the Euler input term B is pre-multiplied by (n+1).

template <typename T, int N>
__global__ __launch_bounds__(kBlock) void bc_prep_kernel(const T *__restrict__ B,
                                                         const T *__restrict__ C,
                                                         typename AccOf<T>::type *__restrict__ bc,
                                                         int64_t rows, int euler) {
    typedef typename AccOf<T>::type Acc;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= rows * N) return;
    const int64_t r = i / N;
    const int n = (int)(i - r * N);
    const Acc bv = (Acc)to_f32(B[i]);
    bc[r * (2 * N) + n] = euler ? bv * (Acc)(n + 1) : bv;
    bc[r * (2 * N) + N + n] = (Acc)to_f32(C[i]) / (Acc)(n + 1);
}

// ---------------------------------------------------------------------------
// One time segment of one 64-channel tile.

// A of the general ZOH path: a tiny stand-in for A ~ 0 keeps (n+1)/A finite.
template <typename Acc>
__device__ __forceinline__ Acc zoh_a(float a) {
    return (__builtin_fabsf(a) < -kTinyA) ? (Acc)kTinyA : (Acc)a;
}

// Factor from the state the aggregate pass carries to the scaled state g:
// the ZOH aggregate passes carry j_n = g_n A_n / (n+1) (A[d,0] g_n on the
// structured path, where A_n = (n+1) A[d,0]), which turns the input term
// B x (n+1)/A_n into B x and saves a multiply per element.
template <int N, bool kStruct, bool kEuler, typename Acc>
__device__ __forceinline__ Acc agg_to_g(const float (&Ar)[N], int n) {
    if constexpr (kEuler) return (Acc)1;
    else if constexpr (kStruct) return (Acc)1 / (Acc)Ar[0];
    else return (Acc)(n + 1) / zoh_a<Acc>(Ar[n]);
}

// Per-channel constants of the update paths.  In fp32 the exponent arguments
// are kept in base-2 units (a2 = A log2 e) so that exp2 needs no scaling
// multiply; fp64 keeps natural units.
template <int N, bool kStruct, bool kEuler, typename Acc>
struct ChanConst {
    Acc a0, inva;       // structured: A[d,0] (base-2 units in fp32) and 1/A[d,0] (ZOH)
    Acc Aeff[N], W[N];  // general: A (base-2 units in fp32) and, for ZOH, (n+1)/A
    __device__ __forceinline__ explicit ChanConst(const float (&Ar)[N]) {
        constexpr Acc unit = sizeof(Acc) == 4 ? (Acc)kLog2e : (Acc)1;
        a0 = (Acc)Ar[0] * unit;
        inva = 0;
        if constexpr (kStruct) {
            if constexpr (!kEuler) inva = (Acc)1 / (Acc)Ar[0];
        } else {
#pragma unroll
            for (int n = 0; n < N; ++n) {
                if constexpr (kEuler) {
                    Aeff[n] = (Acc)Ar[n] * unit;  // no division by A: A = 0 is exact
                    W[n] = 0;
                } else {
                    const Acc ae = zoh_a<Acc>(Ar[n]);
                    Aeff[n] = ae * unit;
                    W[n] = (Acc)(n + 1) / ae;
                }
            }
        }
    }
};

// One time step of one channel: updates the scaled state g and returns
// sum_n (C_t[n]/(n+1)) g_n (kOut) -- D x is added by the caller.
// row = {B_t[n] (times n+1 for Euler), C_t[n]/(n+1)}, wave-uniform.
// kDirect (fp32 only): every lane's |delta A| is known to be at least 2^-13
// for every n, so exp(delta A) - 1 is the plain difference (no small-argument
// polynomial and select).
template <int N, bool kStruct, bool kOut, bool kEuler, typename Acc, bool kDirect = false>
__device__ __forceinline__ Acc scan_step(const ChanConst<N, kStruct, kEuler, Acc> &cc, const Acc (&row)[2 * N],
                                         Acc xv, Acc dv, Acc (&g)[N]) {
    constexpr bool direct = kDirect && sizeof(Acc) == 4;
    auto em1 = [](Acc z, Acc &e) -> Acc {
        if constexpr (direct)
            return expm1_direct_exp2(z, e);
        else
            return expm1_and_exp2(z, e);
    };
    Acc yv = 0;
    if constexpr (kStruct) {
        Acc r;
        const Acc E1 = em1(dv * cc.a0, r);
        // ZOH: the aggregate pass (no y) carries j = A[d,0] g instead of g,
        // which turns x/A[d,0] into x: j <- j + E_n (j + B_t[n] x).  The caller
        // rescales j once at the end of the segment (agg_to_g).
        const Acc xa = kEuler ? dv * xv : (kOut ? xv * cc.inva : xv);
        Acc E = E1;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            if constexpr (kEuler) {
                g[n] = fma_(row[n], xa, fma_(E, g[n], g[n]));
            } else {
                const Acc tt = fma_(row[n], xa, g[n]);
                g[n] = fma_(E, tt, g[n]);
            }
            if constexpr (kOut) yv = fma_(row[N + n], g[n], yv);
            // E_{n+1} = (1 + E_n)(1 + E_1) - 1.  fp32 uses the one-FMA form
            // with r = exp(delta A[d,0]); fp64 keeps E_1 unrounded
            // (E_n + E_1 + E_n E_1).
            if (n + 1 < N) {
                if constexpr (sizeof(Acc) == 8)
                    E = fma_(E, E1, E + E1);
                else
                    E = fma_(E, r, E1);
            }
        }
    } else {
        const Acc dx = dv * xv;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            Acc e;
            const Acc E = em1(dv * cc.Aeff[n], e);
            if constexpr (kEuler) {
                g[n] = fma_(row[n], dx, fma_(E, g[n], g[n]));
            } else {
                // the aggregate pass carries j_n = g_n A_n/(n+1) (agg_to_g)
                const Acc tt = fma_(row[n], kOut ? xv * cc.W[n] : xv, g[n]);
                g[n] = fma_(E, tt, g[n]);
            }
            if constexpr (kOut) yv = fma_(row[N + n], g[n], yv);
        }
    }
    return yv;
}

// B/C rows are read through the constant address space: the kernel never
// writes them, and telling the compiler so keeps them in scalar loads even
// though y leaves through buffer stores it cannot see through.
template <typename Acc>
using const_row_ptr = const __attribute__((address_space(4))) Acc *;

template <int N, typename Acc>
__device__ __forceinline__ void load_row(Acc (&dst)[2 * N], const_row_ptr<Acc> src) {
#pragma unroll
    for (int i = 0; i < 2 * N; ++i) dst[i] = src[i];
}

// Makes the row's scalar registers readable at this point (the wait for
// its load goes here).  One element suffices: the wait covers every
// outstanding scalar load.
template <typename Acc, int M>
__device__ __forceinline__ void row_ready(const Acc (&row)[M]) {
    __asm__ volatile("" ::"s"(row[0]));
}

// The x/delta/y streams of one 64-channel tile over a run of steps: buffer
// descriptors based at (b, t, d0), a per-lane byte offset and the byte stride
// of one time step.  All offsets are 32-bit (the planner keeps a segment's
// span below 1 GiB) and out-of-range accesses are dropped by the
// descriptors' range check.
template <typename T>
struct SegIO {
    __amdgpu_buffer_rsrc_t x, dl, y;
    int32_t voff;  // lane byte offset within a step (0 for idle lanes)
    int32_t row;   // bytes per time step (Dm * sizeof(T))
};

// delta as the recurrence uses it, from the stored value: + bias[d], then
// softplus if asked (kPre); the stored value itself otherwise.
template <typename Acc>
struct DeltaPre {
    Acc bias;
    bool softplus;
};

template <typename T, int N, bool kStruct, bool kOut, bool kEuler, bool kPre, bool kDirect, typename Acc>
__device__ __forceinline__ void run_group(const SegIO<T> &io, const_row_ptr<Acc> bcp, int tb, int nsteps,
                                          const T (&xs)[kPrefetch], const T (&ds)[kPrefetch],
                                          const ChanConst<N, kStruct, kEuler, Acc> &cc, Acc Dd,
                                          const DeltaPre<Acc> &dp, Acc (&g)[N], Acc &lam,
                                          Acc (&rowa)[2 * N], Acc (&rowb)[2 * N]) {
    static_assert(kPrefetch % 2 == 0, "the B/C row buffers alternate within a group");
    const int last = nsteps - 1;
    const bool full = tb + kPrefetch <= nsteps;
    Acc dpre[kPrefetch];
    if constexpr (kPre) {
        // the whole group at once: one uniform branch per kPrefetch steps
        if (dp.softplus) {
#pragma unroll
            for (int k = 0; k < kPrefetch; ++k) dpre[k] = softplus_(to_f32(ds[k]) + dp.bias);
        } else {
#pragma unroll
            for (int k = 0; k < kPrefetch; ++k) dpre[k] = (Acc)to_f32(ds[k]) + dp.bias;
        }
    }
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
        if (full || tb + k < nsteps) {
            // step k uses one buffer while the next step's row lands in the
            // other, so the scalar load has a whole step to arrive (a copy
            // from a "next" into a "current" buffer would wait for it at the
            // end of the step instead)
            Acc(&cur)[2 * N] = (k & 1) ? rowb : rowa;
            Acc(&nxt)[2 * N] = (k & 1) ? rowa : rowb;
            const int tn = tb + k + 1;
            // Scalar loads can complete out of order, so any wait for one
            // waits for all: take this step's row first, then issue the next
            // one, which then has the whole step to arrive.  (Left alone the
            // scheduler puts the load at the end of the step, just before the
            // wait.)
            row_ready(cur);
            load_row<N>(nxt, bcp + (int64_t)(tn < last ? tn : last) * (2 * N));
            __builtin_amdgcn_sched_barrier(0);
            const Acc xv = (Acc)to_f32(xs[k]);
            const Acc dv = kPre ? dpre[k] : (Acc)to_f32(ds[k]);
            const Acc yv = scan_step<N, kStruct, kOut, kEuler, Acc, kDirect>(cc, cur, xv, dv, g);
            if constexpr (kOut) {
                buf_store<kBufNt>(from_acc<T>(fma_(Dd, xv, yv)), io.y, io.voff, (tb + k) * io.row);
            } else {
                lam += dv;
            }
        }
    }
}

template <typename T>
__device__ __forceinline__ void load_group(const SegIO<T> &io, int tb, int last, T (&xs)[kPrefetch],
                                           T (&ds)[kPrefetch]) {
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
        const int t = tb + k;
        const int so = (t < last ? t : last) * io.row;
        xs[k] = buf_load<T, kBufNt>(io.x, io.voff, so);
        ds[k] = buf_load<T, kBufNt>(io.dl, io.voff, so);
    }
}

// Runs `nsteps` (>= 1) time steps.  x/delta are fetched one group of
// kPrefetch steps ahead into alternating register sets (indices clamped into
// the run); the B/C row of the next step is fetched while the current one is
// computed.  Idle lanes of a partial tile shadow a valid channel: they compute
// exactly what that channel's lane computes and store the identical value.
template <typename T, int N, bool kStruct, bool kOut, bool kEuler, bool kPre, typename Acc, bool kDirect = false>
__device__ __forceinline__ void run_segment(const SegIO<T> &io, const_row_ptr<Acc> bcp, int nsteps,
                                            const float (&Ar)[N], Acc Dd, const DeltaPre<Acc> &dp,
                                            Acc (&g)[N], Acc &lam) {
    const ChanConst<N, kStruct, kEuler, Acc> cc(Ar);
    const int last = nsteps - 1;
    T xa[kPrefetch], da[kPrefetch], xb[kPrefetch], db[kPrefetch];
    load_group(io, 0, last, xa, da);
    Acc rowa[2 * N], rowb[2 * N];
    load_row<N>(rowa, bcp);
    for (int tb = 0; tb < nsteps; tb += 2 * kPrefetch) {
        load_group(io, tb + kPrefetch, last, xb, db);
        run_group<T, N, kStruct, kOut, kEuler, kPre, kDirect>(io, bcp, tb, nsteps, xa, da, cc, Dd, dp, g, lam, rowa,
                                                              rowb);
        if (tb + kPrefetch >= nsteps) break;
        load_group(io, tb + 2 * kPrefetch, last, xa, da);
        run_group<T, N, kStruct, kOut, kEuler, kPre, kDirect>(io, bcp, tb + kPrefetch, nsteps, xb, db, cc, Dd, dp, g,
                                                              lam, rowa, rowb);
    }
}

// One run of steps with the choice of exp(delta A) - 1 made once for the
// run (fp32 only): the plain difference when `direct`.
template <typename T, int N, bool kStruct, bool kOut, bool kEuler, bool kPre, typename Acc>
__device__ __forceinline__ void run_segment_choose(bool direct, const SegIO<T> &io, const_row_ptr<Acc> bcp,
                                                   int nsteps, const float (&Ar)[N], Acc Dd,
                                                   const DeltaPre<Acc> &dp, Acc (&g)[N], Acc &lam) {
    if constexpr (sizeof(Acc) == 4) {
        if (direct) {
            run_segment<T, N, kStruct, kOut, kEuler, kPre, Acc, true>(io, bcp, nsteps, Ar, Dd, dp, g, lam);
            return;
        }
    }
    run_segment<T, N, kStruct, kOut, kEuler, kPre, Acc, false>(io, bcp, nsteps, Ar, Dd, dp, g, lam);
}

// Smallest |delta| a wave's lanes meet in steps [0, nsteps) of a run (8
// loads in flight; steps past the run repeat the last one).
template <typename T>
__device__ __forceinline__ float run_min_delta(const SegIO<T> &io, int nsteps) {
    constexpr int kLoads = 8;
    float m = 3.0e38f;
    for (int t = 0; t < nsteps; t += kLoads) {
        uint32_t v[kLoads];
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            const int tk = t + k < nsteps ? t + k : nsteps - 1;
            v[k] = buf_load_raw<T>(io.dl, io.voff, tk * io.row);
        }
#pragma unroll
        for (int k = 0; k < kLoads; ++k) m = __builtin_fminf(m, __builtin_fabsf(raw_to_f32<T>(v[k])));
    }
    return m;
}

// The x/delta/y streams and B/C rows of steps [t, t + n) of batch row b for
// the 64-channel tile at d0 (lane channel d).
template <typename T, typename Acc, int N, bool kOut>
__device__ __forceinline__ SegIO<T> seg_io(const ScanParams &p, int64_t b, int64_t t, int n, int64_t d0,
                                           int64_t d, const_row_ptr<Acc> &bcp) {
    const int64_t off = (b * p.L + t) * p.Dm + d0;
    const int32_t row = (int32_t)(p.Dm * (int64_t)sizeof(T));
    const int32_t span = n * row;
    SegIO<T> io;
    io.x = make_rsrc(static_cast<const T *>(p.x) + off, span);
    io.dl = make_rsrc(static_cast<const T *>(p.delta) + off, span);
    io.y = make_rsrc(kOut ? static_cast<const T *>(p.y) + off : static_cast<const T *>(p.x) + off, kOut ? span : 0);
    io.voff = (int32_t)((d - d0) * (int64_t)sizeof(T));
    io.row = row;
    bcp = (const_row_ptr<Acc>)(static_cast<const Acc *>(p.bc) + (b * p.L + t) * (2 * N));
    return io;
}

// Packed variable-length input: the wave-uniform position in the list of
// sequences.  A sequence starts at cu[k] and ends at cu[k+1] - 1.
struct SeqTrack {
    const_row_ptr<int64_t> cu;  // constant address space: scalar loads
    int64_t nseq;
    int64_t next_start;  // absolute step at which the state restarts next
    int64_t cur;         // current sequence
};

// Largest k in [0, nseq) with cu[k] <= t (the sequence that holds step t,
// skipping empty ones).  Always returns an index in range.
__device__ __forceinline__ int64_t find_seq(const_row_ptr<int64_t> cu, int64_t nseq, int64_t t) {
    int64_t lo = 0, hi = nseq - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Position at the first step t0 of a segment.  If a sequence starts exactly at
// t0, next_start = t0 so that the state restarts before the first step.
__device__ __forceinline__ void seq_begin(SeqTrack &sq, int64_t t0) {
    sq.cur = find_seq(sq.cu, sq.nseq, t0);
    const int64_t start = sq.cu[sq.cur];
    sq.next_start = start == t0 ? t0 : sq.cu[sq.cur + 1];
}

// At step t == sq.next_start: move to the sequence starting at t (skipping
// empty ones) and return its index.
__device__ __forceinline__ int64_t seq_advance(SeqTrack &sq, int64_t t) {
    int64_t k = sq.cur;
    if (sq.cu[k] != t) ++k;
    while (k + 1 < sq.nseq && sq.cu[k + 1] <= t) ++k;
    if (k >= sq.nseq) k = sq.nseq - 1;
    sq.cur = k;
    sq.next_start = sq.cu[k + 1];
    return k;
}

// kOut = false: aggregate pass over segments 0..S-2.
// kOut = true : output pass over segments 0..S-1.
// kStruct selects the waves this launch serves: a wave whose 64 channels all
// have A[d, n] == (n+1) A[d, 0] (and the structured path is allowed) is served
// by the kStruct = true launch, every other wave by the kStruct = false one.
// Keeping the two paths in separate kernels keeps the structured kernel's
// register count (and so its occupancy) free of the general path's.
// kVarlen: packed sequences (ScanParams::cu is set).  A template parameter
// rather than a run-time test so the dense kernels carry none of its code.
template <typename T, int N, bool kOut, bool kStruct, bool kEuler, bool kPre, bool kVarlen>
__global__ __launch_bounds__(kBlock) void scan_segment_kernel(ScanParams p) {
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
    const int64_t d = active ? d0 + lane : d0;  // idle lanes shadow a valid channel
    const int64_t ch = b * p.Dm + d;
    const int64_t BD = p.Bsz * p.Dm;
    const int64_t t0 = (int64_t)s * p.seg_len;
    const int nsteps = uniform((int)((t0 + p.seg_len < p.L ? t0 + p.seg_len : p.L) - t0));
    constexpr bool varlen = kVarlen;

    float Ar[N];
#pragma unroll
    for (int n = 0; n < N; ++n) Ar[n] = p.A[d * N + n];
    bool st = (Ar[0] != 0.f) && (p.force_general == 0);
#pragma unroll
    for (int n = 1; n < N; ++n) st = st && (Ar[n] == (float)(n + 1) * Ar[0]);
    if ((bool)__all(st) != kStruct) return;
    const Acc Dd = (Acc)p.D[d];
    DeltaPre<Acc> dp;
    dp.bias = (kPre && p.delta_bias != nullptr) ? (Acc)p.delta_bias[d] : (Acc)0;
    dp.softplus = p.delta_softplus != 0;

    // Entering state: from the carry pass when time is split (it also holds
    // segment 0's, so h_init is never read here while the last segment may be
    // writing h_final into the same buffer); else h_init read by this lane
    // (packed sequences restart from their own h_init below).
    const Acc *gin = static_cast<const Acc *>(p.gin);
    Acc g[N];
    if (kOut && p.S > 1) {
#pragma unroll
        for (int n = 0; n < N; ++n) g[n] = gin[((int64_t)s * N + n) * BD + ch];
    } else if (kOut && p.h_init != nullptr && !varlen) {
#pragma unroll
        for (int n = 0; n < N; ++n) g[n] = (Acc)p.h_init[ch * N + n] * (Acc)(n + 1);
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) g[n] = 0;
    }

    // General path, fp32 arithmetic, delta as stored: a pre-scan of the
    // segment's delta decides, for the whole wave and segment, whether every
    // |delta A_n| is at least 2^-13, which lets exp(delta A_n) - 1 be the plain
    // difference (the per-element small-argument polynomial and select are
    // about 40% of that loop's instructions).
    bool direct = false;
    if constexpr (!kStruct && !kPre && sizeof(Acc) == 4) {
        float amin = __builtin_fabsf(kEuler ? Ar[0] : zoh_a<float>(Ar[0]));
#pragma unroll
        for (int n = 1; n < N; ++n) amin = __builtin_fminf(amin, __builtin_fabsf(kEuler ? Ar[n] : zoh_a<float>(Ar[n])));
        const_row_ptr<Acc> bcp_unused;
        const SegIO<T> io = seg_io<T, Acc, N, kOut>(p, b, t0, nsteps, d0, d, bcp_unused);
        const float dmin = run_min_delta<T>(io, nsteps);
        direct = __all(dmin * (amin * kLog2e) >= kExpm1DirectZ2);
    }
    Acc lam = 0;
    if constexpr (!varlen) {
        const_row_ptr<Acc> bcp;
        const SegIO<T> io = seg_io<T, Acc, N, kOut>(p, b, t0, nsteps, d0, d, bcp);
        run_segment_choose<T, N, kStruct, kOut, kEuler, kPre>(direct, io, bcp, nsteps, Ar, Dd, dp, g, lam);
    } else {
        // Packed sequences: the segment is cut at every sequence start; each
        // piece runs the plain loop, and between pieces the state restarts from
        // the next sequence's h_init (or zero).
        SeqTrack sq;
        sq.cu = (const_row_ptr<int64_t>)p.cu;
        sq.nseq = p.nseq;
        seq_begin(sq, t0);
        const int64_t t_end = t0 + nsteps;
        bool reset = false;
        int64_t t = t0;
        while (t < t_end) {
            if (t == sq.next_start) {
                const int64_t k = seq_advance(sq, t);
                reset = true;
                // the aggregate pass carries g / agg_to_g
                if (p.h_init != nullptr) {
                    const float *hi = p.h_init + (k * p.Dm + d) * N;
#pragma unroll
                    for (int n = 0; n < N; ++n) {
                        const Acc gn = (Acc)hi[n] * (Acc)(n + 1);
                        g[n] = kOut ? gn : gn / agg_to_g<N, kStruct, kEuler, Acc>(Ar, n);
                    }
                } else {
#pragma unroll
                    for (int n = 0; n < N; ++n) g[n] = 0;
                }
            }
            int64_t piece_end = sq.next_start < t_end ? sq.next_start : t_end;
            if (piece_end <= t) piece_end = t + 1;  // offsets that are not increasing: still progress
            const int n = uniform((int)(piece_end - t));
            const_row_ptr<Acc> bcp;
            const SegIO<T> io = seg_io<T, Acc, N, kOut>(p, b, t, n, d0, d, bcp);
            run_segment_choose<T, N, kStruct, kOut, kEuler, kPre>(direct, io, bcp, n, Ar, Dd, dp, g, lam);
            if constexpr (kOut) {
                // the current sequence ends with this piece
                if (piece_end == sq.next_start && p.h_final != nullptr && active) {
                    float *hf = p.h_final + (sq.cur * p.Dm + d) * N;
#pragma unroll
                    for (int n2 = 0; n2 < N; ++n2) hf[n2] = (float)(g[n2] / (Acc)(n2 + 1));
                }
            }
            t = piece_end;
        }
        if constexpr (!kOut) {
            // one flag per segment for the carry pass: the incoming state does
            // not survive a restart inside the segment
            if (tile == 0 && lane == 0) p.seg_reset[s] = reset ? 1 : 0;
        }
    }

    if (!active) return;
    if constexpr (!kOut) {
        if constexpr (!kEuler) {
#pragma unroll
            for (int n = 0; n < N; ++n) g[n] *= agg_to_g<N, kStruct, kEuler, Acc>(Ar, n);
        }
        Acc *a = static_cast<Acc *>(p.agg) + (int64_t)s * (N + 1) * BD + ch;
#pragma unroll
        for (int n = 0; n < N; ++n) a[(int64_t)n * BD] = g[n];
        a[(int64_t)N * BD] = lam;
    } else {
        if (!kVarlen && s == p.S - 1 && p.h_final != nullptr) {
#pragma unroll
            for (int n = 0; n < N; ++n) p.h_final[ch * N + n] = (float)(g[n] / (Acc)(n + 1));
        }
    }
}

// ---------------------------------------------------------------------------
// Carry between segments: one thread per (state n, channel).  Entering state
// of segment s+1 = exp(A_n * sum(delta over s)) * entering state of s + local
// end state of s; segment 0 enters with h_init (or zero).  Abar is exp(delta
// A) under both input rules, so the decay of a segment only needs its delta sum.

template <typename Acc, int N>
__global__ __launch_bounds__(kBlock) void scan_carry_kernel(ScanParams p) {
    constexpr int kBatch = 32;  // segments whose summaries are fetched together
    const int64_t BD = p.Bsz * p.Dm;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= BD * N) return;
    const int n = (int)(i / BD);
    const int64_t ch = i - (int64_t)n * BD;
    const int64_t d = ch % p.Dm;
    constexpr Acc unit = sizeof(Acc) == 4 ? (Acc)kLog2e : (Acc)1;
    const Acc a = (Acc)p.A[d * N + n] * unit;
    Acc carry = (p.h_init && p.cu == nullptr) ? (Acc)p.h_init[ch * N + n] * (Acc)(n + 1) : (Acc)0;
    const Acc *__restrict__ lam = static_cast<const Acc *>(p.agg) + (int64_t)N * BD + ch;
    const Acc *__restrict__ gl = static_cast<const Acc *>(p.agg) + (int64_t)n * BD + ch;
    Acc *__restrict__ out = static_cast<Acc *>(p.gin) + (int64_t)n * BD + ch;
    const int64_t sa = (int64_t)(N + 1) * BD, sg = (int64_t)N * BD;
    out[0] = carry;
    const int nseg = p.S - 1;
    if (nseg <= 0) return;
    // The summaries of the next batch are in flight while the current batch's
    // FMA chain runs; the decay factors do not depend on the carry.
    Acc lc[kBatch], gc[kBatch], ln[kBatch], gn[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
        const int s = k < nseg ? k : nseg - 1;
        lc[k] = lam[s * sa];
        gc[k] = gl[s * sa];
    }
    for (int s0 = 0; s0 < nseg; s0 += kBatch) {
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int s = (s0 + kBatch + k < nseg) ? s0 + kBatch + k : nseg - 1;
            ln[k] = lam[s * sa];
            gn[k] = gl[s * sa];
        }
        bool cut[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            lc[k] = exp_units(a * lc[k]);
            // a sequence restart inside segment s cuts the incoming state off
            // (selected rather than multiplied by 0, so an inf or NaN state of
            // an earlier sequence cannot leak into the next one)
            cut[k] = p.cu != nullptr && s0 + k < nseg && p.seg_reset[s0 + k] != 0;
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (s0 + k < nseg) {
                carry = cut[k] ? gc[k] : fma_(lc[k], carry, gc[k]);
                out[(int64_t)(s0 + k + 1) * sg] = carry;
            }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            lc[k] = ln[k];
            gc[k] = gn[k];
        }
    }
}

template <typename T, int N, bool kOut, bool kEuler, bool kPre, bool kVarlen>
void launch_both_paths(const ScanParams &p, unsigned grid, hipStream_t s) {
    // Both A paths are launched; each wave runs in exactly one of them.
    hipLaunchKernelGGL((scan_segment_kernel<T, N, kOut, true, kEuler, kPre, kVarlen>), dim3(grid), dim3(kBlock), 0,
                       s, p);
    hipLaunchKernelGGL((scan_segment_kernel<T, N, kOut, false, kEuler, kPre, kVarlen>), dim3(grid), dim3(kBlock), 0,
                       s, p);
}

template <typename T, int N, bool kOut, bool kVarlen>
void launch_variant(const ScanParams &p, unsigned grid, hipStream_t s) {
    const bool pre = p.delta_bias != nullptr || p.delta_softplus != 0;
    if (p.euler_b) {
        if (pre)
            launch_both_paths<T, N, kOut, true, true, kVarlen>(p, grid, s);
        else
            launch_both_paths<T, N, kOut, true, false, kVarlen>(p, grid, s);
    } else {
        if (pre)
            launch_both_paths<T, N, kOut, false, true, kVarlen>(p, grid, s);
        else
            launch_both_paths<T, N, kOut, false, false, kVarlen>(p, grid, s);
    }
}

template <typename T, int N, bool kVarlen>
struct ByN {
    typedef typename AccOf<T>::type Acc;
    static hipError_t prep(const ScanParams &p, hipStream_t s) {
        const int64_t rows = p.Bsz * p.L;
        const int64_t work = rows * N;
        if (work == 0) return hipSuccess;
        const unsigned grid = (unsigned)((work + kBlock - 1) / kBlock);
        hipLaunchKernelGGL((bc_prep_kernel<T, N>), dim3(grid), dim3(kBlock), 0, s, static_cast<const T *>(p.B),
                           static_cast<const T *>(p.C), static_cast<Acc *>(p.bc), rows, p.euler_b);
        return hipGetLastError();
    }
    static hipError_t segments(const ScanParams &p, bool out, hipStream_t s) {
        const int bps = (p.n_tiles + p.waves_per_block - 1) / p.waves_per_block;
        const int nseg = out ? p.S : p.S - 1;
        if (nseg <= 0 || bps == 0) return hipSuccess;
        const unsigned grid = (unsigned)bps * (unsigned)nseg;
        if (out)
            launch_variant<T, N, true, kVarlen>(p, grid, s);
        else
            launch_variant<T, N, false, kVarlen>(p, grid, s);
        return hipGetLastError();
    }
    static hipError_t carry(const ScanParams &p, hipStream_t s) {
        const int64_t work = p.Bsz * p.Dm * N;
        if (work == 0 || p.S <= 1) return hipSuccess;
        const unsigned grid = (unsigned)((work + kBlock - 1) / kBlock);
        hipLaunchKernelGGL((scan_carry_kernel<Acc, N>), dim3(grid), dim3(kBlock), 0, s, p);
        return hipGetLastError();
    }
};

// Every pass of a scan for storage type T; kVarlen must match p.cu != nullptr.
template <typename T, bool kVarlen>
hipError_t scan_pass(ScanPass pass, const ScanParams &p, int N, hipStream_t s) {
    auto run = [&](auto k) -> hipError_t {
        typedef decltype(k) K;
        switch (pass) {
            case ScanPass::kPrep: return K::prep(p, s);
            case ScanPass::kAggregate: return K::segments(p, false, s);
            case ScanPass::kCarry: return K::carry(p, s);
            case ScanPass::kOutput: return K::segments(p, true, s);
        }
        return hipErrorInvalidValue;
    };
    switch (N) {
        case 1: return run(ByN<T, 1, kVarlen>());
        case 2: return run(ByN<T, 2, kVarlen>());
        case 4: return run(ByN<T, 4, kVarlen>());
        case 8: return run(ByN<T, 8, kVarlen>());
        case 16: return run(ByN<T, 16, kVarlen>());
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

}  // namespace ssm
