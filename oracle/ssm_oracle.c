/*
 * Reference oracle for the selective state-space scan -- TEST INFRASTRUCTURE.
 *
 * This file is a plain, slow, sequential fp64 implementation of what the
 * selective-scan hot path computes.  Only the test-suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load it.  It shares no code,
 * header, constant or helper with the HIP library and must never be used as a
 * fallback for it.
 *
 * What it follows (page = "Mamba SSM Nedir? Transformer Alternatifi Rehberi",
 * yapayzekasozluk.tr):
 *   - section "State Space Model Temelleri", continuous model with the D
 *     feed-through term:  h'(t) = A h(t) + B x(t),  y(t) = C h(t) + D x(t).
 *   - section "Ayrik Zamana Gecis", zero-order-hold discretisation:
 *       Abar = exp(delta*A),  Bbar = (delta*A)^-1 (exp(delta*A) - I) delta*B,
 *     and the recurrence  h_t = Abar h_{t-1} + Bbar x_t,  y_t = C h_t.
 *   - section "Mamba'nin Yeniligi: Selective SSM": B_t, C_t and delta_t are
 *     given per token (they are inputs here, produced upstream).
 * The same recurrence is stated on "Mamba: Transformer'a Meydan Okuyan
 * Uzun-Bagimli Model" (matematikkaravani.com), section "Eski fikrin geri
 * donusu: durum uzayi".
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - A is diagonal and real, stored as A[d][n]; the matrix ZOH formula is
 *     then elementwise:  Bbar[n] = delta * phi(delta*A[d][n]) * B[n] with
 *     phi(z) = (exp(z)-1)/z and phi(0) = 1 (the limit, which also covers
 *     A == 0 and delta == 0).
 *   - B_t and C_t are shared by all channels d of a batch row; delta_t and x_t
 *     are per channel.
 *   - y_t uses the updated state h_t, plus D[d]*x_t[d].
 *   - initial state h_{-1} = h0 if given, else 0.
 *
 * Optional variants (flags of the entry points):
 *   - ORACLE_DELTA_SOFTPLUS: the step size is produced from a raw value as
 *     delta = softplus(raw + bias[d]), the activation the "Mamba SSM Nedir?"
 *     page gives for delta in section "Mamba'nin Yeniligi: Selective SSM"
 *     (softplus of a linear projection; bias[d] is that projection's bias).
 *     Without the flag delta = raw + bias[d] (bias NULL means 0).
 *   - ORACLE_EULER_B: the input term is discretised with the Euler rule,
 *     Bbar = delta * B, while Abar stays exp(delta*A).  The bitig.info page
 *     on Mamba-3 (section "Gelistirilmis Ayriklastirma Semasi") says Mamba-1
 *     and -2 discretised with Euler's method; Bbar = delta*B is also the
 *     A -> 0 limit of the ZOH input term.
 *
 * Layouts (row-major, contiguous):
 *   scan:  x, delta, y : [Bsz][L][Dm]      B, C : [Bsz][L][N]
 *          A : [Dm][N]     D, bias : [Dm]   h0, h_final : [Bsz][Dm][N]
 *   step:  x, delta, y : [Bsz][Dm]          B, C : [Bsz][N]
 *          A : [Dm][N]     D, bias : [Dm]   h : [Bsz][Dm][N] (in/out)
 *
 * All arithmetic is IEEE double with libm exp/expm1; build without
 * -ffast-math.
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_DELTA_SOFTPLUS 1
#define ORACLE_EULER_B 2

/* softplus(v) = log(1 + exp(v)), in a form that neither overflows for large v
 * nor loses the tail exp(v) for very negative v. */
static double softplus(double v)
{
    if (v > 0.0)
        return v + log1p(exp(-v));
    return log1p(exp(v));
}

/* The step size the recurrence uses. */
static double step_size(double raw, double bias, int flags)
{
    const double v = raw + bias;
    return (flags & ORACLE_DELTA_SOFTPLUS) ? softplus(v) : v;
}

/* phi(z) = (exp(z) - 1) / z, with its limit 1 at z = 0. */
static double zoh_phi(double z)
{
    if (z == 0.0)
        return 1.0;
    return expm1(z) / z;
}

/* One recurrence step for a single channel: updates h[0..N) in place and
 * returns y.  a: A[d][*], b/c: B_t[*], C_t[*]. */
static double channel_step(double *h, double xt, double dt, const double *a,
                           const double *b, const double *c, double dskip,
                           int64_t N, int euler)
{
    double y = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        const double z = dt * a[n];
        const double abar = exp(z);
        double bbar;
        if (euler)
            bbar = dt * b[n];
        else
            bbar = dt * zoh_phi(z) * b[n];
        h[n] = abar * h[n] + bbar * xt;
        y += c[n] * h[n];
    }
    return y + dskip * xt;
}

int ssm_oracle_scan(const double *x, const double *delta, const double *bias,
                    const double *A, const double *B, const double *C,
                    const double *D, const double *h0, double *y,
                    double *h_final, int64_t Bsz, int64_t L, int64_t Dm,
                    int64_t N, int flags, int nthreads)
{
    if (Bsz < 0 || L < 0 || Dm < 0 || N <= 0)
        return 1;
    const int euler = (flags & ORACLE_EULER_B) != 0;
    const int64_t nchan = Bsz * Dm;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int err = 0;
#pragma omp parallel
    {
        double *h = (double *)malloc((size_t)N * sizeof(double));
        if (!h) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t ch = 0; ch < nchan; ++ch) {
                const int64_t b = ch / Dm, d = ch % Dm;
                const double bias_d = bias ? bias[d] : 0.0;
                for (int64_t n = 0; n < N; ++n)
                    h[n] = h0 ? h0[(b * Dm + d) * N + n] : 0.0;
                for (int64_t t = 0; t < L; ++t) {
                    const int64_t i = (b * L + t) * Dm + d;
                    const int64_t r = (b * L + t) * N;
                    const double dt = step_size(delta[i], bias_d, flags);
                    y[i] = channel_step(h, x[i], dt, A + d * N, B + r,
                                        C + r, D[d], N, euler);
                }
                if (h_final)
                    for (int64_t n = 0; n < N; ++n)
                        h_final[(b * Dm + d) * N + n] = h[n];
            }
            free(h);
        }
    }
    return err;
}

int ssm_oracle_step(const double *x, const double *delta, const double *bias,
                    const double *A, const double *B, const double *C,
                    const double *D, double *h, double *y, int64_t Bsz,
                    int64_t Dm, int64_t N, int flags)
{
    if (Bsz < 0 || Dm < 0 || N <= 0)
        return 1;
    const int euler = (flags & ORACLE_EULER_B) != 0;
    for (int64_t b = 0; b < Bsz; ++b)
        for (int64_t d = 0; d < Dm; ++d) {
            const int64_t i = b * Dm + d;
            const double dt = step_size(delta[i], bias ? bias[d] : 0.0, flags);
            y[i] = channel_step(h + i * N, x[i], dt, A + d * N,
                                B + b * N, C + b * N, D[d], N, euler);
        }
    return 0;
}

/* ------------------------------------------------------------------------
 * Backward (reverse-mode derivative) of the scan.
 *
 * With lambda_t = dL/dh_t (all of h_t's later uses), the recurrence
 * h_t = Abar_t h_{t-1} + k_t B_t x_t  (k_t = delta phi(delta A), or delta for
 * the Euler term) and y_t = sum_n C_t h_t + D x_t give, going back in time:
 *   lambda_t  = C_t dy_t + Abar_{t+1} lambda_{t+1}  (lambda_{L-1} includes dL/dh_final)
 *   dx_t      = D dy_t + sum_n lambda_t k_t B_t
 *   dB_t[n]   = sum_d lambda_t k_t x_t           dC_t[n] = sum_d dy_t h_t
 *   ddelta_t  = sum_n lambda_t (A Abar_t h_{t-1} + dk/ddelta B_t x_t)
 *   dA[d][n]  = sum_{b,t} lambda_t (delta Abar_t h_{t-1} + dk/dA B_t x_t)
 *   dD[d]     = sum_{b,t} dy_t x_t               dh0 = Abar_0 lambda_0
 * with dk/ddelta = Abar (ZOH) or 1 (Euler) and dk/dA = delta^2 phi'(delta A)
 * (ZOH) or 0 (Euler).  With the softplus flag, ddelta is taken back through
 * softplus to the raw input (times sigmoid(raw + bias)); dbias[d] sums it.
 * This is the chain rule applied to the recurrence the forward follows; it is
 * pinned against finite differences of the forward oracle.
 * ---------------------------------------------------------------------- */

/* phi'(z) = (z e^z - e^z + 1) / z^2: a power series near 0 (where the
 * closed form cancels), the closed form elsewhere.  phi'(0) = 1/2. */
static double zoh_dphi(double z)
{
    if (fabs(z) < 1.0) {
        /* sum_{m>=1} m z^(m-1) / (m+1)! */
        double term = 0.5, sum = 0.0; /* m = 1: 1 / 2! */
        for (int m = 1; m < 40; ++m) {
            sum += term;
            term *= z * (double)(m + 1) / ((double)m * (double)(m + 2));
        }
        return sum;
    }
    return (z * exp(z) - expm1(z)) / (z * z);
}

static double sigmoid(double v)
{
    return v >= 0.0 ? 1.0 / (1.0 + exp(-v)) : exp(v) / (1.0 + exp(v));
}

int ssm_oracle_scan_bwd(const double *x, const double *delta, const double *bias,
                        const double *A, const double *B, const double *C,
                        const double *D, const double *h0, const double *dy,
                        const double *dh_final, double *dx, double *ddelta,
                        double *dbias, double *dA, double *dB, double *dC,
                        double *dD, double *dh0, int64_t Bsz, int64_t L,
                        int64_t Dm, int64_t N, int flags, int nthreads)
{
    if (Bsz < 0 || L < 0 || Dm < 0 || N <= 0)
        return 1;
    const int euler = (flags & ORACLE_EULER_B) != 0;
    const int soft = (flags & ORACLE_DELTA_SOFTPLUS) != 0;
    const int64_t BLN = Bsz * L * N;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    const int nth = omp_get_max_threads();
#else
    (void)nthreads;
    const int nth = 1;
#endif
    /* dB, dC sum over channels: one private copy per thread, added in thread
     * order at the end (static schedule, so the result is reproducible). */
    double *priv = NULL;
    if (dB || dC) {
        priv = (double *)calloc((size_t)nth * 2 * (size_t)BLN + 1, sizeof(double));
        if (!priv)
            return 2;
    }
    int err = 0;
#pragma omp parallel
    {
#ifdef _OPENMP
        const int tid = omp_get_thread_num();
#else
        const int tid = 0;
#endif
        double *hs = (double *)malloc((size_t)(L + 1) * (size_t)N * sizeof(double));
        double *lam = (double *)malloc((size_t)N * sizeof(double));
        double *myB = priv ? priv + (size_t)tid * 2 * (size_t)BLN : NULL;
        double *myC = priv ? myB + BLN : NULL;
        if (!hs || !lam) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(static)
            for (int64_t d = 0; d < Dm; ++d) {
                const double *a = A + d * N;
                const double bias_d = bias ? bias[d] : 0.0;
                double dA_d[64];
                double *dAd = N <= 64 ? dA_d : (double *)calloc((size_t)N, sizeof(double));
                for (int64_t n = 0; n < N; ++n)
                    dAd[n] = 0.0;
                double dD_d = 0.0, dbias_d = 0.0;
                for (int64_t b = 0; b < Bsz; ++b) {
                    /* forward, keeping every state: hs[t+1] = h_t, hs[0] = h0 */
                    for (int64_t n = 0; n < N; ++n)
                        hs[n] = h0 ? h0[(b * Dm + d) * N + n] : 0.0;
                    for (int64_t t = 0; t < L; ++t) {
                        const int64_t i = (b * L + t) * Dm + d;
                        const int64_t r = (b * L + t) * N;
                        const double dt = step_size(delta[i], bias_d, flags);
                        for (int64_t n = 0; n < N; ++n) {
                            const double z = dt * a[n];
                            const double k = euler ? dt : dt * zoh_phi(z);
                            hs[(t + 1) * N + n] = exp(z) * hs[t * N + n] + k * B[r + n] * x[i];
                        }
                    }
                    /* backward */
                    for (int64_t n = 0; n < N; ++n)
                        lam[n] = dh_final ? dh_final[(b * Dm + d) * N + n] : 0.0;
                    for (int64_t t = L - 1; t >= 0; --t) {
                        const int64_t i = (b * L + t) * Dm + d;
                        const int64_t r = (b * L + t) * N;
                        const double dt = step_size(delta[i], bias_d, flags);
                        const double g = dy[i];
                        double gx = D[d] * g, gdt = 0.0;
                        for (int64_t n = 0; n < N; ++n) {
                            lam[n] += C[r + n] * g;
                            const double z = dt * a[n];
                            const double abar = exp(z);
                            const double k = euler ? dt : dt * zoh_phi(z);
                            const double dk_ddt = euler ? 1.0 : abar;
                            const double dk_da = euler ? 0.0 : dt * dt * zoh_dphi(z);
                            const double u = B[r + n] * x[i];
                            const double hprev = hs[t * N + n];
                            gx += lam[n] * k * B[r + n];
                            gdt += lam[n] * (a[n] * abar * hprev + dk_ddt * u);
                            dAd[n] += lam[n] * (dt * abar * hprev + dk_da * u);
                            if (myB)
                                myB[r + n] += lam[n] * k * x[i];
                            if (myC)
                                myC[r + n] += g * hs[(t + 1) * N + n];
                            lam[n] *= abar;
                        }
                        dD_d += g * x[i];
                        dx[i] = gx;
                        if (soft)
                            gdt *= sigmoid(delta[i] + bias_d);
                        ddelta[i] = gdt;
                        dbias_d += gdt;
                    }
                    if (dh0)
                        for (int64_t n = 0; n < N; ++n)
                            dh0[(b * Dm + d) * N + n] = lam[n];
                }
                for (int64_t n = 0; n < N; ++n)
                    dA[d * N + n] = dAd[n];
                dD[d] = dD_d;
                if (dbias)
                    dbias[d] = dbias_d;
                if (dAd != dA_d)
                    free(dAd);
            }
        }
        free(hs);
        free(lam);
    }
    if (priv) {
        for (int64_t j = 0; j < BLN; ++j) {
            double sb = 0.0, sc = 0.0;
            for (int th = 0; th < nth; ++th) {
                sb += priv[(size_t)th * 2 * (size_t)BLN + (size_t)j];
                sc += priv[(size_t)th * 2 * (size_t)BLN + (size_t)BLN + (size_t)j];
            }
            if (dB)
                dB[j] = sb;
            if (dC)
                dC[j] = sc;
        }
        free(priv);
    }
    return err;
}

/* ------------------------------------------------------------------------
 * Complex diagonal A: the state update with complex eigenvalues that the
 * bitig.info page on Mamba-3 describes (section "Karmasik Degerli Durum
 * Guncellemesi": complex numbers in the state update give rotation and
 * oscillation).  Readings: A[d][n] = a + i w is complex, the state h is
 * complex, delta, x, B_t, C_t, D and y are real, and
 *   Abar = exp(delta A),  Bbar = delta phi(delta A) B  (complex phi as above),
 *   h_t = Abar h_{t-1} + Bbar x_t,   y_t = sum_n C_t[n] Re(h_t[n]) + D x_t.
 * Layouts: A [Dm][N][2] and h0, h_final [Bsz][Dm][N][2] as (re, im) pairs.
 * ---------------------------------------------------------------------- */

/* (exp(z) - 1) for z = zr + i zi, without cancellation near 0:
 * Re = expm1(zr) cos(zi) - 2 sin^2(zi/2),  Im = exp(zr) sin(zi). */
static void cexpm1(double zr, double zi, double *er, double *ei)
{
    const double s = sin(0.5 * zi);
    *er = expm1(zr) * cos(zi) - 2.0 * s * s;
    *ei = exp(zr) * sin(zi);
}

/* One complex-state step for one channel; h holds (re, im) pairs. */
static double channel_step_complex(double *h, double xt, double dt, const double *a,
                                   const double *b, const double *c, double dskip,
                                   int64_t N, int euler)
{
    double y = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        const double zr = dt * a[2 * n], zi = dt * a[2 * n + 1];
        const double mag = exp(zr);
        const double abr = mag * cos(zi), abi = mag * sin(zi);
        double kr, ki; /* input coefficient Bbar / B */
        if (euler) {
            kr = dt;
            ki = 0.0;
        } else if (zr == 0.0 && zi == 0.0) {
            kr = dt; /* phi(0) = 1 */
            ki = 0.0;
        } else {
            double er, ei;
            cexpm1(zr, zi, &er, &ei);
            const double den = zr * zr + zi * zi; /* (er + i ei) / (zr + i zi) */
            kr = dt * (er * zr + ei * zi) / den;
            ki = dt * (ei * zr - er * zi) / den;
        }
        const double u = b[n] * xt;
        const double hr = h[2 * n], hi = h[2 * n + 1];
        h[2 * n] = abr * hr - abi * hi + kr * u;
        h[2 * n + 1] = abr * hi + abi * hr + ki * u;
        y += c[n] * h[2 * n];
    }
    return y + dskip * xt;
}

int ssm_oracle_scan_complex(const double *x, const double *delta, const double *bias,
                            const double *A, const double *B, const double *C,
                            const double *D, const double *h0, double *y,
                            double *h_final, int64_t Bsz, int64_t L, int64_t Dm,
                            int64_t N, int flags, int nthreads)
{
    if (Bsz < 0 || L < 0 || Dm < 0 || N <= 0)
        return 1;
    const int euler = (flags & ORACLE_EULER_B) != 0;
    const int64_t nchan = Bsz * Dm;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int err = 0;
#pragma omp parallel
    {
        double *h = (double *)malloc((size_t)(2 * N) * sizeof(double));
        if (!h) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t ch = 0; ch < nchan; ++ch) {
                const int64_t b = ch / Dm, d = ch % Dm;
                const double bias_d = bias ? bias[d] : 0.0;
                for (int64_t k = 0; k < 2 * N; ++k)
                    h[k] = h0 ? h0[(b * Dm + d) * 2 * N + k] : 0.0;
                for (int64_t t = 0; t < L; ++t) {
                    const int64_t i = (b * L + t) * Dm + d;
                    const int64_t r = (b * L + t) * N;
                    const double dt = step_size(delta[i], bias_d, flags);
                    y[i] = channel_step_complex(h, x[i], dt, A + d * 2 * N, B + r, C + r, D[d], N, euler);
                }
                if (h_final)
                    for (int64_t k = 0; k < 2 * N; ++k)
                        h_final[(b * Dm + d) * 2 * N + k] = h[k];
            }
            free(h);
        }
    }
    return err;
}

int ssm_oracle_step_complex(const double *x, const double *delta, const double *bias,
                            const double *A, const double *B, const double *C,
                            const double *D, double *h, double *y, int64_t Bsz,
                            int64_t Dm, int64_t N, int flags)
{
    if (Bsz < 0 || Dm < 0 || N <= 0)
        return 1;
    const int euler = (flags & ORACLE_EULER_B) != 0;
    for (int64_t b = 0; b < Bsz; ++b)
        for (int64_t d = 0; d < Dm; ++d) {
            const int64_t i = b * Dm + d;
            const double dt = step_size(delta[i], bias ? bias[d] : 0.0, flags);
            y[i] = channel_step_complex(h + i * 2 * N, x[i], dt, A + d * 2 * N, B + b * N,
                                        C + b * N, D[d], N, euler);
        }
    return 0;
}

/* ------------------------------------------------------------------------
 * Backward of the complex-A scan: the chain rule on the recurrence above, with
 * every complex quantity taken as its (re, im) pair of reals.  For a real loss
 * L and a product w = p q of complex numbers, the pair (dL/dRe p, dL/dIm p) is
 * G_w conj(q) as a complex number, G_w = dL/dRe w + i dL/dIm w; for w = f(p)
 * holomorphic it is G_w conj(f'(p)).  With lambda = G_{h_t}:
 *   lambda_t  += C_t[n] dy_t              (y reads Re h_t)
 *   G_Abar     = lambda conj(h_{t-1}),    G_k = lambda u,   u = B_t[n] x_t
 *   dL/du      = Re(lambda conj(k))       (dx, dB through u)
 *   dL/ddelta += Re(G_Abar conj(A Abar)) + Re(G_k conj(dk/ddelta))
 *   dL/dA     += G_Abar conj(delta Abar)  + G_k conj(dk/dA)
 *   lambda_{t-1} = lambda conj(Abar)
 * where k = delta phi(delta A) = (Abar - 1)/A (ZOH: dk/ddelta = Abar,
 * dk/dA = delta^2 phi'(delta A)) or k = delta (Euler: dk/ddelta = 1).
 * Layouts as ssm_oracle_scan_bwd, with A, dA [Dm][N][2] and h0, dh_final, dh0
 * [Bsz][Dm][N][2] as (re, im) pairs.
 * ---------------------------------------------------------------------- */

/* phi(z) = (exp(z) - 1) / z for complex z, 1 at z = 0 */
static double complex cphi(double complex z)
{
    if (creal(z) == 0.0 && cimag(z) == 0.0)
        return 1.0;
    double er, ei;
    cexpm1(creal(z), cimag(z), &er, &ei);
    return (er + I * ei) / z;
}

/* phi'(z) = (z e^z - (e^z - 1)) / z^2 for complex z; for |z| < 1 its series
 * sum_{m>=1} m z^(m-1) / (m+1)!, which has no cancellation */
static double complex cdphi(double complex z)
{
    if (cabs(z) < 1.0) {
        double complex term = 0.5, sum = 0.0;
        for (int m = 1; m < 40; ++m) {
            sum += term;
            term *= z * (double)(m + 1) / ((double)m * (double)(m + 2));
        }
        return sum;
    }
    double er, ei;
    cexpm1(creal(z), cimag(z), &er, &ei);
    return (z * cexp(z) - (er + I * ei)) / (z * z);
}

int ssm_oracle_scan_complex_bwd(const double *x, const double *delta, const double *bias,
                                const double *A, const double *B, const double *C,
                                const double *D, const double *h0, const double *dy,
                                const double *dh_final, double *dx, double *ddelta,
                                double *dbias, double *dA, double *dB, double *dC,
                                double *dD, double *dh0, int64_t Bsz, int64_t L,
                                int64_t Dm, int64_t N, int flags, int nthreads)
{
    if (Bsz < 0 || L < 0 || Dm < 0 || N <= 0)
        return 1;
    const int euler = (flags & ORACLE_EULER_B) != 0;
    const int soft = (flags & ORACLE_DELTA_SOFTPLUS) != 0;
    const int64_t BLN = Bsz * L * N;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    const int nth = omp_get_max_threads();
#else
    (void)nthreads;
    const int nth = 1;
#endif
    double *priv = NULL;
    if (dB || dC) {
        priv = (double *)calloc((size_t)nth * 2 * (size_t)BLN + 1, sizeof(double));
        if (!priv)
            return 2;
    }
    int err = 0;
#pragma omp parallel
    {
#ifdef _OPENMP
        const int tid = omp_get_thread_num();
#else
        const int tid = 0;
#endif
        /* hs[(t+1) N + n] = h_t as (re, im) pairs, hs[n] = h0 */
        double *hs = (double *)malloc((size_t)(L + 1) * (size_t)(2 * N) * sizeof(double));
        double complex *lam = (double complex *)malloc((size_t)N * sizeof(double complex));
        double complex *dAd = (double complex *)malloc((size_t)N * sizeof(double complex));
        double *myB = priv ? priv + (size_t)tid * 2 * (size_t)BLN : NULL;
        double *myC = priv ? myB + BLN : NULL;
        if (!hs || !lam || !dAd) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(static)
            for (int64_t d = 0; d < Dm; ++d) {
                const double *a = A + d * 2 * N;
                const double bias_d = bias ? bias[d] : 0.0;
                for (int64_t n = 0; n < N; ++n)
                    dAd[n] = 0.0;
                double dD_d = 0.0, dbias_d = 0.0;
                for (int64_t b = 0; b < Bsz; ++b) {
                    /* forward with the forward oracle's own step, keeping every state */
                    for (int64_t k = 0; k < 2 * N; ++k)
                        hs[k] = h0 ? h0[(b * Dm + d) * 2 * N + k] : 0.0;
                    for (int64_t t = 0; t < L; ++t) {
                        const int64_t i = (b * L + t) * Dm + d;
                        const int64_t r = (b * L + t) * N;
                        const double dt = step_size(delta[i], bias_d, flags);
                        for (int64_t k = 0; k < 2 * N; ++k)
                            hs[(t + 1) * 2 * N + k] = hs[t * 2 * N + k];
                        (void)channel_step_complex(hs + (t + 1) * 2 * N, x[i], dt, a, B + r, C + r, D[d], N, euler);
                    }
                    /* backward */
                    for (int64_t n = 0; n < N; ++n) {
                        const int64_t j = ((b * Dm + d) * N + n) * 2;
                        lam[n] = dh_final ? dh_final[j] + I * dh_final[j + 1] : 0.0;
                    }
                    for (int64_t t = L - 1; t >= 0; --t) {
                        const int64_t i = (b * L + t) * Dm + d;
                        const int64_t r = (b * L + t) * N;
                        const double dt = step_size(delta[i], bias_d, flags);
                        const double g = dy[i];
                        double gx = D[d] * g, gdt = 0.0;
                        for (int64_t n = 0; n < N; ++n) {
                            const double complex An = a[2 * n] + I * a[2 * n + 1];
                            const double complex z = dt * An;
                            const double complex abar = cexp(z);
                            const double complex k = euler ? (double complex)dt : dt * cphi(z);
                            const double complex hprev = hs[t * 2 * N + 2 * n] + I * hs[t * 2 * N + 2 * n + 1];
                            const double u = B[r + n] * x[i];
                            lam[n] += C[r + n] * g;
                            const double complex gabar = lam[n] * conj(hprev);
                            const double complex gk = lam[n] * u;
                            const double gu = creal(lam[n] * conj(k));
                            gx += gu * B[r + n];
                            if (myB)
                                myB[r + n] += gu * x[i];
                            if (myC)
                                myC[r + n] += g * hs[(t + 1) * 2 * N + 2 * n];
                            gdt += creal(gabar * conj(An * abar));
                            if (euler) {
                                gdt += creal(gk);
                                dAd[n] += gabar * conj(dt * abar);
                            } else {
                                gdt += creal(gk * conj(abar));
                                dAd[n] += gabar * conj(dt * abar) + gk * conj(dt * dt * cdphi(z));
                            }
                            lam[n] *= conj(abar);
                        }
                        dD_d += g * x[i];
                        dx[i] = gx;
                        if (soft)
                            gdt *= sigmoid(delta[i] + bias_d);
                        ddelta[i] = gdt;
                        dbias_d += gdt;
                    }
                    if (dh0)
                        for (int64_t n = 0; n < N; ++n) {
                            const int64_t j = ((b * Dm + d) * N + n) * 2;
                            dh0[j] = creal(lam[n]);
                            dh0[j + 1] = cimag(lam[n]);
                        }
                }
                for (int64_t n = 0; n < N; ++n) {
                    dA[(d * N + n) * 2] = creal(dAd[n]);
                    dA[(d * N + n) * 2 + 1] = cimag(dAd[n]);
                }
                dD[d] = dD_d;
                if (dbias)
                    dbias[d] = dbias_d;
            }
        }
        free(hs);
        free(lam);
        free(dAd);
    }
    if (priv) {
        for (int64_t j = 0; j < BLN; ++j) {
            double sb = 0.0, sc = 0.0;
            for (int th = 0; th < nth; ++th) {
                sb += priv[(size_t)th * 2 * (size_t)BLN + (size_t)j];
                sc += priv[(size_t)th * 2 * (size_t)BLN + (size_t)BLN + (size_t)j];
            }
            if (dB)
                dB[j] = sb;
            if (dC)
                dC[j] = sc;
        }
        free(priv);
    }
    return err;
}

int ssm_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
