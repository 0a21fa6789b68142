/*
 * libssmscan -- selective state-space scan and recurrent decode step for
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operation (pages: "Mamba SSM Nedir? Transformer Alternatifi Rehberi",
 * yapayzekasozluk.tr, sections "State Space Model Temelleri", "Ayrik Zamana
 * Gecis" and "Mamba'nin Yeniligi: Selective SSM"; and "Mamba: Transformer'a
 * Meydan Okuyan Uzun-Bagimli Model", matematikkaravani.com, section "Eski
 * fikrin geri donusu: durum uzayi"):
 *
 *   for every batch row b, channel d and state n, with a diagonal real A:
 *     Abar   = exp(delta_t[d] * A[d,n])                       (zero-order hold)
 *     Bbar   = (Abar - 1) / A[d,n] * B_t[n]    (limit delta_t[d]*B_t[n] at A=0)
 *     h_t    = Abar * h_{t-1} + Bbar * x_t[d]
 *     y_t[d] = sum_n C_t[n] * h_t[d,n] + D[d] * x_t[d]
 *
 * B_t, C_t and delta_t are per-token inputs (the selection mechanism computes
 * them upstream); B_t and C_t are shared by all channels of a batch row.
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major, contiguous; there are no strides.
 *   - Device pointers.  The caller owns every buffer; the library keeps no
 *     pointer after the call returns.
 *   - Calls are asynchronous: work is enqueued on `stream` (a hipStream_t
 *     passed as void*, NULL = the default stream) and the call returns.  The
 *     caller synchronises.  Buffers must stay valid until the work completes.
 *   - `dtype` (ssm_dtype) selects the storage type of x, delta, B, C and y.
 *     A, D and the state (h_final, h) are always fp32.  Arithmetic: fp32 for
 *     bf16 storage; for fp32 storage the scans compute in fp64 and the decode
 *     steps in fp32 with libm-accurate exp, expm1, sin and cos.
 *   - Return value: SSM_OK (0) or a positive ssm_status.  On an argument error
 *     nothing is enqueued and no device call is made; ssm_last_error() gives
 *     a thread-local description of the most recent failure.
 *   - Preconditions that are documented, not checked: delta >= 0 and A <= 0
 *     (a real part of A that is not negative lets the state grow; "Mamba SSM
 *     Nedir?", section "Sinirliliklar ve Acik Sorular").  Non-finite inputs
 *     propagate.
 *   - A pointer may be NULL only when its tensor has no elements.
 *   - Every pointer must be aligned to its element size.
 *   - Supported state sizes: N in {1, 2, 4, 8, 16} (ssm_scan_ssd_fwd: 32, 64, 128).
 *   - Scans: one time step of x (Dm * element size) must be below 1 GiB, else
 *     SSM_ERR_BAD_DIM (kernels address a time segment with 32-bit offsets).
 *   - Thread safety: calls may come from several host threads.  Two calls that
 *     run concurrently on different streams of one device use separate
 *     library scratch memory (kept per device and stream).
 *   - Library scratch memory (time-chunk summaries, converted B/C rows) is
 *     allocated on first use per (device, stream), grows on demand, and is
 *     kept until ssm_release_workspaces() or process exit.  Allocation
 *     failure returns SSM_ERR_NOMEM.  Calls on one stream share its scratch,
 *     so they must not run concurrently with each other (stream order
 *     guarantees that for eager calls).
 *   - HIP graph capture.  A call made while `stream` is being captured
 *     records kernels that use the stream's scratch buffer; the graph keeps
 *     that buffer's address.  Such a call never allocates or synchronises: if
 *     the stream's scratch is smaller than the call needs it returns
 *     SSM_ERR_CAPTURE and records nothing (make the same call once, eagerly,
 *     on the same stream before capturing).  A buffer that was used during a
 *     capture is never freed when a later eager call grows the stream's
 *     scratch; it is kept until ssm_release_workspaces(), which therefore
 *     invalidates every captured graph that calls into the library.  A graph
 *     replay uses the scratch of the stream it was captured on: do not replay
 *     it concurrently with other library calls on that stream, or with
 *     another replay of a graph captured on it.  ssm_step, ssm_step_ex,
 *     ssm_step_fused and ssm_step_complex use no scratch.
 */
#ifndef SSMSCAN_H
#define SSMSCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSM_F32 = 0,  /* IEEE binary32 */
    SSM_BF16 = 1  /* bfloat16 (upper 16 bits of binary32); y is rounded to nearest even */
} ssm_dtype;

typedef enum {
    SSM_OK = 0,
    SSM_ERR_NULLPTR = 1,        /* a non-empty tensor has a NULL pointer */
    SSM_ERR_BAD_DIM = 2,        /* a negative size, a size whose byte count overflows, or a size
                                   above an entry point's stated limit */
    SSM_ERR_BAD_DTYPE = 3,      /* dtype is not an ssm_dtype */
    SSM_ERR_UNSUPPORTED_N = 4,  /* N not in {1, 2, 4, 8, 16} */
    SSM_ERR_ALIGN = 5,          /* a pointer is not aligned to its element size */
    SSM_ERR_ALIAS = 6,          /* an output overlaps an input or another output */
    SSM_ERR_NOMEM = 7,          /* library scratch memory could not be allocated */
    SSM_ERR_HIP = 8,            /* the HIP runtime reported an error (see ssm_last_error) */
    SSM_ERR_BAD_OPTION = 9,     /* unknown option id or value, or unknown flag bits */
    SSM_ERR_CAPTURE = 10        /* the stream is being captured into a HIP graph and the call
                                   needs more library scratch than the stream already holds */
} ssm_status;

/*
 * Flags of ssm_scan_fused_fwd and ssm_step_fused (bitwise OR).
 *
 * SSM_DELTA_SOFTPLUS: the delta argument holds the raw projection output and
 *   the recurrence uses delta = softplus(delta_in + delta_bias[d]), the
 *   activation the "Mamba SSM Nedir?" page gives for delta (section
 *   "Mamba'nin Yeniligi: Selective SSM").  Without it the recurrence uses
 *   delta_in + delta_bias[d] (delta_bias NULL means 0).
 * SSM_EULER_B: the input term uses the Euler rule, Bbar = delta * B, while
 *   Abar stays exp(delta * A) -- the rule the bitig.info Mamba-3 page (section
 *   "Gelistirilmis Ayriklastirma Semasi") attributes to Mamba-1 and -2.
 *   Without it the input term is the zero-order hold (exp(delta A) - 1)/A * B.
 */
typedef enum {
    SSM_DELTA_SOFTPLUS = 1,
    SSM_EULER_B = 2
} ssm_flags;

/*
 * Full-sequence selective scan, zero initial state.
 *
 *   x, delta : [Bsz][L][Dm]   dtype          input sequence and step sizes
 *   A        : [Dm][N]        fp32           diagonal state matrix per channel
 *   B, C     : [Bsz][L][N]    dtype          per-token input/output projections
 *   D        : [Dm]           fp32           feed-through
 *   y        : [Bsz][L][Dm]   dtype  (out)   y_t as defined above
 *   h_final  : [Bsz][Dm][N]   fp32   (out)   state after the last token; may be
 *                                            NULL (then not written).  With L == 0
 *                                            it is the zero initial state.
 *
 * y must not overlap any input; h_final must not overlap any input or y.
 * Sizes of 0 are valid and do nothing beyond writing h_final.
 * The scan is the recurrence above evaluated in parallel: channels are
 * independent, and time is cut into chunks whose summaries are combined
 * with the composition of affine maps (a1,b1) o (a2,b2) = (a1*a2, a2*b1 + b2)
 * ("Mamba SSM Nedir?", section "Paralel Tarama Algoritmasi").  The result
 * equals the sequential recurrence up to fp32 rounding.
 */
int ssm_scan_fwd(const void *x, const void *delta, const float *A,
                 const void *B, const void *C, const float *D,
                 void *y, float *h_final,
                 int64_t Bsz, int64_t L, int64_t Dm, int64_t N,
                 int dtype, void *stream);

/*
 * Scan with an initial state (resumable prefill): as ssm_scan_fwd, but the
 * recurrence starts from h_init [Bsz][Dm][N] fp32 instead of zero.  h_init may
 * be NULL (zero state).  h_init may be the same buffer as h_final (the final
 * state then overwrites the initial one); otherwise it must not overlap any
 * output.  scan(L1+L2) equals scan(L2, h_init = h_final of scan(L1)) up to
 * fp32 rounding.
 */
int ssm_scan_fwd_ex(const void *x, const void *delta, const float *A,
                    const void *B, const void *C, const float *D,
                    const float *h_init, void *y, float *h_final,
                    int64_t Bsz, int64_t L, int64_t Dm, int64_t N,
                    int dtype, void *stream);

/*
 * ssm_scan_fwd_ex without allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid it).  Arguments, layouts and results as ssm_scan_fwd_ex.
 * Instead of the per-stream scratch it uses a fixed 64 MiB device array that
 * the library holds on every GPU it runs on until the process ends; it calls
 * no allocator and creates no timing events.  The segment plan is shortened
 * when the default one needs more than 64 MiB (results then differ from
 * ssm_scan_fwd_ex by fp32 rounding only).  A call that needs more than
 * 64 MiB with a single segment -- Bsz * L * 2N converted B/C values (4 bytes
 * each for bf16 storage, 8 for fp32) -- returns SSM_ERR_BAD_DIM and enqueues
 * nothing.  Every call on a GPU shares that GPU's array: calls that overlap
 * in time on one GPU (on different streams, from several host threads, or
 * graphs replayed concurrently) race and give wrong results.
 * Nothing in the array needs to start at zero; it keeps the last call's data.
 */
int ssm_scan_fwd_noalloc(const void *x, const void *delta, const float *A,
                         const void *B, const void *C, const float *D,
                         const float *h_init, void *y, float *h_final,
                         int64_t Bsz, int64_t L, int64_t Dm, int64_t N,
                         int dtype, void *stream);

/*
 * Packed variable-length scan (resumable prefill of several sequences at once,
 * without padding).  nseq sequences are concatenated along time in one row:
 * sequence k covers steps cu_seqlens[k] .. cu_seqlens[k+1]-1.
 *
 *   x, delta, y : [L][Dm]        dtype
 *   B, C        : [L][N]         dtype
 *   A           : [Dm][N] fp32;  D : [Dm] fp32
 *   cu_seqlens  : [nseq+1] int64, device memory; cu_seqlens[0] = 0,
 *                 non-decreasing, cu_seqlens[nseq] = L (empty sequences allowed)
 *   h_init      : [nseq][Dm][N] fp32 or NULL -- state each sequence starts from
 *   h_final     : [nseq][Dm][N] fp32 or NULL -- each sequence's last state (its
 *                 h_init, or zero, if the sequence is empty)
 *
 * The state restarts at every sequence start, so y of each sequence equals
 * ssm_scan_fwd_ex over that sequence alone.  cu_seqlens is read on the device
 * and is not validated; values that break the rules above give unspecified
 * results but every access stays inside the buffers.  h_init must not overlap
 * h_final; no output may overlap an input.
 */
int ssm_scan_varlen_fwd(const void *x, const void *delta, const float *A,
                        const void *B, const void *C, const float *D,
                        const int64_t *cu_seqlens, int64_t nseq,
                        const float *h_init, void *y, float *h_final,
                        int64_t L, int64_t Dm, int64_t N, int dtype, void *stream);

/*
 * The scan with every option: delta pre-processing and the input rule
 * (ssm_flags), an initial state, and either a dense batch or packed sequences.
 *
 *   delta_bias : [Dm] fp32 or NULL -- added to delta before softplus
 *   flags      : ssm_flags bits; other bits give SSM_ERR_BAD_OPTION
 *   cu_seqlens : NULL -> dense batch, shapes as in ssm_scan_fwd_ex (h_init may
 *                equal h_final);  non-NULL -> packed sequences as in
 *                ssm_scan_varlen_fwd (Bsz must be 1, nseq sequences, h_init and
 *                h_final [nseq][Dm][N] and not overlapping).  nseq is ignored
 *                when cu_seqlens is NULL.
 * Everything else as in ssm_scan_fwd_ex.  With flags = 0 and delta_bias NULL
 * the result is bit-identical to ssm_scan_fwd_ex / ssm_scan_varlen_fwd.
 */
int ssm_scan_fused_fwd(const void *x, const void *delta, const float *delta_bias,
                       const float *A, const void *B, const void *C, const float *D,
                       const int64_t *cu_seqlens, int64_t nseq,
                       const float *h_init, void *y, float *h_final,
                       int64_t Bsz, int64_t L, int64_t Dm, int64_t N, int dtype,
                       unsigned flags, void *stream);

/*
 * Scan with complex diagonal A: the state update with complex eigenvalues
 * (rotation as well as decay) that the bitig.info page on Mamba-3 describes
 * (section "Karmasik Degerli Durum Guncellemesi").  Per (b, d, n), with
 * A[d][n] = a + i w and a complex state h:
 *   Abar = exp(delta A),  Bbar = (Abar - 1)/A * B_t[n]  (delta B_t[n] with SSM_EULER_B)
 *   h_t = Abar h_{t-1} + Bbar x_t,   y_t = sum_n C_t[n] Re(h_t[n]) + D x_t
 * x, delta, B, C, D, y, delta_bias, dtype and flags are as in
 * ssm_scan_fused_fwd (real); complex arrays are (re, im) fp32 pairs:
 *   A       : [Dm][N][2]
 *   h_init  : [Bsz][Dm][N][2] or NULL (zero); may equal h_final
 *   h_final : [Bsz][Dm][N][2] or NULL
 * Dense batch only.  Other rules as ssm_scan_fwd_ex.
 */
int ssm_scan_complex_fwd(const void *x, const void *delta, const float *delta_bias,
                         const float *A, const void *B, const void *C, const float *D,
                         const float *h_init, void *y, float *h_final,
                         int64_t Bsz, int64_t L, int64_t Dm, int64_t N, int dtype,
                         unsigned flags, void *stream);

/* One decode step with complex A; h [Bsz][Dm][N][2] fp32 updated in place.
 * Dm*N may be at most 2^23 (64 MiB of state per batch row), else
 * SSM_ERR_BAD_DIM.  Arguments otherwise as ssm_step_fused. */
int ssm_step_complex(const void *x, const void *delta, const float *delta_bias,
                     const float *A, const void *B, const void *C, const float *D,
                     float *h, void *y, int64_t Bsz, int64_t Dm, int64_t N, int dtype,
                     unsigned flags, void *stream);

/*
 * Scan with one scalar decay per head: the state-space-duality layer.  The
 * bitig.info page on Mamba-3 (section "Karmasik Degerli Durum Guncellemesi")
 * says Mamba-2 reduced the state transition to real scalars; the "Mamba SSM
 * Nedir?" page (section "Mamba-2 ve Guncel Gelismeler") states that such an
 * SSM equals a masked attention.  Channels form heads of head_dim consecutive
 * channels; head h = d / head_dim has one real A[h] for all N states and one
 * delta per step.  Per (b, d, n):
 *   dt     = delta[b,t,h] (+ delta_bias[h], softplus with SSM_DELTA_SOFTPLUS)
 *   Abar   = exp(dt * A[h])
 *   Bbar   = (Abar - 1) / A[h] * B_t[n]    (dt * B_t[n] at A = 0 or with SSM_EULER_B)
 *   h_t    = Abar * h_{t-1} + Bbar * x_t[d],   y_t[d] = sum_n C_t[n] h_t[d,n] + D[d] x_t[d]
 * which is ssm_scan_fused_fwd with A[d,n] = A[h] and delta[b,t,d] = delta[b,t,h].
 * bf16 storage evaluates it in its chunked matrix form on the matrix cores,
 * exact up to rounding: per 64-step chunk, (C B^T masked by the decays) x for
 * the steps inside the chunk plus C h for the state entering it.
 *   x, y       : [Bsz][L][Dm]  dtype
 *   delta      : [Bsz][L][H]   dtype, H = Dm / head_dim
 *   delta_bias : [H] fp32, or NULL (0)
 *   A          : [H] fp32
 *   B, C       : [Bsz][L][N]   dtype, shared by all heads of a row
 *   D          : [Dm] fp32
 *   h_init     : [Bsz][Dm][N] fp32 or NULL (zero); may equal h_final
 *   h_final    : [Bsz][Dm][N] fp32 or NULL
 *   head_dim   : 64 (the only value supported); Dm must be a multiple of it
 *   N          : 32, 64 or 128
 * x, y, B, C, h_init and h_final must be 16-byte aligned.  bf16 storage
 * multiplies bf16 operands exactly and splits fp32 operands into two bf16
 * terms (about 2^-17 relative per product), accumulating in fp32; fp32
 * storage evaluates the recurrence in fp64.  Other rules as
 * ssm_scan_fused_fwd (dense batch only).
 */
int ssm_scan_ssd_fwd(const void *x, const void *delta, const float *delta_bias,
                     const float *A, const void *B, const void *C, const float *D,
                     const float *h_init, void *y, float *h_final,
                     int64_t Bsz, int64_t L, int64_t Dm, int64_t N, int64_t head_dim,
                     int dtype, unsigned flags, void *stream);

/*
 * Backward of the scan: every input gradient for given output gradients.
 * The chain rule on the recurrence ("Mamba SSM Nedir?", section "Ayrik Zamana
 * Gecis"), as training needs it (section "Paralel Tarama Algoritmasi": the
 * same parallel scan serves training).  With lambda_t = dL/dh_t,
 *   lambda_t = C_t dy_t + Abar_{t+1} lambda_{t+1}   (lambda_{L-1} adds dh_final)
 * and every gradient is a sum over t of lambda_t, the states h_{t-1} and the
 * inputs.
 *
 * Inputs: the forward's x, delta, delta_bias, A, B, C, D, h_init (shapes,
 *   dtype and flags exactly as in ssm_scan_fused_fwd with cu_seqlens NULL;
 *   delta_bias and h_init may be NULL) and
 *   dy       : [Bsz][L][Dm] dtype   dL/dy
 *   dh_final : [Bsz][Dm][N] fp32 or NULL (zero)   dL/dh_final
 * Outputs (overwritten, never accumulated):
 *   dx, ddelta  : [Bsz][L][Dm] dtype  (ddelta is for the delta argument as
 *                 passed: the raw value when SSM_DELTA_SOFTPLUS is set)
 *   ddelta_bias : [Dm] fp32 or NULL
 *   dA          : [Dm][N] fp32       dD : [Dm] fp32
 *   dB, dC      : [Bsz][L][N] fp32   (sums over channels)
 *   dh_init     : [Bsz][Dm][N] fp32 or NULL
 * No output may overlap an input or another output.  The forward states are
 * recomputed (nothing is saved from the forward call).  Library scratch
 * (Acc = 4 bytes for bf16 storage, 8 for fp32; S = ceil(L / segment length),
 * segments of 32 steps for bf16 and 16 for fp32, G groups and R =
 * ceil(Dm / 256) blocks per batch row as ssm_scan_bwd_plan reports):
 *   (3N + 2) * S * Bsz * Dm * Acc      segment summaries and entering states
 * + 2 * N * G * Bsz * Dm * Acc         adjoint entering each group, dA partials
 * + 4 * R * Bsz * L * N * Acc          per-block partial sums of dB and dC
 * + 2 * Bsz * L * N * Acc              converted B/C rows
 * (smaller terms omitted): about 2.5 GB for Bsz=4, L=16384, Dm=5120, N=16.
 * A 32-step (fp32: 16-step) segment of x must span less than 1 GiB
 * (segment length * Dm * element size), else SSM_ERR_BAD_DIM.
 */
int ssm_scan_bwd(const void *x, const void *delta, const float *delta_bias,
                 const float *A, const void *B, const void *C, const float *D,
                 const float *h_init, const void *dy, const float *dh_final,
                 void *dx, void *ddelta, float *ddelta_bias, float *dA,
                 float *dB, float *dC, float *dD, float *dh_init,
                 int64_t Bsz, int64_t L, int64_t Dm, int64_t N, int dtype,
                 unsigned flags, void *stream);

/*
 * Backward of the packed variable-length scan (ssm_scan_varlen_fwd, or
 * ssm_scan_fused_fwd with cu_seqlens): sequences concatenated along time,
 * each with its own initial state, as in training on packed batches.  The
 * chain rule on the recurrence ("Mamba SSM Nedir?", section "Ayrik Zamana
 * Gecis") applied to every sequence alone: the gradients are those of
 * ssm_scan_bwd with Bsz = 1 on that sequence's steps and state rows, with dA,
 * dD and ddelta_bias summed over the sequences.  At a sequence start the
 * adjoint leaving the step is that sequence's dh_init, and the previous
 * sequence's last state receives only its own outputs' and dh_final's share.
 *
 *   x, delta, dy, dx, ddelta : [L][Dm]   dtype
 *   B, C                     : [L][N]    dtype
 *   dB, dC                   : [L][N]    fp32
 *   cu_seqlens               : [nseq+1] int64, device memory, rules as in
 *                              ssm_scan_varlen_fwd (read on the device, not
 *                              validated; values that break the rules give
 *                              unspecified results but every access stays
 *                              inside the buffers)
 *   h_init, dh_final, dh_init: [nseq][Dm][N] fp32 or NULL (h_init, dh_final:
 *                              zero).  An empty sequence gets dh_init =
 *                              dh_final (its final state is its initial one).
 *   A, D, delta_bias, dA, dD, ddelta_bias, dtype, flags: as in ssm_scan_bwd.
 * nseq = 0 is allowed only with L = 0.  Overlap rules, scratch (with Bsz = 1,
 * plus 2 S ints) and the segment size limit as in ssm_scan_bwd.
 */
int ssm_scan_varlen_bwd(const void *x, const void *delta, const float *delta_bias,
                        const float *A, const void *B, const void *C, const float *D,
                        const int64_t *cu_seqlens, int64_t nseq, const float *h_init,
                        const void *dy, const float *dh_final,
                        void *dx, void *ddelta, float *ddelta_bias, float *dA,
                        float *dB, float *dC, float *dD, float *dh_init,
                        int64_t L, int64_t Dm, int64_t N, int dtype,
                        unsigned flags, void *stream);

/*
 * Backward of the complex-A scan (ssm_scan_complex_fwd): the chain rule on
 * its recurrence (the bitig.info page on Mamba-3, section "Karmasik Degerli
 * Durum Guncellemesi"; training as in "Mamba SSM Nedir?", section "Paralel
 * Tarama Algoritmasi").  For the real loss L, the gradient of a complex
 * quantity z is the pair (dL/dRe z, dL/dIm z).  With lambda_t = dL/dh_t,
 *   lambda_t = C_t dy_t + conj(Abar_{t+1}) lambda_{t+1}   (lambda_{L-1} adds dh_final)
 * (the output reads Re h_t, so C_t dy_t enters the real part only).
 *
 * Inputs: the forward's x, delta, delta_bias, A, B, C, D, h_init (shapes,
 *   dtype and flags exactly as in ssm_scan_complex_fwd) and
 *   dy       : [Bsz][L][Dm] dtype
 *   dh_final : [Bsz][Dm][N][2] fp32 or NULL (zero)
 * Outputs (overwritten, never accumulated):
 *   dx, ddelta  : [Bsz][L][Dm] dtype  (ddelta for delta as passed)
 *   ddelta_bias : [Dm] fp32 or NULL
 *   dA          : [Dm][N][2] fp32     dD : [Dm] fp32
 *   dB, dC      : [Bsz][L][N] fp32    (sums over channels)
 *   dh_init     : [Bsz][Dm][N][2] fp32 or NULL
 * No output may overlap an input or another output.  The forward states are
 * recomputed.  Segments of 16 steps; library scratch (Acc = 4 bytes for bf16
 * storage, 8 for fp32; S = ceil(L / 16), G groups, R = ceil(Dm / 256) blocks
 * per batch row for bf16 and ceil(Dm / 128) for fp32):
 *   (6N + 2) * S * Bsz * Dm * Acc      segment summaries and entering states
 * + (4N + 2) * G * Bsz * Dm * Acc      adjoint entering each group, partials
 * + 2 * (R + 1) * Bsz * L * N * Acc    partial sums of dB, dC; B/C rows
 * A 16-step segment of x must span less than 1 GiB, else SSM_ERR_BAD_DIM.
 * Dense batch only.
 */
int ssm_scan_complex_bwd(const void *x, const void *delta, const float *delta_bias,
                         const float *A, const void *B, const void *C, const float *D,
                         const float *h_init, const void *dy, const float *dh_final,
                         void *dx, void *ddelta, float *ddelta_bias, float *dA,
                         float *dB, float *dC, float *dD, float *dh_init,
                         int64_t Bsz, int64_t L, int64_t Dm, int64_t N, int dtype,
                         unsigned flags, void *stream);

/*
 * One recurrent decode step on a resident state, updated in place
 * ("Mamba SSM Nedir?", section "Karmasiklik Karsilastirmasi": inference
 * updates a fixed-size state per token).  bf16 I/O:
 *
 *   x, delta : [Bsz][Dm]     bf16
 *   A        : [Dm][N]       fp32
 *   B, C     : [Bsz][N]      bf16
 *   D        : [Dm]          fp32
 *   h        : [Bsz][Dm][N]  fp32   (in/out)  h <- Abar*h + Bbar*x
 *   y        : [Bsz][Dm]     bf16   (out)     y = sum_n C[n]*h_new[n] + D*x
 *
 * y must not overlap any input or h; h must not overlap any input.
 * Dm*N may be at most 2^24 (64 MiB of state per batch row), else
 * SSM_ERR_BAD_DIM.
 */
int ssm_step(const void *x, const void *delta, const float *A,
             const void *B, const void *C, const float *D,
             float *h, void *y,
             int64_t Bsz, int64_t Dm, int64_t N, void *stream);

/* ssm_step with an explicit storage dtype for x, delta, B, C, y. */
int ssm_step_ex(const void *x, const void *delta, const float *A,
                const void *B, const void *C, const float *D,
                float *h, void *y,
                int64_t Bsz, int64_t Dm, int64_t N, int dtype, void *stream);

/*
 * ssm_step_ex with the options of ssm_scan_fused_fwd: delta_bias [Dm] fp32 or
 * NULL, flags = ssm_flags bits.  Stepping a state through L tokens with the
 * same options reproduces the scan's y and final state.
 */
int ssm_step_fused(const void *x, const void *delta, const float *delta_bias,
                   const float *A, const void *B, const void *C, const float *D,
                   float *h, void *y, int64_t Bsz, int64_t Dm, int64_t N, int dtype,
                   unsigned flags, void *stream);

/* Static description of a status code (never NULL). */
const char *ssm_strerror(int code);

/* Description of the most recent failure on the calling thread ("" if none). */
const char *ssm_last_error(void);

/* Library version: major*10000 + minor*100 + patch. */
int ssm_version(void);

/*
 * Tuning/diagnostic options (process-wide; they change how the work is cut,
 * never what is computed):
 *   SSM_OPT_SEGMENT_LEN  : time-chunk length of the scan; 0 = automatic
 *                          (default).  Values < 0 are rejected.
 *   SSM_OPT_FORCE_GENERAL: 1 = always take the general-A path, even when
 *                          A[d,n] == (n+1)*A[d,0] would allow the structured
 *                          one; 0 = automatic (default).
 *   SSM_OPT_PROFILE      : see ssm_profile_read below.
 *   SSM_OPT_STEP_CHANNELS: work per thread of the decode step.
 */
typedef enum {
    SSM_OPT_SEGMENT_LEN = 1,
    SSM_OPT_FORCE_GENERAL = 2,
    SSM_OPT_PROFILE = 3,      /* 1 = bracket every kernel launch with HIP events (see below) */
    SSM_OPT_STEP_CHANNELS = 4 /* (b, d) channels each decode-step thread updates, in consecutive batch rows: 1, 2 or 4 (default 4) */
} ssm_option;

int ssm_set_option(int option, int64_t value);
int64_t ssm_get_option(int option);

/*
 * Kernel timing for diagnostics and benchmarks.  While SSM_OPT_PROFILE is 1,
 * each kernel the library launches is bracketed by two HIP events recorded on
 * the stream it is launched on.  ssm_profile_read() waits for the recorded
 * events, writes per-kind totals -- total_ms[k] (milliseconds) and
 * launches[k] for k < n, indexed by ssm_kernel_kind -- and clears them.
 * Either output may be NULL.  Returns SSM_OK or SSM_ERR_HIP.
 */
typedef enum {
    SSM_K_BC_PREP = 0,          /* B/C rows converted for the scan */
    SSM_K_SCAN_AGGREGATE = 1,   /* per-segment end states from a zero start */
    SSM_K_SCAN_CARRY = 2,       /* states entering each segment */
    SSM_K_SCAN_OUTPUT = 3,      /* y (and h_final) from the entering states */
    SSM_K_STEP = 4,             /* decode step */
    SSM_K_STATE_INIT = 5,       /* h_final (or dh_init) of empty sequences; zero fills;
                                   sequence-start masks of a packed backward */
    SSM_K_BWD_AGGREGATE = 6,    /* backward: per-segment adjoint summaries */
    SSM_K_BWD_CARRY = 7,        /* backward: adjoint entering each segment */
    SSM_K_BWD_MAIN = 8,         /* backward: gradients per segment */
    SSM_K_BWD_REDUCE = 9,       /* backward: dB, dC, dA, dD sums */
    SSM_K_SSD_AGGREGATE = 10,   /* scalar-decay layer: per-segment end states */
    SSM_K_SSD_CARRY = 11,       /* scalar-decay layer: states entering each segment */
    SSM_K_SSD_OUTPUT = 12,      /* scalar-decay layer: y (and h_final) per chunk */
    SSM_K_COUNT = 13
} ssm_kernel_kind;

int ssm_profile_read(double *total_ms, int64_t *launches, int n);

/*
 * How ssm_scan_fwd would cut a problem: number of time segments and their
 * length, for a device with `compute_units` CUs (0 = ask the current device).
 * Returns SSM_OK or an argument error; makes no device call unless
 * compute_units == 0.
 */
int ssm_scan_plan(int64_t Bsz, int64_t L, int64_t Dm, int64_t N, int dtype,
                  int compute_units, int64_t *segments, int64_t *segment_len);

/*
 * How ssm_scan_bwd would cut a problem: the number of fixed-length time
 * segments and their length (32 steps for bf16 storage, 16 for fp32), and how
 * the main backward pass groups them: each group of `seg_per_group`
 * consecutive segments is walked by one block, from the last segment to the
 * first, carrying the adjoint between them in registers; `groups` =
 * ceil(segments / seg_per_group).  For a device with `compute_units` CUs
 * (0 = ask the current device).  Returns SSM_OK or an argument error; makes
 * no device call unless compute_units == 0.
 */
int ssm_scan_bwd_plan(int64_t Bsz, int64_t L, int64_t Dm, int64_t N, int dtype,
                      int compute_units, int64_t *segments, int64_t *segment_len,
                      int64_t *seg_per_group, int64_t *groups);

/*
 * Issue-rate probes, for calibrating the arithmetic roofline the scan kernels
 * are measured against (they compute nothing of the scan).  Launches `blocks`
 * blocks of 256 threads on `stream`; every thread runs `iters` iterations of
 * a fixed instruction mix in 16 independent dependency chains:
 *   SSM_PROBE_FMA_F32     : 64 v_fma_f32
 *   SSM_PROBE_EXP_F32     : 16 v_exp_f32
 *   SSM_PROBE_FMA_EXP_F32 : 64 v_fma_f32 and 16 v_exp_f32 (independent)
 *   SSM_PROBE_FMA_F64     : 32 v_fma_f64
 *   SSM_PROBE_EMPTY       : nothing (launch overhead)
 *   SSM_PROBE_FMAC_F32    : 64 v_fmac_f32 (two-operand accumulate form, VGPRs)
 *   SSM_PROBE_MUL_F32     : 64 v_mul_f32
 *   SSM_PROBE_ADD_F32     : 64 v_add_f32
 *   SSM_PROBE_FMA_F32_VGPR: 64 v_fma_f32 with VGPR operands only
 *   SSM_PROBE_SCAN_STEP_MIX: one structured-A output step of the scan for
 *                           N = 16 without memory traffic: 63 FMAs and
 *                           1 v_exp_f32 (64 reported), the B/C row as scalar
 *                           operands; one iteration is one wave-step
 * *valu_per_iter and *trans_per_iter (either may be NULL) receive the VALU
 * instructions per iteration (transcendentals included) and the
 * transcendental ones.  `sink` is a device buffer of blocks * 256 floats that
 * the kernel may write (it keeps the chains live).  The caller times the
 * launch.  Returns SSM_OK, SSM_ERR_BAD_DIM (blocks or iters outside [1, 2^24]),
 * SSM_ERR_NULLPTR, SSM_ERR_BAD_OPTION (unknown kind) or SSM_ERR_HIP.
 */
typedef enum {
    SSM_PROBE_FMA_F32 = 0,
    SSM_PROBE_EXP_F32 = 1,
    SSM_PROBE_FMA_EXP_F32 = 2,
    SSM_PROBE_FMA_F64 = 3,
    SSM_PROBE_EMPTY = 4,
    SSM_PROBE_FMAC_F32 = 5,
    SSM_PROBE_MUL_F32 = 6,
    SSM_PROBE_ADD_F32 = 7,
    SSM_PROBE_FMA_F32_VGPR = 8,
    SSM_PROBE_SCAN_STEP_MIX = 9,
    SSM_PROBE_HBM_READ = 16,   /* ssm_probe_hbm: read `bytes` */
    SSM_PROBE_HBM_RMW = 17,    /* ssm_probe_hbm: read and write back `bytes` in place */
    SSM_PROBE_HBM_WRITE = 18   /* ssm_probe_hbm: write `bytes` */
} ssm_probe_kind;

int ssm_probe_issue(int kind, int64_t blocks, int64_t iters, float *sink, void *stream,
                    int64_t *valu_per_iter, int64_t *trans_per_iter);

/*
 * Streaming memory probes, for the practical HBM ceiling beside the 8 TB/s
 * specification: 16-byte nontemporal buffer loads and/or stores over the
 * device buffer [buf, buf + bytes) (16-byte aligned, bytes a positive multiple
 * of 16), enqueued on `stream` as one launch per 512 MiB.  READ moves `bytes`,
 * RMW (every 32-bit value incremented in place) 2 * bytes, WRITE `bytes`;
 * RMW and WRITE change the buffer.  The caller times the calls.  Returns
 * SSM_OK, SSM_ERR_BAD_OPTION, SSM_ERR_NULLPTR, SSM_ERR_ALIGN or SSM_ERR_HIP.
 */
int ssm_probe_hbm(int kind, void *buf, int64_t bytes, void *stream);

/* Free all library scratch memory (all devices and streams), including
 * buffers kept for captured HIP graphs: graphs captured with library calls
 * must not be replayed afterwards.  The caller must make sure no library work
 * is still running. */
int ssm_release_workspaces(void);

#ifdef __cplusplus
}
#endif

#endif /* SSMSCAN_H */
