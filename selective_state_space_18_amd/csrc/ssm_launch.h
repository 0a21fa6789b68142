// Kernel parameter blocks and launcher entry points (internal to libssmscan).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace ssm {

// One scan call, as cut by the host planner.  Scratch arrays hold the
// arithmetic type Acc (fp32 for bf16 storage, fp64 for fp32 storage):
//   bc  : [Bsz*L][2N] Acc -- B_t[n] in the first N slots, C_t[n]/(n+1) in the next N
//   agg : [S-1][N+1][Bsz*Dm] Acc -- per segment: end state from a zero start
//         (slots 0..N-1, scaled state g = (n+1) h) and the sum of delta (slot N)
//   gin : [S][N][Bsz*Dm] Acc -- scaled state entering segment s (used when S > 1)
struct ScanParams {
    const void *x, *delta, *B, *C;
    const float *A, *D, *h_init;
    void *y;
    float *h_final;
    void *bc, *agg, *gin;
    int64_t Bsz, L, Dm;
    int64_t seg_len;   // time steps per segment (last one may be shorter)
    int S;             // number of segments
    int tiles_per_b;   // ceil(Dm / 64): 64-channel wave tiles per batch row
    int n_tiles;       // Bsz * tiles_per_b
    int waves_per_block;
    int force_general; // 1: never take the structured-A path
    // Packed variable-length input (Bsz == 1): cu[0..nseq] are the sequence
    // start offsets; the state restarts at each start from h_init[k] (or 0)
    // and h_final[k] receives each sequence's last state.  nullptr: one
    // sequence per batch row.
    const int64_t *cu;
    int64_t nseq;
    int *seg_reset;    // [S]: 1 if a sequence starts inside segment s (varlen only)
    // delta as stored -> delta as used: + delta_bias[d] (if not null), then
    // softplus (if delta_softplus).  Neither: delta is used as stored.
    const float *delta_bias;
    int delta_softplus;
    int euler_b;       // 1: input term Bbar = delta B (else the ZOH term)
};

struct StepParams {
    const void *x, *delta, *B, *C;
    const float *A, *D;
    float *h;
    void *y;
    int64_t Bsz, Dm;
    const float *delta_bias;  // as in ScanParams
    int delta_softplus;
    int euler_b;
};

// The passes of one scan call, in launch order.
enum class ScanPass { kPrep, kAggregate, kCarry, kOutput };

// One backward call.  f holds the forward inputs, the segment plan and the
// forward scratch (bc, agg, gin); the forward aggregate and carry passes run
// on it unchanged.  Scratch of the backward (Acc = AccOf<T>):
//   ragg  : [S][N+1][B*D] Acc -- per segment s >= 1: the adjoint a zero
//           incoming adjoint leaves at the segment start (times Abar there,
//           scaled-state units) and the sum of delta
//   gout  : [groups][N][B*D] Acc -- adjoint entering the last segment of
//           each group of segments from the right (the main pass carries it
//           through the group)
//           (scaled-state units: dL/dg = dL/dh / (n+1))
//   part_bc : [2 paths][blocks per row][2 (dB, dC)][B*L*N] Acc -- per block
//           sums over its channels
//   part_a  : [groups][B*D][N] Acc -- dA per group of segments (final form)
//   part_d  : [groups][B*D][2] Acc -- dD and d(delta_bias)
//   part_on : [2 paths][blocks per row][B][groups] int -- 1 where the block
//           wrote its part_bc rows, 0 where it had no wave of its path (its
//           rows are then not written and not read)
// Packed sequences (f.cu set, B = 1): f.h_init, dh_final and dh_init are
// [nseq][D][N]; f.seg_reset serves the forward carry and
//   seg_starts : [S] uint32 -- bit i set where a sequence starts at step
//           s * seg_len + i (the reverse carry takes the summary alone of a
//           segment with a start; the aggregate and main passes restart the
//           adjoint, and the state, there)
struct BwdParams {
    ScanParams f;
    const void *dy;          // [B,L,D] storage dtype
    const float *dh_final;   // [B,D,N] or null
    void *dx, *ddelta;       // [B,L,D] storage dtype
    float *dA, *dB, *dC, *dD, *ddelta_bias, *dh_init;
    void *ragg, *gout, *part_bc, *part_a, *part_d;
    int *part_on;
    uint32_t *seg_starts;
    int seg_per_group;       // segments one wave processes in turn
    int n_groups;            // ceil(S / seg_per_group)
    int blocks_per_row;      // ceil(tiles_per_b / 4)
};

// kStarts: the per-segment sequence-start masks (packed sequences only).
enum class BwdPass { kStarts, kAggregate, kCarry, kMain, kReduce };

// Complex diagonal A (cplx_kernels.h).  ScanParams as for the real scan, with
// A [Dm][N][2], h_init/h_final [Bsz][Dm][N][2] as (re, im) pairs and scratch
// bc [Bsz*L][2N], agg [S-1][2N+1][Bsz*Dm], gin [S][2N][Bsz*Dm] (Acc).
// StepParams likewise (h [Bsz][Dm][N][2]).
hipError_t cplx_pass_f32(ScanPass pass, const ScanParams &p, int N, hipStream_t s);
hipError_t cplx_pass_bf16(ScanPass pass, const ScanParams &p, int N, hipStream_t s);
hipError_t cplx_step_f32(const StepParams &p, int N, hipStream_t s);
hipError_t cplx_step_bf16(const StepParams &p, int N, hipStream_t s);
// Backward of the complex-A scan (cbwd_kernels.h), segments of
// cbwd_segment_len() steps.  BwdParams as for the real backward, with A,
// dA [Dm][N][2], h_init, dh_final, dh_init [Bsz][Dm][N][2] and scratch
//   ragg    : [S][2N+1][B*D] Acc (adjoint summaries, re/im at 2n, 2n+1)
//   gout    : [groups][2N][B*D] Acc
//   part_bc : [blocks per row][2][B*L*N] Acc, written by every block
//   part_a  : [groups][B*D][2N] Acc
// blocks_per_row = ceil(tiles_per_b / cbwd_tiles_per_block(dtype, N)); the
// main kernel's blocks fit cbwd_blocks_per_cu(dtype) to a compute unit.
// kStarts is not used.
int cbwd_segment_len();
int cbwd_tiles_per_block(int dtype, int N);
int cbwd_blocks_per_cu(int dtype);
hipError_t cbwd_pass_f32(BwdPass pass, const BwdParams &q, int N, hipStream_t s);
hipError_t cbwd_pass_bf16(BwdPass pass, const BwdParams &q, int N, hipStream_t s);

// Scalar decay per head, chunked matrix form (ssd_kernels.h).  x, y
// [Bsz][L][Dm]; delta [Bsz][L][H]; A, delta_bias [H]; D [Dm]; B, C
// [Bsz][L][N]; h_init, h_final [Bsz][Dm][N]; heads of 64 channels.  Scratch
// (fp32): agg [S-1][Bsz*Dm][N] end state of each segment from zero, dec
// [S-1][Bsz][H] its total log decay, gin [S][Bsz*Dm][N] the state entering it.
struct SsdParams {
    const void *x, *delta, *B, *C;
    const float *A, *D, *delta_bias, *h_init;
    void *y;
    float *h_final;
    float *agg, *dec, *gin;
    int64_t Bsz, L, Dm, H;
    int64_t seg_len;   // a multiple of the 64-step chunk
    int S;
    int delta_softplus;
    int euler_b;
};
enum class SsdPass { kAggregate, kCarry, kOutput };
hipError_t ssd_pass_f32(SsdPass pass, const SsdParams &p, int N, hipStream_t s);
hipError_t ssd_pass_bf16(SsdPass pass, const SsdParams &p, int N, hipStream_t s);

// Segment length the backward kernels are built for (the plan must use it).
int bwd_segment_len(int dtype);
// Per storage type and layout, one translation unit each: bwd_f32.hip,
// bwd_f32_packed.hip, bwd_bf16.hip, bwd_bf16_packed.hip.
hipError_t bwd_pass_f32(BwdPass pass, const BwdParams &q, int N, hipStream_t s);
hipError_t bwd_pass_f32_packed(BwdPass pass, const BwdParams &q, int N, hipStream_t s);
hipError_t bwd_pass_bf16(BwdPass pass, const BwdParams &q, int N, hipStream_t s);
hipError_t bwd_pass_bf16_packed(BwdPass pass, const BwdParams &q, int N, hipStream_t s);

// Bytes per element of the scan's arithmetic type for a storage dtype.
size_t scan_acc_bytes(int dtype);

// Per storage type and layout (dense batch / packed sequences), one
// translation unit each: scan_f32.hip, scan_f32_packed.hip, scan_bf16.hip,
// scan_bf16_packed.hip.
hipError_t scan_pass_f32(ScanPass pass, const ScanParams &p, int N, hipStream_t s);
hipError_t scan_pass_f32_packed(ScanPass pass, const ScanParams &p, int N, hipStream_t s);
hipError_t scan_pass_bf16(ScanPass pass, const ScanParams &p, int N, hipStream_t s);
hipError_t scan_pass_bf16_packed(ScanPass pass, const ScanParams &p, int N, hipStream_t s);

// dtype: 0 = fp32, 1 = bf16.  N in {1,2,4,8,16}.  All return hipSuccess or the
// launch error.
hipError_t launch_bc_prep(const ScanParams &p, int N, int dtype, hipStream_t s);
hipError_t launch_scan_aggregate(const ScanParams &p, int N, int dtype, hipStream_t s);
hipError_t launch_scan_carry(const ScanParams &p, int N, int dtype, hipStream_t s);
hipError_t launch_scan_output(const ScanParams &p, int N, int dtype, hipStream_t s);
hipError_t launch_state_init(const ScanParams &p, int N, hipStream_t s);
// h_final of the empty sequences of a packed variable-length call.
hipError_t launch_varlen_empty(const ScanParams &p, int N, hipStream_t s);
hipError_t launch_step(const StepParams &p, int N, int dtype, hipStream_t s);
// dst[0..count) = v.
hipError_t launch_fill(float *dst, int64_t count, float v, hipStream_t s);
// Channels per thread of the decode-step kernel (1, 2 or 4).
void set_step_unroll(int u);

// The dense scan with initial state (ssm_scan_fwd_ex's arguments) on scratch
// of fixed capacity `cap` bytes instead of the per-stream buffer: resolve(dev,
// &ptr) gives its address on device dev after the arguments are validated.
// The segment plan is shortened until its scratch fits; calls that do not fit
// with one segment fail with SSM_ERR_BAD_DIM.  Allocates nothing and creates
// no timing events.  Returns an ssm_status (abi.cpp).
int scan_fwd_fixed_scratch(const void *x, const void *delta, const float *A, const void *B, const void *C,
                           const float *D, const float *h_init, void *y, float *h_final, int64_t Bsz, int64_t L,
                           int64_t Dm, int64_t N, int dtype, void *stream, size_t cap,
                           int (*resolve)(int dev, void **ptr));
// Records `msg` as the calling thread's last error and returns `code`.
int set_error(int code, const char *msg);

}  // namespace ssm
