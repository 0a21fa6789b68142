// Scan with one scalar decay per head (the state-space-duality layer) in its
// chunked matrix form on the gfx950 matrix cores.  Templates shared by
// ssd_bf16.hip and ssd_f32.hip.
//
// The bitig.info page on Mamba-3 (section "Karmasik Degerli Durum
// Guncellemesi") says Mamba-2 reduced the state transition to real scalars;
// the "Mamba SSM Nedir?" page (section "Mamba-2 ve Guncel Gelismeler") states
// that such an SSM equals a masked attention.  With heads of 64 channels, a
// scalar a = A[h] and per-step dt_t of the head, inside a chunk of 64 steps
// starting from the state H (N x 64, one column per channel):
//   c_t    = a * (dt_0 + ... + dt_t)                (log of the decay so far)
//   k_s    = (exp(a dt_s) - 1) / a                  (dt_s at a = 0, or Euler)
//   y_t    = exp(c_t) C_t H + sum_{s<=t} (C_t . B_s) exp(c_t - c_s) k_s x_s + D x_t
//   H_next = exp(c_63) H + sum_s B_s^T exp(c_63 - c_s) k_s x_s
// Every exponent is <= 0 for a <= 0, so nothing overflows.  The four products
// -- G = B C^T over N, (G o mask) x over the chunk, C H over N and B^T (w x)
// over the chunk -- are 32x32 tiles of v_mfma_f32_32x32x16_bf16.  B, C and x
// are exact bf16 operands; the fp32 operand of each product (the masked G,
// the state H, the weighted x) is split into hi + lo bf16 halves, two
// instructions, leaving about 2^-17 relative error per product.
//
// fp32 storage takes the recurrence itself in fp64 instead (one thread per
// channel and 8 states): fp32 matrix instructions accumulate in fp32, whose
// rounding does not keep the fp32 storage path's error bound.
//
// Layout of work: a block of 4 waves serves two heads of one batch row over a
// segment of chunks; wave w takes head w/2 and channels 32 (w%2) .. +32 of
// it.  Chunk inputs are staged in LDS as stored (one row per step), moved
// there by buffer loads that write LDS directly, while the previous chunk is
// computed; operands whose contraction runs over the steps (x, and B for the
// state update) are read from those rows with gfx950's transposing LDS load,
// the others as two 8-byte pieces per lane.
// Time is cut into segments joined as in the diagonal scan: an aggregate pass
// (end state of each segment from zero, and its total log decay), a carry
// pass, and an output pass that reruns each segment from its entering state.
#pragma once

#include <type_traits>

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {

namespace {

constexpr int kSsdQ = 64;       // chunk length (steps)
constexpr int kSsdP = 64;       // channels per head
constexpr int kSsdHeads = 2;    // heads per block
constexpr int kSsdBlock = 256;  // 4 waves

// LDS row pitch (bf16 elements) for rows of w elements: the pitch in dwords,
// modulo the 64 banks, lies in {10, 14, 18, 26, 38, 46, 50, 54}.  Then 32
// consecutive rows read at one column (row fragments) hit 32 distinct bank
// pairs, and 4 consecutive rows read as 32-byte runs (transposing reads) hit
// 4 disjoint 8-bank ranges.
constexpr bool ssd_pitch_ok(int dw) {
    const int r = dw % 64;
    return r == 10 || r == 14 || r == 18 || r == 26 || r == 38 || r == 46 || r == 50 || r == 54;
}
constexpr int ssd_pitch(int w) {
    int dw = w / 2;
    while (!ssd_pitch_ok(dw)) ++dw;
    return 2 * dw;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// A matrix-operand fragment: 8 k-slots per lane.  For a K = 16 step starting
// at k0, lane group g = lane / 32 holds k0 + 4g + (0..3) in slots 0..3 and
// k0 + 8 + 4g + (0..3) in slots 4..7.  (The instruction pairs slot e of group
// g with hardware k = 8g + e in bf16, or issues one K = 2 instruction per
// slot in fp32; either way A and B fragments built with the same slot order
// contract over k0 .. k0 + 15.)  This order matches the rows a 32x32
// accumulator holds per lane, so accumulators become operands in place.
template <typename T>
struct Frag;
template <>
struct Frag<bf16> {
    bf16x8_t v;
};

__device__ __forceinline__ void mma(f32x16_t &acc, const Frag<bf16> &a, const Frag<bf16> &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}

// v = hi + lo + r with hi, lo bf16 and |r| <= 2^-18 |v|: pairs are rounded
// to nearest even by one packed conversion, and hi is read back as fp32 from
// the packed word (a shift and a mask) for the remainder.
__device__ __forceinline__ void split(const float (&v)[8], Frag<bf16> &hi, Frag<bf16> &lo) {
    u32x4_t h, l;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f32x2_t ab = {v[2 * k], v[2 * k + 1]};
        const unsigned hp = __builtin_bit_cast(unsigned, __builtin_convertvector(ab, bf16x2_t));
        const f32x2_t r = {v[2 * k] - __builtin_bit_cast(float, hp << 16),
                           v[2 * k + 1] - __builtin_bit_cast(float, hp & 0xffff0000u)};
        h[k] = hp;
        l[k] = __builtin_bit_cast(unsigned, __builtin_convertvector(r, bf16x2_t));
    }
    hi.v = __builtin_bit_cast(bf16x8_t, h);
    lo.v = __builtin_bit_cast(bf16x8_t, l);
}

// The fragment of one LDS row (matrix row or column, k contiguous) for the
// K = 16 step at k0.
__device__ __forceinline__ Frag<bf16> lds_frag(const bf16 *row, int k0, int g) {
    const uint2 a = *reinterpret_cast<const uint2 *>(row + k0 + 4 * g);
    const uint2 b = *reinterpret_cast<const uint2 *>(row + k0 + 8 + 4 * g);
    const u32x4_t u = {a.x, a.y, b.x, b.y};
    Frag<bf16> f;
    f.v = __builtin_bit_cast(bf16x8_t, u);
    return f;
}
// The fragment of the K = 16 step at row k0 of a row-major LDS matrix (rows
// = k, pitch in elements) for the 32 columns col0 .. col0 + 31, one column
// per lane (lane % 32), read with the transposing LDS load: within each 16-lane
// group, lane m addresses row r0 + m/4, columns c0 + 4 (m%4) .. + 3, and lane
// i receives column c0 + i of rows r0 .. r0 + 3.  Two such loads fill slots
// 0..3 (rows k0 + 4g + 0..3) and 4..7 (rows k0 + 8 + 4g + 0..3).
__device__ __forceinline__ Frag<bf16> tr_frag(const bf16 *base, int pitch, int k0, int col0, int lane) {
    const int row = k0 + 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const bf16 *q = base + row * pitch + col;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)q);
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(q + 8 * pitch));
    const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
    const u32x4_t u = {a.x, a.y, b.x, b.y};
    Frag<bf16> f;
    f.v = __builtin_bit_cast(bf16x8_t, u);
    return f;
}
__device__ __forceinline__ float frag_elem(const Frag<bf16> &f, int e) { return static_cast<float>(f.v[e]); }

// 8 slot values from an LDS array of floats indexed by k.
__device__ __forceinline__ void lds_slots(const float *v, int k0, int g, float (&o)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(v + k0 + 4 * g);
    const float4 b = *reinterpret_cast<const float4 *>(v + k0 + 8 + 4 * g);
    o[0] = a.x, o[1] = a.y, o[2] = a.z, o[3] = a.w;
    o[4] = b.x, o[5] = b.y, o[6] = b.z, o[7] = b.w;
}

// exp(z) - 1 on the transcendental unit (relative error near 1e-7).
__device__ __forceinline__ float ssd_expm1(float z) {
    float e;
    return expm1_and_exp(z, e);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;

// Rows 0..63 of a chunk operand (row r at byte r * row_bytes of the
// descriptor, kRowDw dwords each) into LDS rows `pitch` elements apart: one
// dword load per row that writes straight into LDS (lane l moves dword l to
// the row start + 4 l), rows dealt out to the 4 waves.  The row offset goes in
// the scalar offset, which the descriptor's range check includes: bytes
// outside the range arrive as zeros.  Nothing waits here: the caller waits
// for the vector-memory counter before the rows are read.
template <int kRowDw>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t r, bf16 *dst, int pitch, int32_t row_bytes, int wave,
                                         int lane) {
    static_assert(kRowDw == 16 || kRowDw == 32 || kRowDw == 64, "rows of 16, 32 or 64 dwords");
    // The row addresses are the same in every chunk; hidden behind the empty
    // asm they are formed here (a scalar add each) rather than hoisted out of
    // the chunk loop, where they would not fit in scalar registers.
    lds_char_t *base = (lds_char_t *)dst;
    __asm__ volatile("" : "+s"(base), "+s"(row_bytes));
#pragma unroll
    for (int i = 0; i < kSsdQ / 4; ++i) {
        const int row = wave + 4 * i;
        if (kRowDw == 64 || lane < kRowDw)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(base + row * pitch * (int)sizeof(bf16)), 4,
                                                     lane * 4, row * row_bytes, 0, 0);
    }
}
// Wait until every vector-memory operation of this wave (the row loads above
// among them) has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// A barrier for handing LDS buffers between waves: this wave's LDS accesses
// are complete and every wave has arrived.  Unlike __syncthreads it does not
// wait for the wave's vector-memory operations (row loads into LDS still in
// flight, stores), which its release fence would.  The empty asm statements
// keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// The state tiles of one wave (N x 32, fp32) to or from [Bsz][Dm][N]
// memory: lane (channel, g) holds n = 32 nt + 8 m + 4 g + (0..3) in
// registers 4m .. 4m+3 of tile nt -- four 16-byte pieces per tile.
template <int N>
__device__ __forceinline__ void state_load(f32x16_t (&hs)[N / 32], const float *src, int g) {
#pragma unroll
    for (int nt = 0; nt < N / 32; ++nt)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float4 v = *reinterpret_cast<const float4 *>(src + 32 * nt + 8 * m + 4 * g);
            hs[nt][4 * m] = v.x, hs[nt][4 * m + 1] = v.y, hs[nt][4 * m + 2] = v.z, hs[nt][4 * m + 3] = v.w;
        }
}
template <int N>
__device__ __forceinline__ void state_store(const f32x16_t (&hs)[N / 32], float *dst, int g) {
#pragma unroll
    for (int nt = 0; nt < N / 32; ++nt)
#pragma unroll
        for (int m = 0; m < 4; ++m)
            *reinterpret_cast<float4 *>(dst + 32 * nt + 8 * m + 4 * g) =
                make_float4(hs[nt][4 * m], hs[nt][4 * m + 1], hs[nt][4 * m + 2], hs[nt][4 * m + 3]);
}

// LDS of one block, chunk rows as stored (row = step) at the pitches above,
// one __shared__ array per buffer so that the compiler can tell them apart
// (it then inserts no wait for a row load in flight into one buffer before
// reading another).
//
// Output pass (two blocks per compute unit): x (the block's 128 channels)
// and the step scalars are double-buffered -- the next chunk's rows arrive
// while the current chunk is in use, the chunk loop unrolled by two so that
// each buffer's role is fixed in each half -- and the single B and C buffers
// are refilled as soon as every wave is done with them.  sc holds, per head:
// c_t log2(e), k_t, w_t, exp(c_t), exp(-c_t) k_t.
//
// Aggregate pass (four blocks per compute unit, no C): one buffer each, rows
// loaded and then used; the other resident blocks cover the wait.  Each wave
// keeps its w_t in a row of its own.
template <typename T, int N, bool kOut>
__global__ __launch_bounds__(kSsdBlock, kOut ? 2 : 4) void ssd_chunk_kernel(SsdParams p) {
    static_assert(std::is_same<T, bf16>::value, "the matrix-core path stores bf16");
    constexpr int kNT = N / 32;  // 32-row state tiles
    constexpr int kNS = N / 16;  // K = 16 steps over the state
    constexpr int kPX = ssd_pitch(kSsdHeads * kSsdP);
    constexpr int kPN = ssd_pitch(N);
    constexpr int kScH = kOut ? kSsdHeads : 1, kScR = kOut ? 5 : 1, kScQ = kOut ? kSsdQ : 1;
    typedef float Scalars[kScH][kScR][kScQ];
    __shared__ __attribute__((aligned(16))) bf16 lx0[kSsdQ * kPX];
    __shared__ __attribute__((aligned(16))) bf16 lx1[(kOut ? kSsdQ : 1) * kPX];
    __shared__ __attribute__((aligned(16))) bf16 lb0[kSsdQ * kPN];
    __shared__ __attribute__((aligned(16))) bf16 lc[(kOut ? kSsdQ : 1) * kPN];
    __shared__ __attribute__((aligned(16))) Scalars lsc0;
    __shared__ __attribute__((aligned(16))) Scalars lsc1;
    __shared__ __attribute__((aligned(16))) float lw[kOut ? 1 : kSsdBlock / kWave][kSsdQ];
    static_assert(kOut ? 2 * kSsdQ * kPX * 2 + 2 * kSsdQ * kPN * 2 + 2 * (int)sizeof(Scalars) + 4 * 64 <= 81920
                       : kSsdQ * kPX * 2 + kSsdQ * kPN * 2 + 4 * kSsdQ * 4 + 64 <= 40960,
                  "the blocks resident on one compute unit must fit its 160 KB of LDS");
    // The row buffers are written only by the row loads, which the compiler
    // does not count as stores to them: let their addresses escape so that
    // reads of them are not folded away.
    __asm__ volatile("" ::"s"(lx0), "s"(lx1), "s"(lb0), "s"(lc) : "memory");

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int hh = wave >> 1;   // head of the block
    const int dh = wave & 1;    // channel half of the head
    const int g = lane >> 5;
    const int li = lane & 31;

    const int nhp = (int)((p.H + kSsdHeads - 1) / kSsdHeads);
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int hp = lb % nhp;
    const int rest = lb / nhp;
    const int64_t b = rest % p.Bsz;
    const int seg = (int)(rest / p.Bsz);
    const int heads_here = (int)(p.H - (int64_t)hp * kSsdHeads < kSsdHeads ? p.H - (int64_t)hp * kSsdHeads : kSsdHeads);
    const bool head_ok = hh < heads_here;
    const int64_t h = (int64_t)hp * kSsdHeads + (head_ok ? hh : 0);
    const int64_t col0 = (int64_t)hp * kSsdHeads * kSsdP;     // first channel of the block
    const int64_t d = h * kSsdP + 32 * dh + li;                // this lane's channel
    const int ncols = heads_here * kSsdP;
    const int64_t BD = p.Bsz * p.Dm;
    const int xcol = kSsdP * hh + 32 * dh;                     // this wave's first column of x rows

    const float a = p.A[h];
    const float bias = p.delta_bias ? p.delta_bias[h] : 0.f;
    const float Dd = p.D[d];

    f32x16_t hs[kNT];
    if (kOut && (p.S > 1 || p.h_init != nullptr)) {
        const float *src = p.S > 1 ? p.gin + ((int64_t)seg * BD + b * p.Dm + d) * N : p.h_init + (b * p.Dm + d) * N;
        state_load<N>(hs, src, g);
    } else {
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) hs[nt][r] = 0.f;
    }

    const int64_t nchunks = (p.L + kSsdQ - 1) / kSsdQ;
    const int64_t cps = p.seg_len / kSsdQ;
    const int64_t ch_begin = (int64_t)seg * cps;
    const int64_t ch_end = ch_begin + cps < nchunks ? ch_begin + cps : nchunks;
    auto rows_of = [&](int64_t c) -> int { return (int)(p.L - c * kSsdQ < kSsdQ ? p.L - c * kSsdQ : kSsdQ); };
    const T *xblk = static_cast<const T *>(p.x) + b * p.L * p.Dm + col0;
    const T *bblk = static_cast<const T *>(p.B) + b * p.L * N;
    const T *cblk = static_cast<const T *>(p.C) + b * p.L * N;

    // ---- operand rows of chunk c into LDS (no wait)
    auto fetch_x = [&](bf16 *dst, int64_t c) {
        const int32_t bytes = (int32_t)(((int64_t)(rows_of(c) - 1) * p.Dm + ncols) * (int64_t)sizeof(T));
        dma_rows<kSsdHeads * kSsdP / 2>(make_rsrc(xblk + c * kSsdQ * p.Dm, bytes), dst, kPX,
                                        (int32_t)(p.Dm * (int64_t)sizeof(T)), wave, lane);
    };
    auto fetch_bc = [&](const T *src, bf16 *dst, int64_t c) {
        dma_rows<N / 2>(make_rsrc(src + c * kSsdQ * N, rows_of(c) * N * (int)sizeof(T)), dst, kPN,
                        N * (int)sizeof(T), wave, lane);
    };

    // ---- delta of step `lane` of chunk c as stored (0 past the sequence or
    // the segment).  It stays in the stored type until used, so that the
    // compiler's wait for it sits at the use, not at the load.
    auto load_delta = [&](int64_t c) -> T {
        const int64_t n = c < ch_end ? rows_of(c) : 0;
        const T *dp = static_cast<const T *>(p.delta) + (b * p.L + c * kSsdQ) * p.H;
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(dp, (int32_t)(n * p.H * (int64_t)sizeof(T)));
        return buf_load<T>(rd, (int32_t)(((int64_t)lane * p.H + h) * (int64_t)sizeof(T)), 0);
    };

    // ---- step scalars of chunk c for this wave's head (lane = step); log
    // decays in base-2 units (c2 = c log2 e) for the exp2 unit.  The output
    // pass keeps all five per head in scw (written by one wave of the head);
    // the aggregate pass needs only w_t, which every wave writes to its own
    // row wrow.  Returns the chunk's total log decay; `split` tells whether
    // the causal mask may be factored (below).
    auto scalars = [&](Scalars &scw, float *wrow, int64_t c, T dstored, bool &split) -> float {
        float dt = 0.f;
        if (lane < rows_of(c)) {
            float v = to_f32(dstored) + bias;
            if (p.delta_softplus) v = softplus_(v);
            dt = v;
        }
        const float la = dt * a;
        float c2 = la * kLog2e;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float o = __shfl_up(c2, off);
            if (lane >= off) c2 += o;
        }
        const float cend2 = __shfl(c2, kWave - 1);
        // |a| below 1e-20 (zero included) takes the exact a -> 0 limit dt
        const float k = (p.euler_b || __builtin_fabsf(a) < 1e-20f) ? dt : ssd_expm1(la) / a;
        // A chunk whose whole decay stays above 2^-64 keeps exp(-c_s) k_s
        // below 2^64 k_s: far inside fp32 range, so the mask factors into a
        // row scale and a column weight.  (cend2 is the same on every lane;
        // the readfirstlane makes the branch scalar.)
        split = __builtin_amdgcn_readfirstlane((int)(cend2 >= -64.f)) != 0;
        if constexpr (!kOut) {
            wrow[lane] = fast_exp2(cend2 - c2) * k;
        } else if (dh == 0) {
            scw[hh][0][lane] = c2;
            scw[hh][1][lane] = k;
            scw[hh][2][lane] = fast_exp2(cend2 - c2) * k;
            scw[hh][3][lane] = fast_exp2(c2);
            scw[hh][4][lane] = split ? fast_exp2(-c2) * k : 0.f;
        }
        return cend2 * 0.6931471805599453f;
    };

    // y of the previous chunk, held until the next chunk's rows are in (so
    // that waiting for those does not wait for these stores): rows t of
    // 32 tt + 8 (r / 4) + 4 g + r % 4 in pair r / 2 of tile tt
    bf16x2_t ypend[2][8];
    int64_t ypend_t0 = -1;
    auto store_y = [&]() {
        T *Yp = static_cast<T *>(p.y) + (b * p.L + ypend_t0) * p.Dm;
        const int nrows = rows_of(ypend_t0 / kSsdQ);
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(Yp, (int32_t)((int64_t)nrows * p.Dm * (int64_t)sizeof(T)));
        const int32_t vrow = (int32_t)(((int64_t)(4 * g) * p.Dm + d) * (int64_t)sizeof(T));
        const int32_t rowb = (int32_t)(p.Dm * (int64_t)sizeof(T));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tq = 32 * tt + 8 * (r / 4) + (r % 4);  // t minus 4g
                buf_store(ypend[tt][r / 2][r % 2], ry, vrow, tq * rowb);
            }
    };

    // ---- H = exp(c_end) H + B^T (w x) over the chunk's rows in xr / br:
    // the hi and lo halves of the weighted x in separate passes over the
    // state tiles
    auto state_update = [&](const bf16 *xr, const bf16 *br, const float *w, float cend) {
        const float decay = fast_exp2(cend * kLog2e);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) hs[nt][r] *= decay;
#pragma unroll
        for (int j = 0; j < kSsdQ / 16; ++j) {
            float wv[8];
            lds_slots(w, 16 * j, g, wv);
            const Frag<T> xj = tr_frag(xr, kPX, 16 * j, xcol, lane);
#pragma unroll
            for (int e = 0; e < 8; ++e) wv[e] *= frag_elem(xj, e);
            Frag<T> whi, wlo;
            split(wv, whi, wlo);
            Frag<T> bt[kNT];
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) bt[nt] = tr_frag(br, kPN, 16 * j, 32 * nt, lane);
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) mma(hs[nt], bt[nt], whi);
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) mma(hs[nt], bt[nt], wlo);
        }
    };

    float dec_total = 0.f;
    float cend_cur = 0.f, cend_next = 0.f;
    bool split_cur = true, split_next = true;

    if constexpr (kOut) {
        // ---- one chunk of the output pass: its rows are in xr / br and lc, its
        // scalars in scr; the next chunk's go to xw / bw / scw
        auto chunk = [&](int64_t ch, const bf16 *xr, bf16 *xw, const bf16 *br, bf16 *bw, const Scalars &scr,
                         Scalars &scw) {
            const bool more = ch + 1 < ch_end;
            wait_vmem();      // this wave's row loads of the chunk have landed
            __syncthreads();  // ... and every wave's; the step scalars are written
            dec_total += cend_cur;
            if (kOut && ypend_t0 >= 0 && head_ok) store_y();
            const T delta_next = load_delta(ch + 1);
            if (more) fetch_x(xw, ch + 1);
            const float(*sc)[kSsdQ] = scr[hh];

            if constexpr (kOut) {
                // ---- y = exp(c_t) (C H) + (G o mask) x + D x over two 32-step row
                // tiles.  One sweep over the state dimension accumulates C H for
                // both row tiles and the three causal tiles of G^T = B C^T (rows
                // s, columns t: (0,0), (0,1), (1,1)), which share the C fragments;
                // hi and lo halves of the split state go in separate passes so
                // that consecutive matrix instructions feed different
                // accumulators.
                f32x16_t yacc[2], g00, g01, g11;
#pragma unroll
                for (int r = 0; r < 16; ++r) yacc[0][r] = yacc[1][r] = g00[r] = g01[r] = g11[r] = 0.f;
                if (head_ok) {
#pragma unroll
                    for (int j = 0; j < kNS; ++j) {
                        const Frag<T> c0 = lds_frag(lc + li * kPN, 16 * j, g);
                        const Frag<T> c1 = lds_frag(lc + (32 + li) * kPN, 16 * j, g);
                        const Frag<T> b0 = lds_frag(br + li * kPN, 16 * j, g);
                        const Frag<T> b1 = lds_frag(br + (32 + li) * kPN, 16 * j, g);
                        float hv[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) hv[e] = hs[j / 2][8 * (j % 2) + e];
                        Frag<T> hhi, hlo;
                        split(hv, hhi, hlo);
                        mma(yacc[0], c0, hhi);
                        mma(yacc[1], c1, hhi);
                        mma(g00, b0, c0);
                        mma(g01, b0, c1);
                        mma(g11, b1, c1);
                        mma(yacc[0], c0, hlo);
                        mma(yacc[1], c1, hlo);
                    }
                }
                // the next chunk's step scalars, here where the wait for its delta
                // only covers what was issued at the top of this chunk
                if (more) cend_next = scalars(scw, nullptr, ch + 1, delta_next, split_next);
                // Let the y stores, the x rows and the delta issued at the top
                // complete now, a sweep after their issue: otherwise the first
                // reuse of a stored register would wait on the vector-memory
                // counter after the row loads below and so for them too.
                wait_vmem();
                lds_barrier();  // every wave is done with C
                if (more) fetch_bc(cblk, lc, ch + 1);
                if (head_ok) state_update(xr, br, sc[2], cend_cur);
                lds_barrier();  // every wave is done with B
                if (more) fetch_bc(bblk, bw, ch + 1);

                if (head_ok) {
                    // y rows times exp(c_t)
                    auto row_scale = [&]() {
#pragma unroll
                        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                            for (int m = 0; m < 4; ++m) {
                                const float4 e4 = *reinterpret_cast<const float4 *>(&sc[3][32 * tt + 8 * m + 4 * g]);
                                yacc[tt][4 * m] *= e4.x, yacc[tt][4 * m + 1] *= e4.y;
                                yacc[tt][4 * m + 2] *= e4.z, yacc[tt][4 * m + 3] *= e4.w;
                            }
                    };
                    // mask and weight the G^T tiles -- M[t][s] = G[s][t] exp(c_t - c_s)
                    // k_s for s <= t (lane = t, registers = s) -- split them, and add
                    // M x, one 16-step half of each 32-step column tile at a time,
                    // alternating the two row tiles.  With the factored decay the
                    // tiles carry only exp(-c_s) k_s and the row scale exp(c_t) is
                    // applied once to C H + M x; otherwise each weight takes its own
                    // exponential and the row scale goes on C H alone.
                    auto mask_mx = [&](auto factored) {
                        constexpr bool kF = decltype(factored)::value;
                        const float ct0 = kF ? 0.f : sc[0][li], ct1 = kF ? 0.f : sc[0][32 + li];
                        // On a diagonal tile, register 4 m + q of this lane holds
                        // s - t = 8 m + q - (li - 4 g): the lane masks of the
                        // compares depend on the lane alone.  Formed here (one
                        // compare each) instead of hoisted out of the chunk loop,
                        // where they would not fit in scalar registers.
                        int diag = li - 4 * g;
                        __asm__ volatile("" : "+v"(diag));
                        auto masked = [&](const f32x16_t &gt, int st, int tt, float ct, int hf, Frag<T> &mh,
                                          Frag<T> &ml) {
                            float mv[8];
#pragma unroll
                            for (int m2 = 0; m2 < 2; ++m2) {
                                const int m = 2 * hf + m2;
                                const int s0 = 32 * st + 8 * m + 4 * g;
                                float ws[4];
                                if constexpr (kF) {
                                    const float4 w4 = *reinterpret_cast<const float4 *>(&sc[4][s0]);
                                    ws[0] = w4.x, ws[1] = w4.y, ws[2] = w4.z, ws[3] = w4.w;
                                } else {
                                    const float4 c4 = *reinterpret_cast<const float4 *>(&sc[0][s0]);
                                    const float4 k4 = *reinterpret_cast<const float4 *>(&sc[1][s0]);
                                    ws[0] = fast_exp2(ct - c4.x) * k4.x, ws[1] = fast_exp2(ct - c4.y) * k4.y;
                                    ws[2] = fast_exp2(ct - c4.z) * k4.z, ws[3] = fast_exp2(ct - c4.w) * k4.w;
                                }
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    const float v = gt[4 * m + q] * ws[q];
                                    // below the diagonal tile every entry is kept
                                    mv[4 * m2 + q] = (st < tt || 8 * m + q <= diag) ? v : 0.f;
                                }
                            }
                            split(mv, mh, ml);
                        };
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf) {
                            const Frag<T> x0 = tr_frag(xr, kPX, 16 * hf, xcol, lane);       // steps 0..31
                            const Frag<T> x1 = tr_frag(xr, kPX, 32 + 16 * hf, xcol, lane);  // steps 32..63
                            Frag<T> h00, l00, h01, l01, h11, l11;
                            masked(g00, 0, 0, ct0, hf, h00, l00);
                            masked(g01, 0, 1, ct1, hf, h01, l01);
                            masked(g11, 1, 1, ct1, hf, h11, l11);
                            mma(yacc[0], h00, x0);
                            mma(yacc[1], h01, x0);
                            mma(yacc[0], l00, x0);
                            mma(yacc[1], h11, x1);
                            mma(yacc[1], l01, x0);
                            mma(yacc[1], l11, x1);
                        }
                    };
                    if (split_cur) {
                        mask_mx(std::true_type{});
                        row_scale();
                    } else {
                        row_scale();
                        mask_mx(std::false_type{});
                    }
                    // + D x, with x from transposing reads of this wave's columns
                    // (slot e of the K = 16 step at 32 tt + 16 hf is the row of
                    // register 8 hf + e of row tile tt), rounded to the stored type
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf) {
                            const Frag<T> xf = tr_frag(xr, kPX, 32 * tt + 16 * hf, xcol, lane);
#pragma unroll
                            for (int e = 0; e < 8; e += 2) {
                                const f32x2_t v = {fma_(Dd, frag_elem(xf, e), yacc[tt][8 * hf + e]),
                                                   fma_(Dd, frag_elem(xf, e + 1), yacc[tt][8 * hf + e + 1])};
                                ypend[tt][(8 * hf + e) / 2] = __builtin_convertvector(v, bf16x2_t);
                            }
                        }
                    ypend_t0 = ch * kSsdQ;
                }
            }
            cend_cur = cend_next;
            split_cur = split_next;
        };

        if (ch_begin < ch_end) {
            const T d0 = load_delta(ch_begin);
            fetch_x(lx0, ch_begin);
            fetch_bc(bblk, lb0, ch_begin);
            fetch_bc(cblk, lc, ch_begin);
            cend_cur = scalars(lsc0, nullptr, ch_begin, d0, split_cur);
        }
        for (int64_t ch = ch_begin; ch < ch_end; ch += 2) {
            // even chunks of the segment read x and the scalars from buffers 0
            // and fill buffers 1, odd ones the other way round
            chunk(ch, lx0, lx1, lb0, lb0, lsc0, lsc1);
            if (ch + 1 < ch_end) chunk(ch + 1, lx1, lx0, lb0, lb0, lsc1, lsc0);
        }
    } else {
        // aggregate pass: rows of the chunk in, then its state update; the
        // delta is fetched one chunk ahead
        float *wrow = lw[kOut ? 0 : wave];
        T delta_next = load_delta(ch_begin);
        for (int64_t ch = ch_begin; ch < ch_end; ++ch) {
            fetch_x(lx0, ch);
            fetch_bc(bblk, lb0, ch);
            const T delta_cur = delta_next;
            delta_next = load_delta(ch + 1);
            wait_vmem();      // this wave's row loads have landed
            __syncthreads();  // ... and every wave's
            bool factored;    // (the aggregate pass has no mask)
            const float cend = scalars(lsc0, wrow, ch, delta_cur, factored);
            dec_total += cend;
            if (head_ok) state_update(lx0, lb0, wrow, cend);
            lds_barrier();    // every wave is done with the rows
        }
    }

    if (!head_ok) return;
    if constexpr (kOut) {
        if (ypend_t0 >= 0) store_y();
        if (seg == p.S - 1 && p.h_final != nullptr) state_store<N>(hs, p.h_final + (b * p.Dm + d) * N, g);
    } else {
        state_store<N>(hs, p.agg + ((int64_t)seg * BD + b * p.Dm + d) * N, g);
        if (dh == 0 && lane == 0) p.dec[(int64_t)seg * p.Bsz * p.H + b * p.H + h] = dec_total;
    }
}

// States entering each segment: gin[0] = h_init (or 0); gin[s] =
// exp(dec[s-1]) gin[s-1] + agg[s-1].  One thread per (b, d, n).
__global__ __launch_bounds__(256) void ssd_carry_kernel(SsdParams p, int N) {
    const int64_t BDN = p.Bsz * p.Dm * N;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= BDN) return;
    const int64_t bd = i / N;
    const int64_t b = bd / p.Dm, d = bd - b * p.Dm;
    const int64_t h = d / kSsdP;
    float s = p.h_init ? p.h_init[i] : 0.f;
    p.gin[i] = s;
    for (int k = 1; k < p.S; ++k) {
        s = fma_(expf(p.dec[(int64_t)(k - 1) * p.Bsz * p.H + b * p.H + h]), s, p.agg[(int64_t)(k - 1) * BDN + i]);
        p.gin[(int64_t)k * BDN + i] = s;
    }
}

template <typename T, int N>
hipError_t ssd_pass_n(SsdPass pass, const SsdParams &p, hipStream_t s) {
    const unsigned nhp = (unsigned)((p.H + kSsdHeads - 1) / kSsdHeads);
    switch (pass) {
        case SsdPass::kAggregate:
            if (p.S <= 1) return hipSuccess;
            hipLaunchKernelGGL((ssd_chunk_kernel<T, N, false>), dim3(nhp * (unsigned)p.Bsz * (unsigned)(p.S - 1)),
                               dim3(kSsdBlock), 0, s, p);
            break;
        case SsdPass::kCarry: {
            if (p.S <= 1) return hipSuccess;
            const int64_t n = p.Bsz * p.Dm * N;
            hipLaunchKernelGGL(ssd_carry_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, N);
            break;
        }
        case SsdPass::kOutput:
            hipLaunchKernelGGL((ssd_chunk_kernel<T, N, true>), dim3(nhp * (unsigned)p.Bsz * (unsigned)p.S),
                               dim3(kSsdBlock), 0, s, p);
            break;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t ssd_pass(SsdPass pass, const SsdParams &p, int N, hipStream_t s) {
    switch (N) {
        case 32: return ssd_pass_n<T, 32>(pass, p, s);
        case 64: return ssd_pass_n<T, 64>(pass, p, s);
        case 128: return ssd_pass_n<T, 128>(pass, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

}  // namespace ssm
