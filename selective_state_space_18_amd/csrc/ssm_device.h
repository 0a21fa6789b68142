// Device-side helpers shared by the libssmscan kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// Stand-in used for |A| < 1e-20 (A == 0 included) in the general-A path: the
// ZOH input coefficient (exp(z)-1)/A then evaluates to its A -> 0 limit delta
// (z = delta*A is tiny and expm1 is accurate there), and 1/A stays finite.
constexpr float kTinyA = -1e-20f;

typedef __bf16 bf16;

// Arithmetic type per storage type.  bf16 storage: fp32 state and arithmetic.
// fp32 storage: fp64 state and arithmetic (CDNA4 issues fp64 FMA at the
// non-packed fp32 rate), rounded to fp32 only when written out.
template <typename T>
struct AccOf;
template <>
struct AccOf<bf16> {
    typedef float type;
};
template <>
struct AccOf<float> {
    typedef double type;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename T>
__device__ __forceinline__ T from_acc(float v);
template <typename T>
__device__ __forceinline__ T from_acc(double v);
template <>
__device__ __forceinline__ float from_acc<float>(float v) { return v; }
template <>
__device__ __forceinline__ float from_acc<float>(double v) { return static_cast<float>(v); }
// v_cvt_pk_bf16_f32: round to nearest even
template <>
__device__ __forceinline__ bf16 from_acc<bf16>(float v) { return static_cast<bf16>(v); }
template <>
__device__ __forceinline__ bf16 from_acc<bf16>(double v) { return static_cast<bf16>(static_cast<float>(v)); }

__device__ __forceinline__ float fma_(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fma_(double a, double b, double c) { return __builtin_fma(a, b, c); }
__device__ __forceinline__ float abs_(float a) { return __builtin_fabsf(a); }
__device__ __forceinline__ double abs_(double a) { return __builtin_fabs(a); }

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// exp(z) - 1, also returning exp(z) in `e`.
//  fp64: ocml expm1 / exp.
//  fp32: exp2 on the transcendental unit, and for |z| < 2^-6 the cubic Taylor
//        polynomial z(1 + z/2 + z^2/6), whose truncation error there is below
//        z^4/24 (relative 2e-7).  This keeps the ZOH input coefficient
//        (exp(z)-1)/A accurate when delta*A is small, where exp(z)-1 alone
//        would cancel.
__device__ __forceinline__ double expm1_and_exp(double z, double& e) {
    const double m = expm1(z);
    e = m + 1.0;
    return m;
}
__device__ __forceinline__ float expm1_and_exp(float z, float& e) {
    e = fast_exp2(z * kLog2e);
    const float poly = z * __builtin_fmaf(z, __builtin_fmaf(z, 1.0f / 6.0f, 0.5f), 1.0f);
    return (__builtin_fabsf(z) < 0.015625f) ? poly : (e - 1.0f);
}

// The same for an argument already in base-2 units (z2 = z log2(e)), which
// saves the scaling multiply: the cubic is z(1 + z/2 + z^2/6) with z = z2 ln2
// folded into its coefficients, used for |z| < 2^-6.
__device__ __forceinline__ float expm1_and_exp2(float z2, float& e) {
    constexpr float c1 = 0.6931471805599453f;        // ln2
    constexpr float c2 = 0.2402265069591007f;        // ln2^2 / 2
    constexpr float c3 = 0.05550410866482158f;       // ln2^3 / 6
    e = fast_exp2(z2);
    const float poly = z2 * __builtin_fmaf(z2, __builtin_fmaf(z2, c3, c2), c1);
    return (__builtin_fabsf(z2) < 0.015625f * kLog2e) ? poly : (e - 1.0f);
}
__device__ __forceinline__ double expm1_and_exp2(double z, double& e) { return expm1_and_exp(z, e); }

// exp2(z2) - 1 as a plain difference, for fp32 callers that know |z| >= 2^-13
// (|z2| >= kExpm1DirectZ2) on every lane.  exp2 is accurate to about an ulp
// (2^-24 near 1), so the difference carries a relative error of at most about
// 2 * 2^-24 / 2^-13 = 2^-10 at the threshold, falling as 1/|z| above it: half
// an ulp of the bf16 outputs of the kernels that use it, at worst.
constexpr float kExpm1DirectZ2 = 1.4426950408889634f / 8192.0f;
__device__ __forceinline__ float expm1_direct_exp2(float z2, float& e) {
    e = fast_exp2(z2);
    return e - 1.0f;
}

// Raw buffer descriptor over [base, base + bytes): loads outside read 0 and
// stores outside are dropped by the hardware range check.  Word 3 is the
// gfx9-family raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

constexpr int kBufNt = 2;  // buffer cache-policy bit: nontemporal

// kAux: cache-policy bits of the access (0, or kBufNt for data streamed once).
template <typename T, int kAux = 0>
__device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, int32_t voff, int32_t soff) {
    static_assert(sizeof(T) == 2 || sizeof(T) == 4, "bf16 or fp32");
    if constexpr (sizeof(T) == 2)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kAux));
    else
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kAux));
}
// The raw bits of one stored value, one per 32-bit register (a bf16 load
// zero-extends).  Keeping prefetched bf16 values apart like this matters: two
// bf16 packed into one register make the compiler wait for both loads at once.
template <typename T, int kAux = 0>
__device__ __forceinline__ uint32_t buf_load_raw(__amdgpu_buffer_rsrc_t r, int32_t voff, int32_t soff) {
    static_assert(sizeof(T) == 2 || sizeof(T) == 4, "bf16 or fp32");
    if constexpr (sizeof(T) == 2)
        return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kAux);
    else
        return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kAux);
}
template <typename T>
__device__ __forceinline__ float raw_to_f32(uint32_t u) {
    if constexpr (sizeof(T) == 2)
        return __builtin_bit_cast(float, u << 16);  // bf16 -> fp32 is exact
    else
        return __builtin_bit_cast(float, u);
}

template <int kAux = 0>
__device__ __forceinline__ void buf_store(bf16 v, __amdgpu_buffer_rsrc_t r, int32_t voff, int32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, voff, soff, kAux);
}
template <int kAux = 0>
__device__ __forceinline__ void buf_store(float v, __amdgpu_buffer_rsrc_t r, int32_t voff, int32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, kAux);
}

// Accurate fp32 variant (ocml expm1f), for the fp32-storage decode step.
__device__ __forceinline__ float expm1_and_exp_precise(float z, float& e) {
    const float m = expm1f(z);
    e = m + 1.0f;
    return m;
}

// softplus(v) = log(1 + exp(v)) = max(v, 0) + log1p(exp(-|v|)).
//  fp64: ocml log1p / exp.
//  fp32: u = exp(-|v|) on the transcendental unit; log1p(u) is the quartic
//        series u - u^2/2 + u^3/3 - u^4/4 for u < 2^-5 (truncation below
//        u^5/5, relative 2e-7), else log2(1 + u) ln 2 on the transcendental
//        unit (1 + u rounds by at most 2^-24 against a result of at least
//        0.03).  Large v gives u = 0 and returns v; NaN propagates.
__device__ __forceinline__ double softplus_(double v) {
    const double m = v < 0.0 ? 0.0 : v;
    return m + log1p(exp(-__builtin_fabs(v)));
}
__device__ __forceinline__ float softplus_(float v) {
    constexpr float kLn2 = 0.6931471805599453f;
    const float u = fast_exp2(-__builtin_fabsf(v) * kLog2e);
    const float series = u * __builtin_fmaf(u, __builtin_fmaf(u, __builtin_fmaf(u, -0.25f, 1.0f / 3.0f), -0.5f), 1.0f);
    const float lg = __builtin_amdgcn_logf(1.0f + u) * kLn2;
    const float m = v < 0.f ? 0.f : v;
    return m + (u < 0.03125f ? series : lg);
}

// Accurate fp32 softplus (ocml log1pf / expf), for the fp32-storage decode step.
__device__ __forceinline__ float softplus_precise(float v) {
    const float m = v < 0.f ? 0.f : v;
    return m + log1pf(expf(-__builtin_fabsf(v)));
}

// exp of an argument in the arithmetic type's exponent units: natural units
// in fp64 (ocml exp), base-2 units in fp32 (z already multiplied by log2 e).
__device__ __forceinline__ double exp_units(double z) { return exp(z); }
__device__ __forceinline__ float exp_units(float z2) { return fast_exp2(z2); }

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// K consecutive values of T at byte offset voff + soff of a buffer: one
// vector load where kVec guarantees the alignment, else one per value.
template <typename T, int K, bool kVec, int kAux>
__device__ __forceinline__ void load_run(__amdgpu_buffer_rsrc_t r, int32_t voff, int32_t soff, T (&v)[K]) {
    constexpr int bytes = K * (int)sizeof(T);
    if constexpr (kVec && bytes == 16) {
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kAux);
        __builtin_memcpy(v, &w, 16);
    } else if constexpr (kVec && bytes == 8) {
        const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kAux);
        __builtin_memcpy(v, &w, 8);
    } else if constexpr (kVec && bytes == 4) {
        const unsigned w = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kAux);
        __builtin_memcpy(v, &w, 4);
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if constexpr (sizeof(T) == 4)
                v[k] = __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, voff + 4 * k, soff, kAux));
            else
                v[k] = __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b16(r, voff + 2 * k, soff, kAux));
        }
    }
}

// K consecutive fp32 values stored at byte offset voff + soff of a buffer,
// as one vector store where kVec guarantees the alignment.
template <int K, bool kVec, int kAux>
__device__ __forceinline__ void store_run(const float (&v)[K], __amdgpu_buffer_rsrc_t r, int32_t voff, int32_t soff) {
    if constexpr (kVec && K == 4) {
        u32x4 w;
        __builtin_memcpy(&w, v, 16);
        __builtin_amdgcn_raw_buffer_store_b128(w, r, voff, soff, kAux);
    } else if constexpr (kVec && K == 2) {
        u32x2 w;
        __builtin_memcpy(&w, v, 8);
        __builtin_amdgcn_raw_buffer_store_b64(w, r, voff, soff, kAux);
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v[k]), r, voff + 4 * k, soff, kAux);
    }
}

// Sum over aligned groups of Q <= 8 lanes by DPP (every lane of a group gets
// the group's sum): quad permutations, then the mirror within 8 lanes, which
// pairs each quad with the other quad of its half-row.
template <int Q>
__device__ __forceinline__ float lane_group_sum(float v) {
    static_assert(Q == 1 || Q == 2 || Q == 4 || Q == 8, "groups of 1, 2, 4 or 8 lanes");
    if constexpr (Q >= 2)
        v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // lanes 1,0,3,2
    if constexpr (Q >= 4)
        v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // lanes 2,3,0,1
    if constexpr (Q >= 8)
        v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));  // lane i <- 7-i
    return v;
}

// Wave-uniform value (the compiler then keeps it in an SGPR).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// blockIdx -> logical block so that consecutive logical blocks run on the same
// XCD (dispatch places block i on XCD i % 8).  Bijective for any grid size.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    constexpr int kXcd = 8;
    const int q = nblocks / kXcd, r = nblocks % kXcd;
    const int xcd = bid % kXcd, local = bid / kXcd;
    return xcd * q + (xcd < r ? xcd : r) + local;
}

}  // namespace ssm
