// gspn_device.h -- device helpers shared by the GSPN HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gspn {

// ---------------------------------------------------------------- dtypes
// bf16 is carried as its 16-bit pattern; widening to fp32 is exact.
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// fp32 -> storage type; bf16 rounds to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float from_f32(float v, float*) { return v; }
__device__ __forceinline__ uint16_t from_f32(float v, uint16_t*) {
    __bf16 b = (__bf16)v;
    return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v;
    v.x = (__bf16)lo;
    v.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- lanes
// Neighbour exchange along a line held one position per lane (wave64).
// from_left(v):  lane i receives lane i-1's value; lane 0 receives 0.
// from_right(v): lane i receives lane i+1's value; lane 63 receives 0.
__device__ __forceinline__ float from_left(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x138 /* wave_shr:1 */, 0xf, 0xf, true));
}
__device__ __forceinline__ float from_right(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x130 /* wave_shl:1 */, 0xf, 0xf, true));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ---------------------------------------------------------------- weights
struct Taps {
    float w0, w1, w2;
};

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float fast_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// Row-stochastic tridiagonal weights of one pixel.
//
// w_t = sigmoid(a_t) / sum of sigmoid(a_s) over the taps s that exist
// ("Key design 1: stability-context condition", GSPN CVPR 2025 paper notes:
// sigmoid on the non-zero entries of a row, then divide by the row sum).
// has0 / has2 tell whether the taps toward position p-1 / p+1 exist; a
// missing tap gets weight 0 and its raw value is never used.
//
// With e_t = exp(-a_t) and q_t = 1 + e_t (so sigmoid(a_t) = 1 / q_t):
//   w_0 = q1 q2 / D,  w_1 = q0 q2 / D,  w_2 = q0 q1 / D,
//   D = q1 q2 + q0 q2 + q0 q1,
// three exponentials and one reciprocal.  A missing tap is given q = 1 and
// its product term is dropped from D.  This form cannot overflow while every
// existing tap is >= -40; rows with a smaller tap take the slower per-tap
// sigmoid form, and rows whose sigmoids all underflow use exp(a_t - max a)
// (sigmoid(a) equals exp(a) to fp32 precision there).
__device__ __forceinline__ Taps normalise_taps(float a0, float a1, float a2, bool has0, bool has2) {
    const float kNegLog2e = -1.44269504088896340736f;
    const float kInf = __builtin_inff();
    a0 = has0 ? a0 : kInf;
    a2 = has2 ? a2 : kInf;
    Taps r;
    if (fminf(fminf(a0, a1), a2) >= -40.0f) {
        const float q0 = 1.0f + fast_exp2(a0 * kNegLog2e);
        const float q1 = 1.0f + fast_exp2(a1 * kNegLog2e);
        const float q2 = 1.0f + fast_exp2(a2 * kNegLog2e);
        const float p12 = has0 ? q1 * q2 : 0.0f;
        const float p02 = q0 * q2;
        const float p01 = has2 ? q0 * q1 : 0.0f;
        const float inv = fast_rcp(p12 + p02 + p01);
        r.w0 = p12 * inv;
        r.w1 = p02 * inv;
        r.w2 = p01 * inv;
    } else {
        // sigmoid(a) = 1 / (1 + exp(-a)); exp overflow gives 1/inf = 0
        const float s0 = has0 ? fast_rcp(1.0f + fast_exp2(a0 * kNegLog2e)) : 0.0f;
        const float s1 = fast_rcp(1.0f + fast_exp2(a1 * kNegLog2e));
        const float s2 = has2 ? fast_rcp(1.0f + fast_exp2(a2 * kNegLog2e)) : 0.0f;
        const float ssum = s0 + s1 + s2;
        if (ssum > 1e-30f) {
            const float inv = 1.0f / ssum;
            r.w0 = s0 * inv;
            r.w1 = s1 * inv;
            r.w2 = s2 * inv;
        } else {
            const float kLog2e = 1.44269504088896340736f;
            const float b0 = has0 ? a0 : -kInf, b2 = has2 ? a2 : -kInf;
            const float amax = fmaxf(fmaxf(b0, a1), b2);
            const float e0 = has0 ? fast_exp2((a0 - amax) * kLog2e) : 0.0f;
            const float e1 = fast_exp2((a1 - amax) * kLog2e);
            const float e2 = has2 ? fast_exp2((a2 - amax) * kLog2e) : 0.0f;
            const float inv = 1.0f / (e0 + e1 + e2);
            r.w0 = e0 * inv;
            r.w1 = e1 * inv;
            r.w2 = e2 * inv;
        }
    }
    return r;
}

// normalise_taps' fast form alone, for staged taps that are already
// sanitised: finite, >= -40, and 0 where a tap is missing or unused (any
// finite value gives the same weights there, since the missing tap's
// product term is dropped and its q cancels).  Returns (w0, w2).
__device__ __forceinline__ float2 normalise_fast(float a0, float a1, float a2, bool has0, bool has2) {
    const float kNegLog2e = -1.44269504088896340736f;
    const float q0 = 1.0f + fast_exp2(a0 * kNegLog2e);
    const float q1 = 1.0f + fast_exp2(a1 * kNegLog2e);
    const float q2 = 1.0f + fast_exp2(a2 * kNegLog2e);
    const float p12 = has0 ? q1 * q2 : 0.0f;
    const float p01 = has2 ? q0 * q1 : 0.0f;
    const float inv = fast_rcp(fmaf(q0, q2, p12) + p01);
    return make_float2(p12 * inv, p01 * inv);
}

}  // namespace gspn
