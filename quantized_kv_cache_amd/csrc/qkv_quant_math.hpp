// Per-lane arithmetic of the row quantizer: one lane holds 8 consecutive
// values of a row, a quantization group is LPG adjacent lanes.  Shared by the
// quantize kernel and the decode that appends a token before attending, so
// both write the same bits.
//
// Affine groups (MLX page "add fast::quantized_kv_update", kernels/quantized.h
// affine_quantize): s = max((max - min) / (2^bits - 1), eps) and b = min are
// rounded to the scale dtype DT before the codes are taken, and
// c = clamp(round_half_even((x - b) / s), 0, 2^bits - 1).  Q8_0 blocks
// (llama.cpp page "Metal: Optimize q8_0 KV - #25556"): d = fp16(amax / 127),
// c = clamp(round_half_even(x / d), -127, 127), 0 when d = 0.
//
// The divisions are exact IEEE fp32 quotients reached without a division
// instruction per element: with y = RN(1/b) and q = RN(a y), the residual
// r = a - b q is exact in one fused multiply-add and RN(q + r y) is the
// correctly rounded a / b (Markstein's correction step).  For fp16 and bf16
// divisors y is the hardware reciprocal refined by one Newton step; fp32
// sources keep the IEEE division for the codes.  min/max take finite inputs.
#pragma once

#include "qkv_device.hpp"
#include "qkv_internal.hpp"

namespace qkv {
namespace qm {

// Reduction over LANES adjacent lanes (aligned, a power of two <= 16), every
// lane receiving the result: DPP quad permutations for the first two steps,
// then half-row and row mirrors (lane i of 8 or 16 meets lane 7 - i or 15 - i,
// which lies in the other half once the halves are reduced).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int LANES, bool MAX>
__device__ __forceinline__ float group_reduce(float x) {
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
    if constexpr (LANES >= 2) x = op(x, dpp_f32<0xB1>(x));    // quad_perm [1,0,3,2]
    if constexpr (LANES >= 4) x = op(x, dpp_f32<0x4E>(x));    // quad_perm [2,3,0,1]
    if constexpr (LANES >= 8) x = op(x, dpp_f32<0x141>(x));   // row_half_mirror
    if constexpr (LANES >= 16) x = op(x, dpp_f32<0x140>(x));  // row_mirror
    return x;
}

// RN(1 / b) for a divisor b with a 16-bit (fp16 or bf16) significand: the
// hardware reciprocal (within one ulp) and one Newton step.  Every fp16 divisor
// and every bf16 divisor >= 1e-7 was checked on the CPU from each starting
// value within one ulp of 1 / b: the step lands on the correctly rounded
// reciprocal.
__device__ __forceinline__ float recip_rn16(float b) {
    const float y0 = __builtin_amdgcn_rcpf(b);
    const float e = __builtin_fmaf(-b, y0, 1.0f);
    return __builtin_fmaf(e, y0, y0);
}

// RN(a / b) from y = RN(1 / b): one product and two fused multiply-adds.
__device__ __forceinline__ float div_by_recip(float a, float b, float y) {
    const float q = a * y;
    const float r = __builtin_fmaf(-q, b, a);
    return __builtin_fmaf(r, y, q);
}

// round_half_even(x) for |x| < 2^22 as an integer in the low bits of the
// result's bit pattern (1.5 * 2^23 + n), clamped to [lo, hi].
__device__ __forceinline__ int32_t rne_clamp(float x, int lo, int hi) {
    const int32_t u = __float_as_int(x + 12582912.0f);
    return min(max(u, 0x4B400000 + lo), 0x4B400000 + hi) - 0x4B400000;
}

// Affine codes of the lane's 8 values: w[0] (4-bit: the whole 32-bit word,
// byte k holding codes 2k and 2k + 1 in its low and high nibble) or w[0..1]
// (8-bit: one byte per code); s32 and mn are the group's scale before its
// rounding to DT and its minimum (stored rounded to DT).
template <int DT, int BITS, int LPG>
__device__ __forceinline__ void quantize_affine8(const float v[8], uint32_t w[2], float& s32, float& mn) {
#pragma clang fp contract(off)
    constexpr int NL = (1 << BITS) - 1;
    mn = v[0];
    float mx = v[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) { mn = fminf(mn, v[i]); mx = fmaxf(mx, v[i]); }
    mn = group_reduce<LPG, false>(mn);
    mx = group_reduce<LPG, true>(mx);
    const float eps = round_to<DT>(1e-7f);
    s32 = div_by_recip(mx - mn, (float)NL, 1.0f / (float)NL);
    if (s32 < eps) s32 = eps;
    const float s = round_to<DT>(s32);
    const float bias = round_to<DT>(mn);
    const float y = DT == DT_F32 ? 1.0f : recip_rn16(s);
    // code i = clamp(round_half_even(qt_i), 0, NL): v_cvt_pk_u8_f32 rounds
    // half to even, saturates to [0, 255] and inserts the byte into a register
    // in one instruction (checked on the GPU against rint with saturation on
    // ties, their neighbours, negative values and values past 255); 4-bit
    // quotients are first limited to 15, which commutes with the rounding
    float qt[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float a = v[i] - bias;
        qt[i] = DT == DT_F32 ? a / s : div_by_recip(a, s, y);
        if constexpr (BITS == 4) qt[i] = fminf(qt[i], (float)NL);
    }
    if constexpr (BITS == 4) {
        uint32_t ev = 0, od = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            ev = __builtin_amdgcn_cvt_pk_u8_f32(qt[2 * k], (uint32_t)k, ev);
            od = __builtin_amdgcn_cvt_pk_u8_f32(qt[2 * k + 1], (uint32_t)k, od);
        }
        w[0] = ev | (od << 4);
        w[1] = 0u;
    } else {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            lo = __builtin_amdgcn_cvt_pk_u8_f32(qt[k], (uint32_t)k, lo);
            hi = __builtin_amdgcn_cvt_pk_u8_f32(qt[4 + k], (uint32_t)k, hi);
        }
        w[0] = lo;
        w[1] = hi;
    }
}

// Q8_0 codes of the lane's 8 values (one byte each in w[0..1]) and the
// block's fp16 scale d (LPG = 4 lanes per block of 32).
template <int DT, int LPG>
__device__ __forceinline__ void quantize_q8_0_8(const float v[8], uint32_t w[2], uint16_t& dh) {
#pragma clang fp contract(off)
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = group_reduce<LPG, true>(amax);
    const float d32 = div_by_recip(amax, 127.0f, 1.0f / 127.0f);
    dh = f32_to_f16(d32);
    const float d = f16_to_f32(dh);
    // d = 0 (an all-zero block) gives codes 0: y = 0 makes every quotient 0
    const float y = d != 0.0f ? recip_rn16(d) : 0.0f;
    int32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float qt = DT == DT_F32 ? (d != 0.0f ? v[i] / d : 0.0f) : div_by_recip(v[i], d, y);
        c[i] = rne_clamp(qt, -127, 127);
    }
    w[0] = ((uint32_t)c[0] & 0xffu) | (((uint32_t)c[1] & 0xffu) << 8) | (((uint32_t)c[2] & 0xffu) << 16) |
           ((uint32_t)c[3] << 24);
    w[1] = ((uint32_t)c[4] & 0xffu) | (((uint32_t)c[5] & 0xffu) << 8) | (((uint32_t)c[6] & 0xffu) << 16) |
           ((uint32_t)c[7] << 24);
}

// One new K row and one new V row (D fp16 values each, at k_new / v_new)
// quantized by one wave into pack rows whose codes, scales and biases start at
// the given row pointers (fp16 scales; affine or Q8_0): lanes 0 .. D/8 - 1
// take the K row, lanes 32 .. 32 + D/8 - 1 the V row, 8 values per lane, so
// every group lies in one DPP row of lanes.  The stores are issued, not
// waited for.
template <int MODE, int BITS, int GS, int D>
__device__ __forceinline__ void append_rows(const uint16_t* k_new, const uint16_t* v_new, uint8_t* kcodes,
                                            uint8_t* vcodes, uint8_t* kscales, uint8_t* vscales, uint8_t* kbiases,
                                            uint8_t* vbiases) {
    constexpr int LPR = D / 8;                                  // lanes per row
    constexpr int LPG = (MODE == MODE_Q8_0 ? 32 : GS) / 8;      // lanes per group
    constexpr int ROWB = D * BITS / 8;
    static_assert(LPR <= 32 && (MODE == MODE_AFFINE || MODE == MODE_Q8_0), "one row per half wave");
    const int lane = threadIdx.x & 63;
    const bool is_v = lane >= 32;
    const int lr = lane & 31;
    const bool on = lr < LPR;
    uint4 x = uint4{0u, 0u, 0u, 0u};
    if (on) x = *(const uint4*)((is_v ? v_new : k_new) + 8 * lr);
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
    float vals[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) vals[i] = f16_to_f32((uint16_t)(xw[i >> 1] >> (16 * (i & 1))));
    uint32_t w[2];
    float s32 = 0.0f, mn = 0.0f;
    uint16_t dh = 0;
    if constexpr (MODE == MODE_Q8_0) quantize_q8_0_8<DT_F16, LPG>(vals, w, dh);
    else quantize_affine8<DT_F16, BITS, LPG>(vals, w, s32, mn);
    if (!on) return;
    uint8_t* codes = (is_v ? vcodes : kcodes) + lr * (ROWB / LPR);
    if constexpr (BITS == 4) *(uint32_t*)codes = w[0];
    else *(uint2*)codes = uint2{w[0], w[1]};
    if (lr % LPG == 0) {
        const int so = (lr / LPG) * 2;
        if constexpr (MODE == MODE_Q8_0) {
            *(uint16_t*)((is_v ? vscales : kscales) + so) = dh;
        } else {
            *(uint16_t*)((is_v ? vscales : kscales) + so) = f32_to_f16(s32);
            *(uint16_t*)((is_v ? vbiases : kbiases) + so) = f32_to_f16(mn);
        }
    }
}

}  // namespace qm
}  // namespace qkv
