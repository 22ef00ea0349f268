// Device helpers for the gfx950 kernels: scalar formats and storage access.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkv {

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
// v_cvt_f16_f32: round to nearest even, binary16 subnormals kept.
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}
// Round to nearest even on the bit pattern; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int DT>
__device__ __forceinline__ float load_as_f32(const void* p, int64_t i) {
    if constexpr (DT == 0) return ((const float*)p)[i];
    else if constexpr (DT == 1) return f16_to_f32(((const uint16_t*)p)[i]);
    else return bf16_to_f32(((const uint16_t*)p)[i]);
}

template <int DT>
__device__ __forceinline__ void store_from_f32(void* p, int64_t i, float v) {
    if constexpr (DT == 0) ((float*)p)[i] = v;
    else if constexpr (DT == 1) ((uint16_t*)p)[i] = f32_to_f16(v);
    else ((uint16_t*)p)[i] = f32_to_bf16(v);
}

// The value v as stored in dtype DT, widened back to fp32.
template <int DT>
__device__ __forceinline__ float round_to(float v) {
    if constexpr (DT == 0) return v;
    else if constexpr (DT == 1) return f16_to_f32(f32_to_f16(v));
    else return bf16_to_f32(f32_to_bf16(v));
}

__device__ __forceinline__ float load_mask(const void* p, int dt, int64_t i) {
    if (dt == 0) return ((const float*)p)[i];
    if (dt == 1) return f16_to_f32(((const uint16_t*)p)[i]);
    return bf16_to_f32(((const uint16_t*)p)[i]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 8 (or 4) consecutive 16-bit values at p, which the API only requires to be
// 2-byte aligned: one 16-byte (8-byte) load when the caller knows p is that
// aligned, 16-bit loads otherwise.
__device__ __forceinline__ uint4 load_h8(const uint16_t* p, bool aligned16) {
    if (aligned16) return *(const uint4*)p;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)p[2 * i] | ((uint32_t)p[2 * i + 1] << 16);
    return uint4{w[0], w[1], w[2], w[3]};
}
__device__ __forceinline__ uint2 load_h4(const uint16_t* p, bool aligned8) {
    if (aligned8) return *(const uint2*)p;
    return uint2{(uint32_t)p[0] | ((uint32_t)p[1] << 16), (uint32_t)p[2] | ((uint32_t)p[3] << 16)};
}

// Makes x live in SGPRs at this point.  Kernels pin every argument they read
// at their start, so that all argument loads are issued together and waited
// for once (a later first read would cost another trip to memory).
template <typename T>
__device__ __forceinline__ void pin_sgpr(const T& x) {
    __asm__ __volatile__("" ::"s"(x));
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace qkv
