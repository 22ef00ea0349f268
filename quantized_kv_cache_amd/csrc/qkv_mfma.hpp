// Small device helpers shared by the matrix-core attention kernels: fp16
// vector views of packed registers, byte permutes, the 16x16x32 f16 MFMA,
// the packed-code -> fp16-subnormal conversions and the 4-lane reductions.
#pragma once

#include <type_traits>

#include "qkv_device.hpp"

namespace qkv {
namespace mf {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// v_perm_b32: selector bytes 0-3 pick bytes of lo, 4-7 bytes of hi, 0x0C gives 0.
__device__ __forceinline__ uint32_t perm_b(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}
__device__ __forceinline__ h8 to_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    u4 v = {a, b, c, d};
    return __builtin_bit_cast(h8, v);
}
__device__ __forceinline__ h4 to_h4(uint32_t a, uint32_t b) {
    u2 v = {a, b};
    return __builtin_bit_cast(h4, v);
}
__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u(h2 h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ float lo_f16(uint32_t u) { return f16_to_f32((uint16_t)(u & 0xffffu)); }
__device__ __forceinline__ float hi_f16(uint32_t u) { return f16_to_f32((uint16_t)(u >> 16)); }

__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 16 blocks of 4x4x4 with the A operand of block ABID broadcast to all blocks.
template <int ABID>
__device__ __forceinline__ f4 mfma4_bcast(h4 a, h4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 4, ABID, 0);
}

// f(std::integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Byte 'byte' of the chunks of two keys -> [key a byte, 0, key b byte, 0].
__device__ __forceinline__ uint32_t pair_bytes(const uint32_t* wa, const uint32_t* wb, int byte) {
    const uint32_t sel = (uint32_t)(byte & 3) | 0x0C00u | ((uint32_t)(4 + (byte & 3)) << 16) |
                         0x0C000000u;
    return perm_b(wb[byte >> 2], wa[byte >> 2], sel);
}

// Code t of the lane's chunk for a pair of keys, as fp16 subnormal halves
// c * 2^-24 (4-bit odd codes arrive as 16 c).
template <int BITS>
__device__ __forceinline__ uint32_t pair_sub(const uint32_t* wa, const uint32_t* wb, int t) {
    if constexpr (BITS == 4) {
        const uint32_t x = pair_bytes(wa, wb, t >> 1);
        return (t & 1) ? (x & 0x00F000F0u) : (x & 0x000F000Fu);
    } else {
        return pair_bytes(wa, wb, t);
    }
}

// As pair_sub, but a 4-bit odd code arrives as its whole byte, lo + 16 hi:
// a product accumulated from it minus the one from the even code (lo) of the
// same byte is 16 times the product of the odd code (saves the mask).
template <int BITS>
__device__ __forceinline__ uint32_t pair_sub_byte(const uint32_t* wa, const uint32_t* wb, int t) {
    if constexpr (BITS == 4) {
        const uint32_t x = pair_bytes(wa, wb, t >> 1);
        return (t & 1) ? x : (x & 0x000F000Fu);
    } else {
        return pair_bytes(wa, wb, t);
    }
}

// Compiler-only ordering of a wave's LDS scratch: LDS instructions of one
// wave execute in order, so no wait on outstanding global loads is needed.
__device__ __forceinline__ void lds_order() { __asm__ __volatile__("" ::: "memory"); }

// Reductions over the four lanes n, n+16, n+32, n+48 (v_permlane*_swap).
__device__ __forceinline__ float max4(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float sum4(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Reductions over all 64 lanes; every lane gets the result.  Within each row
// of 16 lanes by DPP (quad permutes, then the half-row and row mirrors pair
// lanes of different quads and halves), then across rows by max4 / sum4:
// VALU-only, no LDS round trips.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));     // quad_perm [1, 0, 3, 2]
    x = fmaxf(x, dpp_f<0x4E>(x));     // quad_perm [2, 3, 0, 1]
    x = fmaxf(x, dpp_f<0x141>(x));    // row_half_mirror
    x = fmaxf(x, dpp_f<0x140>(x));    // row_mirror
    return max4(x);
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    x += dpp_f<0x141>(x);
    x += dpp_f<0x140>(x);
    return sum4(x);
}

// A raw buffer resource over rows [row0, row0 + min(tile, end - row0)) of a
// plane with the given byte stride; rows past 'end' read as zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint8_t* base, int64_t row0,
                                                             int64_t end, int tile, uint32_t stride,
                                                             uint32_t row_bytes) {
    const int64_t rows = min((int64_t)tile, end - row0);
    const uint32_t bytes = rows > 0 ? (uint32_t)(rows - 1) * stride + row_bytes : 0u;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + row0 * (int64_t)stride), (short)0,
                                             (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t buf32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t buf16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
// 16 bytes per lane from the buffer straight into LDS: lane l's bytes land
// at lds + 16 l (the wave writes 1 KB there; completion counts in vmcnt).
__device__ __forceinline__ void buf_to_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0,
                                             0);
}
// nw (1, 2 or a multiple of 4) consecutive dwords
__device__ __forceinline__ void bufn(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* dst, int nw) {
    if (nw == 1) {
        dst[0] = buf32(r, off);
    } else if (nw == 2) {
        auto x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
        dst[0] = x[0];
        dst[1] = x[1];
    } else {
#pragma unroll
        for (int q4 = 0; q4 < nw; q4 += 4) {
            auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 4 * q4), 0, 0);
            dst[q4] = x[0];
            dst[q4 + 1] = x[1];
            dst[q4 + 2] = x[2];
            dst[q4 + 3] = x[3];
        }
    }
}

}  // namespace mf
}  // namespace qkv
