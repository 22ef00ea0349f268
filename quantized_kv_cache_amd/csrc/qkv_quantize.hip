// Group quantization of K/V rows into a pack (quantize a whole tensor, or
// append new tokens at an offset).
//
// Formats: group-wise affine (MLX page "add fast::quantized_kv_update",
// kernels/quantized.h affine_quantize; MLX CUDA page "Fixed mma and working
// dequant", quantized.cu affine_quantize) and Q8_0 (llama.cpp page "Metal:
// Optimize q8_0 KV - #25556").  The append semantics follow the kv_update
// kernel on the MLX page: the new token of each (batch, head) is quantized
// into the cache row at the offset.
//
// Mapping (wave64): each lane owns 8 consecutive values of a row (one 16-byte
// load for fp16/bf16, two for fp32); a group of gs values is gs/8 adjacent
// lanes, so its min/max (or absmax) is a butterfly over at most 16 lanes; a
// row is D/8 lanes, so one wave covers 512/D rows and every load and store of
// the wave is contiguous.  Each lane writes one packed word (4-bit) or two
// (8-bit, Q8_0); the first lane of a group writes its scale and bias.
//
// A dense fp16 pack (the unquantized cache) takes the fp16 values as they are.
//
// Bit-exactness: min/max are exact; the scale division, the subtract and the
// code division are IEEE fp32 (no fused multiply-add is possible in these
// expressions); codes round half to even (v_rndne_f32); scale and bias are
// rounded to their dtype before the codes are computed from them.
#include "qkv_device.hpp"
#include "qkv_internal.hpp"

namespace qkv {

namespace {

template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t off, float v[8]) {
    if constexpr (DT == DT_F32) {
        const float4* p = (const float4*)((const float*)base + off);
        float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        uint4 w = *(const uint4*)((const uint16_t*)base + off);
        uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint16_t lo = (uint16_t)(ws[i] & 0xffffu), hi = (uint16_t)(ws[i] >> 16);
            if constexpr (DT == DT_F16) { v[2 * i] = f16_to_f32(lo); v[2 * i + 1] = f16_to_f32(hi); }
            else { v[2 * i] = bf16_to_f32(lo); v[2 * i + 1] = bf16_to_f32(hi); }
        }
    }
}

template <int LANES>
__device__ __forceinline__ float group_min(float x) {
#pragma unroll
    for (int o = 1; o < LANES; o <<= 1) x = fminf(x, __shfl_xor(x, o, 64));
    return x;
}
template <int LANES>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
    for (int o = 1; o < LANES; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

// DT: source (and, for affine, scale) dtype.  MODE: affine / Q8_0.
template <int DT, int MODE, int BITS, int GS, int D>
__global__ __launch_bounds__(256) void quantize_rows_kernel(QuantLaunch p) {
    constexpr int LPR = D / 8;                 // lanes per row
    constexpr int RPW = 64 / LPR;              // rows per wave
    constexpr int GSZ = (MODE == MODE_Q8_0) ? 32 : GS;
    constexpr int LPG = GSZ / 8;               // lanes per group
    constexpr int NG = D / GSZ;                // groups per row
    const QuantJob& job = p.job[blockIdx.y];

    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t row = wave * RPW + lane / LPR;
    const int lr = lane % LPR;
    if (row >= p.rows) return;                 // whole rows (hence groups) leave together

    const int64_t t = row % p.T;
    const int64_t bh = row / p.T;
    const int64_t h = bh % p.H;
    const int64_t b = bh / p.H;
    const int64_t src = b * job.xs0 + h * job.xs1 + t * job.xs2 + (int64_t)lr * 8;
    const int64_t dst = b * job.sb + h * job.sh + (p.offset + t) * job.sl;

    if constexpr (MODE == MODE_DENSE) {
        // a dense fp16 cache stores the values themselves
        const uint4 raw = *(const uint4*)((const uint16_t*)job.x + src);
        ((uint4*)((uint8_t*)job.codes + dst * (int64_t)(D * 2)))[lr] = raw;
        return;
    } else {
    float v[8];
    load8<DT>(job.x, src, v);

    if constexpr (MODE == MODE_AFFINE) {
        constexpr float NL = (float)((1 << BITS) - 1);
        float mn = v[0], mx = v[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) { mn = fminf(mn, v[i]); mx = fmaxf(mx, v[i]); }
        mn = group_min<LPG>(mn);
        mx = group_max<LPG>(mx);
        const float eps = round_to<DT>(1e-7f);
        float s32 = (mx - mn) / NL;
        if (s32 < eps) s32 = eps;
        const float s = round_to<DT>(s32);
        const float bias = round_to<DT>(mn);
        uint32_t c[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float q = __builtin_rintf((v[i] - bias) / s);
            q = fminf(fmaxf(q, 0.0f), NL);
            c[i] = (uint32_t)q;
        }
        uint8_t* crow = (uint8_t*)job.codes + dst * (int64_t)(D * BITS / 8);
        if constexpr (BITS == 4) {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) w |= c[i] << (4 * i);
            ((uint32_t*)crow)[lr] = w;
        } else {
            uint2 w;
            w.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
            w.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
            ((uint2*)crow)[lr] = w;
        }
        if (lr % LPG == 0) {
            const int64_t si = dst * NG + lr / LPG;
            store_from_f32<DT>(job.scales, si, s32);
            store_from_f32<DT>(job.biases, si, mn);
        }
    } else {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
        amax = group_max<LPG>(amax);
        const float d32 = amax / 127.0f;
        const uint16_t dh = f32_to_f16(d32);
        const float d = f16_to_f32(dh);
        uint32_t c[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float q = 0.0f;
            if (d != 0.0f) {
                q = __builtin_rintf(v[i] / d);
                q = fminf(fmaxf(q, -127.0f), 127.0f);
            }
            c[i] = (uint32_t)(int32_t)q & 0xffu;
        }
        uint8_t* crow = (uint8_t*)job.codes + dst * (int64_t)D;
        uint2 w;
        w.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
        w.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
        ((uint2*)crow)[lr] = w;
        if (lr % LPG == 0) ((uint16_t*)job.scales)[dst * NG + lr / LPG] = dh;
    }
    }
}

// The general path: affine codes of any width, symmetric 4/5-bit blocks, and
// head size 96.  One thread per quantization group (per 32-block for the
// symmetric formats): two passes over the group's values (its range, then
// its codes), the codes packed into the group's words of the row's bit
// stream (a group of GS values at BITS bits starts on a word boundary since
// GS * BITS is a multiple of 32).  The arithmetic is that of the fast kernel
// above.
template <int DT>
__device__ __forceinline__ float load1(const void* base, int64_t off) {
    return load_as_f32<DT>(base, off);
}

template <int DT, int MODE, int BITS, int GS>
__global__ __launch_bounds__(256) void quantize_groups_kernel(QuantLaunch p, int D) {
    const QuantJob& job = p.job[blockIdx.y];
    const int ng = D / GS;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / ng;
    const int g = (int)(gid % ng);
    if (row >= p.rows) return;
    const int64_t t = row % p.T;
    const int64_t bh = row / p.T;
    const int64_t h = bh % p.H;
    const int64_t b = bh / p.H;
    const int64_t src = b * job.xs0 + h * job.xs1 + t * job.xs2 + (int64_t)g * GS;
    const int64_t dst = b * job.sb + h * job.sh + (p.offset + t) * job.sl;
    uint32_t* wout = (uint32_t*)((uint8_t*)job.codes + dst * (int64_t)(D * BITS / 8)) + g * (GS * BITS / 32);

    uint64_t acc = 0;
    int nacc = 0, wi = 0;
    auto put = [&](uint32_t c) {
        acc |= (uint64_t)c << nacc;
        nacc += BITS;
        if (nacc >= 32) {
            wout[wi++] = (uint32_t)acc;
            acc >>= 32;
            nacc -= 32;
        }
    };
    if constexpr (MODE == MODE_AFFINE) {
        constexpr float NL = (float)((1 << BITS) - 1);
        float mn = load1<DT>(job.x, src), mx = mn;
        for (int i = 1; i < GS; ++i) {
            const float v = load1<DT>(job.x, src + i);
            mn = fminf(mn, v);
            mx = fmaxf(mx, v);
        }
        const float eps = round_to<DT>(1e-7f);
        float s32 = (mx - mn) / NL;
        if (s32 < eps) s32 = eps;
        const float s = round_to<DT>(s32);
        const float bias = round_to<DT>(mn);
        for (int i = 0; i < GS; ++i) {
            float q = __builtin_rintf((load1<DT>(job.x, src + i) - bias) / s);
            q = fminf(fmaxf(q, 0.0f), NL);
            put((uint32_t)q);
        }
        store_from_f32<DT>(job.scales, dst * ng + g, s32);
        store_from_f32<DT>(job.biases, dst * ng + g, mn);
    } else {
        constexpr float QM = (float)((1 << (BITS - 1)) - 1);
        float amax = 0.0f;
        for (int i = 0; i < GS; ++i) amax = fmaxf(amax, fabsf(load1<DT>(job.x, src + i)));
        const uint16_t dh = f32_to_f16(amax / QM);
        const float d = f16_to_f32(dh);
        for (int i = 0; i < GS; ++i) {
            float q = 0.0f;
            if (d != 0.0f) {
                q = __builtin_rintf(load1<DT>(job.x, src + i) / d);
                q = fminf(fmaxf(q, -QM), QM);
            }
            put((uint32_t)(int32_t)q & ((1u << BITS) - 1u));
        }
        ((uint16_t*)job.scales)[dst * ng + g] = dh;
    }
}

template <int DT, int MODE, int BITS, int GS>
hipError_t launch_groups(int D, const QuantLaunch& p, int njobs, hipStream_t stream) {
    if (D % GS) return hipErrorNotSupported;
    const int64_t n = p.rows * (D / GS);
    const int64_t blocks = (n + 255) / 256;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((quantize_groups_kernel<DT, MODE, BITS, GS>), dim3((unsigned)blocks, njobs), dim3(256),
                       0, stream, p, D);
    return hipGetLastError();
}

template <int DT, int BITS>
hipError_t groups_by_gs(int gs, int D, const QuantLaunch& p, int njobs, hipStream_t s) {
    if (gs == 32) return launch_groups<DT, MODE_AFFINE, BITS, 32>(D, p, njobs, s);
    if (gs == 64) return launch_groups<DT, MODE_AFFINE, BITS, 64>(D, p, njobs, s);
    if (gs == 128) return launch_groups<DT, MODE_AFFINE, BITS, 128>(D, p, njobs, s);
    return hipErrorNotSupported;
}

template <int DT>
hipError_t dispatch_groups(int mode, int bits, int gs, int D, const QuantLaunch& p, int njobs, hipStream_t s) {
    if (mode == MODE_QSYM) {
        if (bits == 4) return launch_groups<DT, MODE_QSYM, 4, 32>(D, p, njobs, s);
        if (bits == 5) return launch_groups<DT, MODE_QSYM, 5, 32>(D, p, njobs, s);
        return hipErrorNotSupported;
    }
    if (mode == MODE_Q8_0) return launch_groups<DT, MODE_QSYM, 8, 32>(D, p, njobs, s);
    if (mode != MODE_AFFINE) return hipErrorNotSupported;
    switch (bits) {
        case 2: return groups_by_gs<DT, 2>(gs, D, p, njobs, s);
        case 3: return groups_by_gs<DT, 3>(gs, D, p, njobs, s);
        case 4: return groups_by_gs<DT, 4>(gs, D, p, njobs, s);
        case 5: return groups_by_gs<DT, 5>(gs, D, p, njobs, s);
        case 6: return groups_by_gs<DT, 6>(gs, D, p, njobs, s);
        case 8: return groups_by_gs<DT, 8>(gs, D, p, njobs, s);
    }
    return hipErrorNotSupported;
}

template <int DT, int MODE, int BITS, int GS, int D>
hipError_t launch_q(const QuantLaunch& p, int njobs, hipStream_t stream) {
    constexpr int RPW = 64 / (D / 8);
    const int64_t waves = (p.rows + RPW - 1) / RPW;
    const int64_t blocks = (waves + 3) / 4;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((quantize_rows_kernel<DT, MODE, BITS, GS, D>), dim3((unsigned)blocks, njobs),
                       dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int DT, int MODE, int BITS, int GS>
hipError_t dispatch_d(int D, const QuantLaunch& p, int njobs, hipStream_t s) {
    switch (D) {
        case 64: return launch_q<DT, MODE, BITS, GS, 64>(p, njobs, s);
        case 128: return launch_q<DT, MODE, BITS, GS, 128>(p, njobs, s);
        case 256: return launch_q<DT, MODE, BITS, GS, 256>(p, njobs, s);
    }
    return hipErrorNotSupported;
}

template <int DT>
hipError_t dispatch_fmt(int mode, int bits, int gs, int D, const QuantLaunch& p, int njobs,
                        hipStream_t s) {
    if (mode == MODE_Q8_0) return dispatch_d<DT, MODE_Q8_0, 8, 32>(D, p, njobs, s);
    if (mode == MODE_DENSE) {
        if constexpr (DT == DT_F16) return dispatch_d<DT, MODE_DENSE, 16, 32>(D, p, njobs, s);
        return hipErrorNotSupported;
    }
    if (bits == 4) {
        if (gs == 32) return dispatch_d<DT, MODE_AFFINE, 4, 32>(D, p, njobs, s);
        if (gs == 64) return dispatch_d<DT, MODE_AFFINE, 4, 64>(D, p, njobs, s);
        if (gs == 128) return dispatch_d<DT, MODE_AFFINE, 4, 128>(D, p, njobs, s);
    } else if (bits == 8) {
        if (gs == 32) return dispatch_d<DT, MODE_AFFINE, 8, 32>(D, p, njobs, s);
        if (gs == 64) return dispatch_d<DT, MODE_AFFINE, 8, 64>(D, p, njobs, s);
        if (gs == 128) return dispatch_d<DT, MODE_AFFINE, 8, 128>(D, p, njobs, s);
    }
    return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_quantize(int x_dtype, int mode, int bits, int group_size, int D,
                           const QuantLaunch& p, int njobs, hipStream_t stream) {
    if (mode != MODE_DENSE && !fast_format(mode, bits, D)) {
        switch (x_dtype) {
            case DT_F32: return dispatch_groups<DT_F32>(mode, bits, group_size, D, p, njobs, stream);
            case DT_F16: return dispatch_groups<DT_F16>(mode, bits, group_size, D, p, njobs, stream);
            case DT_BF16: return dispatch_groups<DT_BF16>(mode, bits, group_size, D, p, njobs, stream);
        }
        return hipErrorNotSupported;
    }
    switch (x_dtype) {
        case DT_F32: return dispatch_fmt<DT_F32>(mode, bits, group_size, D, p, njobs, stream);
        case DT_F16: return dispatch_fmt<DT_F16>(mode, bits, group_size, D, p, njobs, stream);
        case DT_BF16: return dispatch_fmt<DT_BF16>(mode, bits, group_size, D, p, njobs, stream);
    }
    return hipErrorNotSupported;
}

}  // namespace qkv
