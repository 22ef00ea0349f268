// Dequantization of a quantized K/V pack into a dense fp16 pack: the fp16
// scratch copy of the llama.cpp page "Metal: Optimize q8_0 KV - #25556"
// (merged #27390: kernel_flash_attn_ext_dequant_to_f16 dequantizes K and V
// into contiguous F16 buffers before the F16 flash attention runs on them),
// with the element value of the MLX page "add fast::quantized_kv_update"
// (kernels/quantized.h: scale * code + bias).
//
// Element j of a row: affine fp16(fp32(s) * c + fp32(b)) with the product and
// the sum each rounded in fp32 (no fused multiply-add), Q8_0 fp16(fp32(d) * c)
// (an exact product), so the result is the oracle's fp32 dequantized value
// rounded to fp16.
//
// Mapping (wave64): a lane owns 8 consecutive elements of a row (their codes
// lie in one quantization group), so it reads one word of 4-bit codes or two
// of 8-bit codes plus the group's scale and bias, and writes one 16-byte
// chunk; a row is D / 8 lanes and every wave access is contiguous.
#include "qkv_device.hpp"
#include "qkv_internal.hpp"

namespace qkv {

namespace {

template <int MODE, int BITS, int D>
__global__ __launch_bounds__(256) void dequant_rows_kernel(DequantLaunch p) {
#pragma clang fp contract(off)
    constexpr int LPR = D / 8;                 // lanes per row
    constexpr int RPW = 64 / LPR;              // rows per wave
    constexpr int ROWB = D * BITS / 8;
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t row = wave * RPW + lane / LPR;
    const int lr = lane % LPR;
    if (row >= p.rows) return;
    const int64_t t = row % p.L;
    const int64_t bh = row / p.L;
    const int64_t h = bh % p.H;
    const int64_t b = bh / p.H;
    const int64_t src = b * p.sb + h * p.sh + t * p.sl;
    const int64_t dst = b * p.db + h * p.dh + t * p.dl;
    const int ng = D / p.gs;
    const int g = (lr * 8) / p.gs;

    uint32_t w[2];
    const uint8_t* crow = (const uint8_t*)p.codes + src * ROWB;
    if constexpr (BITS == 4) {
        w[0] = ((const uint32_t*)crow)[lr];
        w[1] = 0u;
    } else {
        const uint2 x = ((const uint2*)crow)[lr];
        w[0] = x.x;
        w[1] = x.y;
    }
    const float s = f16_to_f32(((const uint16_t*)p.scales)[src * ng + g]);
    const float bias = MODE == MODE_AFFINE ? f16_to_f32(((const uint16_t*)p.biases)[src * ng + g]) : 0.0f;
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        float v[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int i = e + k;
            float c;
            if constexpr (BITS == 4) c = (float)((w[0] >> (4 * i)) & 15u);
            else if constexpr (MODE == MODE_Q8_0) c = (float)(int8_t)((w[i >> 2] >> (8 * (i & 3))) & 0xFFu);
            else c = (float)((w[i >> 2] >> (8 * (i & 3))) & 0xFFu);
            const float prod = s * c;
            v[k] = MODE == MODE_AFFINE ? prod + bias : prod;
        }
        o[e / 2] = (uint32_t)f32_to_f16(v[0]) | ((uint32_t)f32_to_f16(v[1]) << 16);
    }
    ((uint4*)((uint16_t*)p.out + dst * D))[lr] = uint4{o[0], o[1], o[2], o[3]};
}

template <int MODE, int BITS, int D>
hipError_t launch_d(const DequantLaunch& p, hipStream_t stream) {
    constexpr int RPW = 64 / (D / 8);
    const int64_t waves = (p.rows + RPW - 1) / RPW;
    const int64_t blocks = (waves + 3) / 4;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((dequant_rows_kernel<MODE, BITS, D>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int MODE, int BITS>
hipError_t by_d(int D, const DequantLaunch& p, hipStream_t s) {
    switch (D) {
        case 64: return launch_d<MODE, BITS, 64>(p, s);
        case 128: return launch_d<MODE, BITS, 128>(p, s);
        case 256: return launch_d<MODE, BITS, 256>(p, s);
    }
    return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_dequantize(int mode, int bits, int group_size, int D, const DequantLaunch& p,
                             hipStream_t stream) {
    (void)group_size;
    if (mode == MODE_Q8_0) return by_d<MODE_Q8_0, 8>(D, p, stream);
    if (mode == MODE_AFFINE && bits == 4) return by_d<MODE_AFFINE, 4>(D, p, stream);
    if (mode == MODE_AFFINE && bits == 8) return by_d<MODE_AFFINE, 8>(D, p, stream);
    return hipErrorNotSupported;
}

}  // namespace qkv
