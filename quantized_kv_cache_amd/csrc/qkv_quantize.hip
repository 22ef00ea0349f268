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
// lanes, so its min/max (or absmax) is a DPP reduction over at most 16 lanes;
// a row is D/8 lanes, so one wave covers 512/D rows per pass and every load
// and store of the wave is contiguous.  A workgroup takes a run of rows of
// one (batch, head), which it finds from the grid's y coordinate, so no
// 64-bit index division is needed; each wave makes two passes whose loads are
// issued together.  Each lane writes one packed word (4-bit) or two (8-bit,
// Q8_0); the first lane of a group writes its scale and bias.
//
// A dense fp16 pack (the unquantized cache) takes the fp16 values as they are.
//
// Bit-exactness: min/max are exact; the subtract is IEEE fp32; scale and
// bias are rounded to their dtype before the codes are computed from them;
// codes round half to even.  The two divisions are exact IEEE fp32 quotients
// reached without a division instruction per element: with y = RN(1/b) and
// q = RN(a y), the residual r = a - b q is exact in one fused multiply-add
// and RN(q + r y) is the correctly rounded a / b (Markstein's correction
// step).  For fp16 and bf16 divisors y is the hardware reciprocal refined by
// one Newton step.  Both steps were checked on the CPU against the IEEE
// operations: the reciprocal for every fp16 and bf16 divisor from every start
// within one ulp; the quotient for (max - min) / (2^bits - 1) and amax / 127
// over a dense sample of all non-negative fp32 values, and for the code
// quotients over every fp16 and bf16 divisor at every numerator within four
// ulps of each half-integer quotient up to 300 (where a one-ulp difference
// could move a code).  fp32 sources keep the IEEE division for the codes.
// The file is compiled for finite inputs (a NaN or an infinity in a group
// gives unspecified codes for that group), so min/max need no NaN handling.
#include <algorithm>

#include "qkv_device.hpp"
#include "qkv_internal.hpp"
#include "qkv_quant_math.hpp"

namespace qkv {

namespace {

typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

using namespace qm;

constexpr int kQuantPasses = 2;   // row passes per wave, loads issued together

// A raw buffer resource over `rows` rows (0 .. RPW) of a plane starting at
// base, rows `stride` bytes apart and `row_bytes` long: loads past the last
// row read zeros and stores there are dropped, so a pass needs no bounds
// branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pass_rsrc(const uint8_t* base, int64_t rows, uint32_t stride,
                                                              uint32_t row_bytes) {
    const uint32_t bytes = rows > 0 ? (uint32_t)(rows - 1) * stride + row_bytes : 0u;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

// Cache policy of the row kernel's source loads and code stores: nt
// (non-temporal).  Both streams are touched once and every code store of a
// wave covers whole cache lines, so they are kept out of the L2s and leave no
// dirty lines for the end of the kernel to write back (batched 8-bit cache
// tensor 78.6-79.3 -> 75.3-75.6 us, Q8_0 tensor 10.3 -> 9.1 us).  The 2- and
// 4-byte scale and bias stores of the group leaders keep the default policy:
// as non-temporal stores they reach memory as separate partial-line writes
// (46.8 MB written per 64K 4-bit K tensor against 37.7 MB).
constexpr int kStream = 2;

// 8 consecutive source values as fp32 (fp32: two 16-byte loads, else one).
template <int DT>
__device__ __forceinline__ void load8_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, float v[8]) {
    if constexpr (DT == DT_F32) {
        const auto a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kStream);
        const auto b = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 16), 0, kStream);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = __uint_as_float(a[i]);
            v[4 + i] = __uint_as_float(b[i]);
        }
    } else {
        const auto w = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kStream);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint16_t lo = (uint16_t)(w[i] & 0xffffu), hi = (uint16_t)(w[i] >> 16);
            if constexpr (DT == DT_F16) { v[2 * i] = f16_to_f32(lo); v[2 * i + 1] = f16_to_f32(hi); }
            else { v[2 * i] = bf16_to_f32(lo); v[2 * i + 1] = bf16_to_f32(hi); }
        }
    }
}

template <int DT>
__device__ __forceinline__ void store_scale_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    if constexpr (DT == DT_F32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)off, 0, 0);
    else if constexpr (DT == DT_F16) __builtin_amdgcn_raw_buffer_store_b16(f32_to_f16(v), r, (int)off, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, (int)off, 0, 0);
}
// The same value written to LDS at byte offset off of a staging block.
template <int DT>
__device__ __forceinline__ void stage_scale(uint8_t* blk, uint32_t off, float v) {
    if constexpr (DT == DT_F32) *(uint32_t*)(blk + off) = __float_as_uint(v);
    else if constexpr (DT == DT_F16) *(uint16_t*)(blk + off) = f32_to_f16(v);
    else *(uint16_t*)(blk + off) = f32_to_bf16(v);
}

// DT: source (and, for affine, scale) dtype.  MODE: affine / Q8_0 / dense.
// Every address is a wave-uniform base (scalar, 64-bit) plus a lane offset
// that does not change between passes (32-bit): the host keeps a source row
// stride and a pack row stride below 2^27 bytes.
template <int DT, int MODE, int BITS, int GS, int D>
__global__ __launch_bounds__(256) void quantize_rows_kernel(QuantLaunch p) {
#pragma clang fp contract(off)
    constexpr int LPR = D / 8;                 // lanes per row
    constexpr int RPW = 64 / LPR;              // rows per wave and pass
    constexpr int U = kQuantPasses;
    constexpr int RPB = 4 * RPW * U;           // rows per workgroup
    constexpr int GSZ = (MODE == MODE_Q8_0) ? 32 : GS;
    constexpr int LPG = GSZ / 8;               // lanes per group
    constexpr int NG = D / GSZ;                // groups per row
    constexpr int ES = DT == DT_F32 ? 4 : 2;   // source element bytes
    constexpr int ROWB = MODE == MODE_DENSE ? 2 * D : D * BITS / 8;   // code bytes of a row
    constexpr int SS = MODE == MODE_AFFINE ? ES : 2;                  // scale element bytes
    constexpr int SROWB = NG * SS;
    const QuantJob& job = p.job[blockIdx.z];
    pin_sgpr(job.x); pin_sgpr(job.codes); pin_sgpr(job.scales); pin_sgpr(job.biases);
    pin_sgpr(job.xs0); pin_sgpr(job.xs1); pin_sgpr(job.xs2);
    pin_sgpr(job.sb); pin_sgpr(job.sh); pin_sgpr(job.sl);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane % LPR;
    const int lrow = lane / LPR;               // the lane's row within a pass
    const uint32_t xstride = (uint32_t)(job.xs2 * ES);
    const uint32_t cstride = (uint32_t)(job.sl * ROWB);
    const uint32_t sstride = (uint32_t)(job.sl * SROWB);
    const uint32_t o_x = (uint32_t)lrow * xstride + (uint32_t)lr * 8 * ES;
    const uint32_t o_c = (uint32_t)lrow * cstride + (uint32_t)lr * (ROWB / LPR);
    const uint32_t o_s = (uint32_t)lrow * sstride + (uint32_t)(lr / LPG) * SS;
    const bool leader = lr % LPG == 0;
    // first row of each pass of this wave, relative to the (batch, head)
    const int64_t t0 = (int64_t)blockIdx.x * RPB;
    const int64_t tw = t0 + wave * RPW * U;
    const uint32_t H = (uint32_t)p.H;
    // Scale (and bias) rows of the workgroup's RPB pack rows, gathered: when
    // the rows are consecutive (row stride 1), all inside [0, T) and their
    // scale block is 16-byte aligned, the group leaders put their values into
    // an LDS copy of the block, which whole 16-byte non-temporal stores then
    // write: full lines reach memory and none stay dirty in the L2s for the
    // end of the kernel.  Otherwise each leader stores its own value.
    constexpr int SBLK = RPB * SROWB;           // bytes of the block's scales
    constexpr bool CAN_GATHER = MODE != MODE_DENSE && SBLK > 0 && SBLK % 16 == 0 && SBLK / 16 <= 128;
    __shared__ __attribute__((aligned(16))) uint8_t s_blk[2][CAN_GATHER ? SBLK : 16];
    const uint32_t o_blk = (uint32_t)(wave * RPW * U + lrow) * SROWB + (uint32_t)(lr / LPG) * SS;
    for (uint32_t bh = blockIdx.y; bh < (uint32_t)p.BH; bh += gridDim.y) {
        const uint32_t b = bh / H;
        const uint32_t h = bh - b * H;
        const int64_t xrow0 = (int64_t)b * job.xs0 + (int64_t)h * job.xs1;    // elements
        const int64_t prow0 = (int64_t)b * job.sb + (int64_t)h * job.sh + p.offset;   // pack rows
        uint8_t* sblk = (uint8_t*)job.scales + (prow0 + t0) * SROWB;
        uint8_t* bblk = MODE == MODE_AFFINE ? (uint8_t*)job.biases + (prow0 + t0) * SROWB : sblk;
        const bool gather = CAN_GATHER && job.sl == 1 && t0 + RPB <= p.T &&
                            ((reinterpret_cast<uintptr_t>(sblk) | reinterpret_cast<uintptr_t>(bblk)) & 15) == 0;
        __amdgpu_buffer_rsrc_t rc[U], rs[U], rb[U];
        uint4 raw[U];
        float v[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = tw + u * RPW;
            const int64_t rows = min((int64_t)RPW, p.T - t);
            const auto rx = pass_rsrc((const uint8_t*)job.x + (xrow0 + t * job.xs2) * ES, rows, xstride, D * ES);
            rc[u] = pass_rsrc((const uint8_t*)job.codes + (prow0 + t * job.sl) * ROWB, rows, cstride, ROWB);
            if constexpr (MODE != MODE_DENSE) {
                rs[u] = pass_rsrc((const uint8_t*)job.scales + (prow0 + t * job.sl) * SROWB, rows, sstride, SROWB);
                if constexpr (MODE == MODE_AFFINE)
                    rb[u] = pass_rsrc((const uint8_t*)job.biases + (prow0 + t * job.sl) * SROWB, rows, sstride, SROWB);
            }
            if constexpr (MODE == MODE_DENSE) {
                const auto w = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)o_x, 0, 0);
                raw[u] = uint4{w[0], w[1], w[2], w[3]};
            } else {
                load8_buf<DT>(rx, o_x, v[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (MODE == MODE_DENSE) {
                // a dense fp16 cache stores the values themselves
                const u4 w = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
                __builtin_amdgcn_raw_buffer_store_b128(w, rc[u], (int)o_c, 0, kStream);
            } else if constexpr (MODE == MODE_AFFINE) {
                uint32_t w[2];
                float s32, mn;
                quantize_affine8<DT, BITS, LPG>(v[u], w, s32, mn);
                if constexpr (BITS == 4) {
                    __builtin_amdgcn_raw_buffer_store_b32(w[0], rc[u], (int)o_c, 0, kStream);
                } else {
                    const u2 wv = {w[0], w[1]};
                    __builtin_amdgcn_raw_buffer_store_b64(wv, rc[u], (int)o_c, 0, kStream);
                }
                if (leader) {
                    if (gather) {
                        stage_scale<DT>(s_blk[0], o_blk + u * RPW * SROWB, s32);
                        stage_scale<DT>(s_blk[1], o_blk + u * RPW * SROWB, mn);
                    } else {
                        store_scale_buf<DT>(rs[u], o_s, s32);
                        store_scale_buf<DT>(rb[u], o_s, mn);
                    }
                }
            } else {
                uint32_t w[2];
                uint16_t dh;
                quantize_q8_0_8<DT, LPG>(v[u], w, dh);
                const u2 wv = {w[0], w[1]};
                __builtin_amdgcn_raw_buffer_store_b64(wv, rc[u], (int)o_c, 0, kStream);
                if (leader) {
                    if (gather) *(uint16_t*)(s_blk[0] + o_blk + u * RPW * SROWB) = dh;
                    else __builtin_amdgcn_raw_buffer_store_b16(dh, rs[u], (int)o_s, 0, 0);
                }
            }
        }
        if constexpr (CAN_GATHER) {
            if (gather) {                      // uniform over the workgroup
                __syncthreads();
                constexpr int NB = MODE == MODE_AFFINE ? 2 : 1;
                if ((int)threadIdx.x < NB * SBLK / 16) {
                    const int k = (int)threadIdx.x / (SBLK / 16);
                    const uint32_t off = 16u * ((uint32_t)threadIdx.x % (SBLK / 16));
                    const uint4 x = *(const uint4*)(s_blk[k] + off);
                    const u4 w = {x.x, x.y, x.z, x.w};
                    __builtin_amdgcn_raw_buffer_store_b128(w, pass_rsrc(k ? bblk : sblk, 1, 0, SBLK), (int)off, 0,
                                                           kStream);
                }
                __syncthreads();               // the block is read before the next (batch, head) fills it
            }
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
    constexpr int RPB = 4 * (64 / (D / 8)) * kQuantPasses;
    const int64_t bx = (p.T + RPB - 1) / RPB;
    if (bx == 0 || p.BH == 0) return hipSuccess;
    if (bx > 0x7fffffff || p.BH > 0x7fffffff) return hipErrorInvalidValue;
    const unsigned by = (unsigned)std::min<int64_t>(p.BH, 65535);
    hipLaunchKernelGGL((quantize_rows_kernel<DT, MODE, BITS, GS, D>), dim3((unsigned)bx, by, njobs),
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
