// Single-query decode (fp16 queries, at most 4 query heads per kv head) for
// the formats whose codes are a bit stream per row: affine codes of 2, 3, 5
// and 6 bits (and 4/8 bits at head size 96), the symmetric 4/5-bit blocks and
// Q8_0 at head size 96.  What is computed is the decode of the MLX page "add
// fast::quantized_kv_update" (sdpa_vector.h quant_sdpa_vector: scores from
// packed codes through q . (s c + b) = s (q . c) + b (sum q) per group, online
// softmax, merge of partial softmax states), over the packed layout of the MLX
// CUDA page "Fixed mma and working dequant" (quantized_utils.cuh: any bit
// width packs into whole words) read as one least-significant-first bit
// stream per row, and the symmetric blocks of the llama.cpp page "Metal:
// Optimize q8_0 KV - #25556" (merged #27390 text: q4_0/q5_0 caches).
//
// Work layout (wave64): a workgroup of 4 waves takes one key split of one
// (batch, kv head); wave w takes the split's 64-key tiles w, w + 4, ... (a
// fixed order, so every call gives the same bits), with its own running
// softmax, and the 4 waves' states are combined at the end.  No barrier is
// taken inside the loop.
//
//  * q K^T: lane l holds key l of the tile -- the words of its row's code
//    stream, its group scales and biases -- and extracts each code with a
//    bit-field extract (a funnel shift first where a code straddles two
//    words; offsets are compile-time constants); signed codes are taken in
//    offset form (top bit flipped) with -2^(BITS-1) d folded into the bias.  The 4 heads' pre-scaled
//    queries sit in LDS as [d][head] fp32, so one broadcast read gives the 4
//    factors of a d; per group, z_h += s_g (q_h . c) + b_g (sum_{d in g} q_h).
//  * softmax per head over the wave's 64 scores (log2 units; the maximum by
//    DPP and cross-row swaps), rescaling the running state once per tile.
//  * P V: the lane dequantizes its key's value row (s c + b, rounded once to
//    fp16) into the wave's LDS tile [key][D] (a row stride of D + 2 halves, an
//    odd number of words, so the 64 row writes of a column fall on distinct
//    banks) and its 4 probabilities into [key][head]; then lane l owns the
//    pairs of d 2l + 128 i, reads one word per key and accumulates 4 heads.
//
// With several splits each workgroup writes its (m, l, o) state in the
// 16-row layout of the split merge kernels, which combine them.
#include "qkv_internal.hpp"
#include "qkv_mfma.hpp"

namespace qkv {

namespace {

using namespace mf;

constexpr int SW = 4;           // waves per workgroup
constexpr int STK = 64;         // keys per wave tile
constexpr int WS_ROWS = 16;     // rows per tile in the split workspace (the merge kernels' layout)

// Code of element E of a row from its words (compile-time bit position), as
// an unsigned value.  Signed codes (symmetric blocks, Q8_0: two's complement)
// come out in offset form, c + 2^(BITS-1) (the top bit flipped), and the
// caller subtracts 2^(BITS-1) d through the group's bias term, so no signed
// conversion is needed.
template <int BITS, bool SIGNED, int E>
__device__ __forceinline__ float code_of(const uint32_t* w) {
    constexpr int bit = E * BITS;
    constexpr int wi = bit >> 5, sh = bit & 31;
    uint32_t x;
    if constexpr (sh + BITS <= 32) x = w[wi];
    else x = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh);
    constexpr int s2 = (sh + BITS <= 32) ? sh : 0;
    uint32_t u = __builtin_amdgcn_ubfe(x, s2, BITS);
    if constexpr (SIGNED) u ^= 1u << (BITS - 1);
    return (float)u;
}

// Load nw words of a row at byte offset off (off and the row stride are
// multiples of the access width).
template <int ROWB>
__device__ __forceinline__ void load_row(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* w) {
    constexpr int NW = ROWB / 4;
    if constexpr (ROWB % 16 == 0) {
#pragma unroll
        for (int i = 0; i < NW; i += 4) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 4 * i), 0, 0);
            w[i] = x[0]; w[i + 1] = x[1]; w[i + 2] = x[2]; w[i + 3] = x[3];
        }
    } else if constexpr (ROWB % 8 == 0) {
#pragma unroll
        for (int i = 0; i < NW; i += 2) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)(off + 4 * i), 0, 0);
            w[i] = x[0]; w[i + 1] = x[1];
        }
    } else {
#pragma unroll
        for (int i = 0; i < NW; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(off + 4 * i), 0, 0);
    }
}

template <int MODE, int BITS, int GS, int D>
__global__ __launch_bounds__(SW * 64) void attn_decode_stream(AttnLaunch p) {
    constexpr int GSZ = MODE == MODE_AFFINE ? GS : 32;    // elements per scale
    constexpr int NG = D / GSZ;
    constexpr int ROWB = D * BITS / 8;                    // code bytes of a row
    constexpr int NWD = ROWB / 4;                         // words of a row
    constexpr bool SIGNED = MODE != MODE_AFFINE;
    constexpr float kOff = SIGNED ? -(float)(1 << (BITS - 1)) : 0.0f;   // bias of offset codes, per unit scale
    constexpr int VROW = D + 2;                           // LDS value row (halves)
    constexpr int DPL = (D + 127) / 128;                  // d pairs per lane in P V
    static_assert(ROWB % 4 == 0, "whole words per row");
    static_assert(NG <= 8, "at most 8 groups per row");

    __shared__ __attribute__((aligned(16))) float s_q[D][4];     // pre-scaled q, [d][head]
    __shared__ float s_qs[NG][4];                                // per-group sums of q
    __shared__ __attribute__((aligned(16))) _Float16 s_v[SW][STK * VROW];
    __shared__ __attribute__((aligned(16))) float s_p[SW][STK][4];
    __shared__ float s_ml[SW][2][4];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int split = blockIdx.x;
    const int64_t kvh = blockIdx.y;
    const int64_t b = blockIdx.z;
    pin_sgpr(p.q); pin_sgpr(p.Hq); pin_sgpr(p.Hk); pin_sgpr(p.G); pin_sgpr(p.L); pin_sgpr(p.chunk);
    pin_sgpr(p.scale); pin_sgpr(p.mask_kind); pin_sgpr(p.S);
    pin_sgpr(p.k.codes); pin_sgpr(p.k.scales); pin_sgpr(p.k.biases);
    pin_sgpr(p.k.sb); pin_sgpr(p.k.sh); pin_sgpr(p.k.sl);
    pin_sgpr(p.v.codes); pin_sgpr(p.v.scales); pin_sgpr(p.v.biases);
    pin_sgpr(p.v.sb); pin_sgpr(p.v.sh); pin_sgpr(p.v.sl);
    const int G = p.G;
    const int64_t bk = b * p.Hk + kvh;

    const int64_t j0 = (int64_t)split * p.chunk;
    const int64_t j1 = min(p.L, j0 + p.chunk);
    const int ntiles = j1 > j0 ? (int)((j1 - j0 + STK - 1) / STK) : 0;

    // queries of the kv head's G heads, times scale log2 e (heads past G: 0)
    const float sl = p.scale * kLog2e;
    for (int i = tid; i < D * 4; i += SW * 64) {
        const int d = i >> 2, h = i & 3;
        const _Float16* qrow = (const _Float16*)p.q + (b * p.Hq + kvh * G + min(h, G - 1)) * D;
        s_q[d][h] = h < G ? (float)qrow[d] * sl : 0.0f;
    }
    __syncthreads();
    if (tid < NG * 4) {
        const int g = tid >> 2, h = tid & 3;
        float s = 0.0f;
        for (int e = 0; e < GSZ; ++e) s += s_q[g * GSZ + e][h];
        s_qs[g][h] = s;
    }
    __syncthreads();

    const int64_t krow0 = b * p.k.sb + kvh * p.k.sh;
    const int64_t vrow0 = b * p.v.sb + kvh * p.v.sh;
    constexpr int SROWB = NG * 2;
    const uint8_t* kc = (const uint8_t*)p.k.codes + krow0 * ROWB;
    const uint8_t* vc = (const uint8_t*)p.v.codes + vrow0 * ROWB;
    const uint8_t* ksc = (const uint8_t*)p.k.scales + krow0 * SROWB;
    const uint8_t* vsc = (const uint8_t*)p.v.scales + vrow0 * SROWB;
    const uint8_t* kbi = (const uint8_t*)p.k.biases + krow0 * SROWB;
    const uint8_t* vbi = (const uint8_t*)p.v.biases + vrow0 * SROWB;
    const uint32_t kcs = (uint32_t)(p.k.sl * ROWB), vcs = (uint32_t)(p.v.sl * ROWB);
    const uint32_t kss = (uint32_t)(p.k.sl * SROWB), vss = (uint32_t)(p.v.sl * SROWB);

    // one key row (K or V) of the lane: its code words and its groups' fp16
    // scales and biases
    struct Row {
        uint32_t w[NWD];
        uint32_t s[NG], b[NG];
    };
    auto load_rowset = [&](int tt, const uint8_t* codes, const uint8_t* scales, const uint8_t* biases,
                           uint32_t cs, uint32_t ss, Row& R) {
        const int64_t row0 = j0 + (int64_t)tt * STK;
        load_row<ROWB>(rows_rsrc(codes, row0, j1, STK, cs, ROWB), (uint32_t)lane * cs, R.w);
        const auto rs = rows_rsrc(scales, row0, j1, STK, ss, SROWB);
#pragma unroll
        for (int g = 0; g < NG; ++g) R.s[g] = buf16(rs, (uint32_t)lane * ss + 2 * g);
        if constexpr (MODE == MODE_AFFINE) {
            const auto rb = rows_rsrc(biases, row0, j1, STK, ss, SROWB);
#pragma unroll
            for (int g = 0; g < NG; ++g) R.b[g] = buf16(rb, (uint32_t)lane * ss + 2 * g);
        } else {
#pragma unroll
            for (int g = 0; g < NG; ++g) R.b[g] = 0u;
        }
    };
    auto load_k = [&](int tt, Row& R) { load_rowset(tt, kc, ksc, kbi, kcs, kss, R); };
    auto load_v = [&](int tt, Row& R) { load_rowset(tt, vc, vsc, vbi, vcs, vss, R); };

    float m_h[4], l_h[4];
    float o[DPL][2][4];                                   // [pair][d of the pair][head]
#pragma unroll
    for (int h = 0; h < 4; ++h) { m_h[h] = -INFINITY; l_h[h] = 0.0f; }
#pragma unroll
    for (int i = 0; i < DPL; ++i)
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int h = 0; h < 4; ++h) o[i][e][h] = 0.0f;
    _Float16* vt = s_v[wave];

    // scores of the lane's key for the 4 heads (log2 units), then the online
    // softmax: the probabilities of the tile
    auto scores = [&](const Row& K, int tt, float pr[4]) {
        const int64_t j = j0 + (int64_t)tt * STK + lane;
        // ---- scores of the lane's key for the 4 heads (log2 units)
        float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        // 32 elements (BITS words of the row) at a time.  The chunk's words, the
        // q pointer and the chunk's sums pass through empty asm statements, so
        // the compiler cannot extract the codes or read the q factors of later
        // chunks early (which keeps 4 D q values and D codes live and spills).
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        static_for<0, D / 32>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            constexpr int g = 32 * c / GSZ;
            uint32_t wc[BITS];
#pragma unroll
            for (int i = 0; i < BITS; ++i) {
                wc[i] = K.w[c * BITS + i];
                __asm__ __volatile__("" : "+v"(wc[i]));
            }
            int qo = 128 * c;                             // floats: 32 d x 4 heads per chunk
            __asm__ __volatile__("" : "+v"(qo));
            const float* sq = &s_q[0][0] + qo;
            static_for<0, 32>([&](auto ec) {
                constexpr int e = decltype(ec)::value;
                const float cv = code_of<BITS, SIGNED, e>(wc);
                const f4 qv = *(const f4*)(sq + 4 * e);
#pragma unroll
                for (int h = 0; h < 4; ++h) acc[h] = __builtin_fmaf(qv[h], cv, acc[h]);
            });
            if constexpr ((32 * (c + 1)) % GSZ == 0) {       // the group ends with this chunk
                const float sc = f16_to_f32((uint16_t)K.s[g]);
                const float bb = SIGNED ? kOff * sc : f16_to_f32((uint16_t)K.b[g]);
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    z[h] = __builtin_fmaf(sc, acc[h], __builtin_fmaf(bb, s_qs[g][h], z[h]));
                    acc[h] = 0.0f;
                }
            }
#pragma unroll
            for (int h = 0; h < 4; ++h) __asm__ __volatile__("" : "+v"(acc[h]), "+v"(z[h]));
        });
        const bool valid = j < j1;
#pragma unroll
        for (int h = 0; h < 4; ++h) if (!valid || h >= G) z[h] = -INFINITY;
        if (p.mask_kind == MASK_ADDITIVE && valid) {
#pragma unroll
            for (int h = 0; h < 4; ++h)
                if (h < G)
                    z[h] += kLog2e * load_mask(p.mask, p.mask_dtype,
                                               b * p.ms0 + (kvh * G + h) * p.ms1 + j * p.ms3);
        }
        // ---- online softmax per head, one rescale per tile
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const float mt = wave_max(z[h]);
            const float mn = fmaxf(m_h[h], mt);
            const float alpha = (m_h[h] == -INFINITY) ? 0.0f : fast_exp2(m_h[h] - mn);
            m_h[h] = mn;
            l_h[h] *= alpha;
#pragma unroll
            for (int i = 0; i < DPL; ++i) { o[i][0][h] *= alpha; o[i][1][h] *= alpha; }
            pr[h] = (mn == -INFINITY || z[h] == -INFINITY) ? 0.0f : fast_exp2(z[h] - mn);
            l_h[h] += pr[h];
        }
    };
    // the key's value row (fp16) and probabilities to the wave's LDS tile, then
    // o += P V over the tile
    auto values = [&](const Row& V, const float pr[4]) {
        static_for<0, D / 32>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            constexpr int g = 32 * c / GSZ;
            uint32_t wc[BITS];
#pragma unroll
            for (int i = 0; i < BITS; ++i) {
                wc[i] = V.w[c * BITS + i];
                __asm__ __volatile__("" : "+v"(wc[i]));
            }
            const float sc = f16_to_f32((uint16_t)V.s[g]);
            const float bb = SIGNED ? kOff * sc : f16_to_f32((uint16_t)V.b[g]);
            _Float16* dst = vt + lane * VROW + 32 * c;
            static_for<0, 16>([&](auto ic) {
                constexpr int e = 2 * decltype(ic)::value;
                const float x0 = __builtin_fmaf(sc, code_of<BITS, SIGNED, e>(wc), bb);
                const float x1 = __builtin_fmaf(sc, code_of<BITS, SIGNED, e + 1>(wc), bb);
                const uint32_t w = (uint32_t)f32_to_f16(x0) | ((uint32_t)f32_to_f16(x1) << 16);
                *(uint32_t*)(dst + e) = w;
            });
        });
        *(f4*)&s_p[wave][lane][0] = f4{pr[0], pr[1], pr[2], pr[3]};
        lds_order();
        // ---- o[h][d] += sum_key p[key][h] V[key][d]: lane l owns d = 2 l + 128 i (+1)
#pragma unroll 4
        for (int key = 0; key < STK; ++key) {
            const f4 pk = *(const f4*)&s_p[wave][key][0];
#pragma unroll
            for (int i = 0; i < DPL; ++i) {
                const int d = 2 * lane + 128 * i;
                if (d < D) {
                    const uint32_t w = *(const uint32_t*)(vt + key * VROW + d);
                    const float v0 = f16_to_f32((uint16_t)(w & 0xffffu)), v1 = f16_to_f32((uint16_t)(w >> 16));
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        o[i][0][h] = __builtin_fmaf(pk[h], v0, o[i][0][h]);
                        o[i][1][h] = __builtin_fmaf(pk[h], v1, o[i][1][h]);
                    }
                }
            }
        }
        lds_order();
    };

    // One K row set and one V row set in registers: the next tile's K rows
    // are requested once the scores of the current tile are done, its V rows
    // once the current values are in LDS, so each load overlaps the other
    // half of a tile's work.
    Row kr, vr;
    int tt = wave;
    if (tt < ntiles) { load_k(tt, kr); load_v(tt, vr); }
    while (tt < ntiles) {
        const int tn = tt + SW;
        float pr[4];
        scores(kr, tt, pr);
        if (tn < ntiles) load_k(tn, kr);
        values(vr, pr);
        if (tn < ntiles) load_v(tn, vr);
        tt = tn;
    }

    // ---- combine the 4 waves' states (through the LDS value tiles)
#pragma unroll
    for (int h = 0; h < 4; ++h) l_h[h] = wave_sum(l_h[h]);
    __syncthreads();                                      // every wave is done with its tiles
    float* xo = (float*)&s_v[0][0];                       // [wave][head][D] fp32
    static_assert(SW * 4 * D * 4 <= SW * STK * VROW * 2, "the state fits the value tiles");
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
        const int d = 2 * lane + 128 * i;
        if (d < D) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                xo[(wave * 4 + h) * D + d] = o[i][0][h];
                xo[(wave * 4 + h) * D + d + 1] = o[i][1][h];
            }
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < 4; ++h) { s_ml[wave][0][h] = m_h[h]; s_ml[wave][1][h] = l_h[h]; }
    }
    __syncthreads();
    const int64_t tile = bk;                              // one 16-row tile per (batch, kv head)
    for (int i = tid; i < G * D; i += SW * 64) {
        const int h = i / D, d = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < SW; ++w) M = fmaxf(M, s_ml[w][0][h]);
        float Lh = 0.0f, oh = 0.0f;
#pragma unroll
        for (int w = 0; w < SW; ++w) {
            const float mw = s_ml[w][0][h];
            const float f = mw == -INFINITY ? 0.0f : fast_exp2(mw - M);
            Lh += f * s_ml[w][1][h];
            oh += f * xo[(w * 4 + h) * D + d];
        }
        if (p.S == 1) {
            const float inv = Lh > 0.0f ? 1.0f / Lh : 0.0f;
            ((uint16_t*)p.out)[(b * p.Hq + kvh * G + h) * D + d] = f32_to_f16(oh * inv);
        } else {
            p.part_o[((tile * p.S + split) * WS_ROWS + h) * D + d] = oh;
            if (d == 0) {
                p.part_ml[((tile * p.S + split) * WS_ROWS + h) * 2] = M;
                p.part_ml[((tile * p.S + split) * WS_ROWS + h) * 2 + 1] = Lh;
            }
        }
    }
}

template <int MODE, int BITS, int GS, int D>
hipError_t launch_s(int64_t B, const AttnLaunch& p, hipStream_t stream) {
    dim3 grid(p.S, (unsigned)p.Hk, (unsigned)B);
    hipLaunchKernelGGL((attn_decode_stream<MODE, BITS, GS, D>), grid, dim3(SW * 64), 0, stream, p);
    return hipGetLastError();
}

// the instantiated shapes: the group divides the row, and the matrix-core
// kernels do not already take the format
template <int MODE, int BITS, int GS, int D>
constexpr bool stream_shape() {
    return D % GS == 0 && !fast_format(MODE, BITS, D);
}

template <int MODE, int BITS, int GS>
hipError_t by_d(int D, int64_t B, const AttnLaunch& p, hipStream_t s) {
    switch (D) {
        case 64: if constexpr (stream_shape<MODE, BITS, GS, 64>()) return launch_s<MODE, BITS, GS, 64>(B, p, s); else break;
        case 96: if constexpr (stream_shape<MODE, BITS, GS, 96>()) return launch_s<MODE, BITS, GS, 96>(B, p, s); else break;
        case 128: if constexpr (stream_shape<MODE, BITS, GS, 128>()) return launch_s<MODE, BITS, GS, 128>(B, p, s); else break;
        case 256: if constexpr (stream_shape<MODE, BITS, GS, 256>()) return launch_s<MODE, BITS, GS, 256>(B, p, s); else break;
    }
    return hipErrorNotSupported;
}

template <int BITS>
hipError_t by_gs(int gs, int D, int64_t B, const AttnLaunch& p, hipStream_t s) {
    if (gs == 32) return by_d<MODE_AFFINE, BITS, 32>(D, B, p, s);
    if (gs == 64) return by_d<MODE_AFFINE, BITS, 64>(D, B, p, s);
    if (gs == 128) return by_d<MODE_AFFINE, BITS, 128>(D, B, p, s);
    return hipErrorNotSupported;
}

}  // namespace

bool stream_decode_supported(int q_dtype, int mode, int bits, int group_size, int scale_dtype, int D,
                             int G, int64_t Lq) {
    if (q_dtype != DT_F16 || Lq != 1 || G < 1 || G > 4) return false;
    if (D != 64 && D != 96 && D != 128 && D != 256) return false;
    if (fast_format(mode, bits, D)) return false;         // the matrix-core kernels take these
    if (mode == MODE_Q8_0) return D % 32 == 0;
    if (mode == MODE_QSYM) return (bits == 4 || bits == 5) && group_size == 32;
    if (mode != MODE_AFFINE || scale_dtype != DT_F16) return false;
    if (bits != 2 && bits != 3 && bits != 4 && bits != 5 && bits != 6 && bits != 8) return false;
    if (group_size != 32 && group_size != 64 && group_size != 128) return false;
    return D % group_size == 0;
}

int stream_decode_key_quantum() { return STK * SW; }

hipError_t launch_attn_stream(int mode, int bits, int D, int64_t B, const AttnLaunch& p,
                              hipStream_t stream) {
    const int gs = 1 << p.gs_log2;
    if (mode == MODE_Q8_0) return by_d<MODE_Q8_0, 8, 32>(D, B, p, stream);
    if (mode == MODE_QSYM) {
        if (bits == 4) return by_d<MODE_QSYM, 4, 32>(D, B, p, stream);
        if (bits == 5) return by_d<MODE_QSYM, 5, 32>(D, B, p, stream);
        return hipErrorNotSupported;
    }
    switch (bits) {
        case 2: return by_gs<2>(gs, D, B, p, stream);
        case 3: return by_gs<3>(gs, D, B, p, stream);
        case 4: return by_gs<4>(gs, D, B, p, stream);
        case 5: return by_gs<5>(gs, D, B, p, stream);
        case 6: return by_gs<6>(gs, D, B, p, stream);
        case 8: return by_gs<8>(gs, D, B, p, stream);
    }
    return hipErrorNotSupported;
}

}  // namespace qkv
