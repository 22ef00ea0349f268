// Generic attention over a quantized KV cache: every supported combination of
// query dtype (fp32 / fp16 / bf16), cache format (affine 4/8-bit, Q8_0), head
// size and GQA factor, for decode (Lq = 1) and prefill (Lq > 1).
//
//   out[b,h,i,:] = softmax_j(scale * q[b,h,i,:] . K^[b,h/G,j,:] + m_ij) V^[b,h/G,j,:]
//
// (MLX page "add fast::quantized_kv_update": fast.cpp
// quantized_scaled_dot_product_attention -- q reshaped to
// [B, Hk, Hq/Hk, L, D] so each kv head serves G query heads -- and
// sdpa_vector.h quant_sdpa_vector for the online softmax and the merge of
// partial softmax states.)
//
// Work decomposition: one workgroup per (key split, row tile, batch x kv head).
// The rows of a kv head are its G query heads times Lq queries, packed as
// row p = i*G + g, so one tile shares every K/V load among the GQA heads (as
// the llama.cpp page "Metal: Optimize q8_0 KV - #25556" does for two heads)
// and, for prefill, among neighbouring queries.  Keys are consumed in blocks
// of 32: scores (8 lanes per key, butterfly sum), an online-softmax update per
// row, the V block dequantized once into LDS, then o = o*alpha + P V.  Thread
// t holds the packed K and V words of key t / 8, d slice t % 8 of a block
// (one quantization group) in registers; the next block's words are requested
// before the current block is processed, so a block costs one memory round
// trip at most (the first block's loads overlap the query loads).
// With several splits each workgroup writes its (m, l, o) state to the
// workspace and the split merge kernel combines them with the log-sum-exp
// rule and writes the output.  This kernel favours generality over
// speed; the matrix-core kernels cover the fp16 hot shapes.
#include <type_traits>

#include "qkv_device.hpp"
#include "qkv_internal.hpp"
#include "qkv_merge.hpp"

namespace qkv {

namespace {

constexpr int KB = 32;      // keys per block
constexpr int WS_ROWS = 16; // rows per tile in the split workspace (the merge kernels' layout)

// The packed words of one d slice (DPK = D / 8 consecutive d, inside one
// quantization group) of one K row and one V row, with their scale / bias.
template <int MODE, int BITS, int D>
struct RawSlice {
    static constexpr int DPK = D / 8;
    static constexpr int W = DPK * BITS / 32 > 0 ? DPK * BITS / 32 : 1;
    uint32_t k[W], v[W];
    float ks, kb, vs, vb;
};

// Element e of a slice, dequantized in fp32: affine s c + b, Q8_0 d c.
template <int MODE, int BITS>
__device__ __forceinline__ float slice_elem(const uint32_t* w, float s, float b, int e) {
    if constexpr (MODE == MODE_Q8_0) {
        const int8_t c = (int8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xFFu);
        return s * (float)c;
    } else {
        const uint32_t c = (w[(e * BITS) >> 5] >> ((e * BITS) & 31)) & ((1u << BITS) - 1u);
        return s * (float)c + b;
    }
}

// The general formats (affine 2/3/5/6-bit, symmetric 4/5-bit blocks, head
// size 96): the words of a row's bit stream that cover the slice's
// DPK * BITS bits, funnel-shifted so that the slice starts at bit 0 (the
// element offsets are then compile-time constants), and the scale / bias of
// the slice's first and last quantization group (a slice of D / 8 <= 32
// elements spans at most two groups of >= 32).
template <int MODE, int BITS, int D>
struct StreamSlice {
    static constexpr int DPK = D / 8;
    static constexpr int W = (DPK * BITS + 31) / 32;     // words of the aligned slice
    uint32_t k[W], v[W];
    float ks[2], kb[2], vs[2], vb[2];
    int split;                                           // first element of the second group
};

template <int MODE, int BITS>
__device__ __forceinline__ float stream_elem(const uint32_t* w, const float* s, const float* b, int split,
                                             int e) {
    const int bit = e * BITS;
    uint32_t u = w[bit >> 5] >> (bit & 31);
    if ((bit & 31) + BITS > 32) u |= w[(bit >> 5) + 1] << (32 - (bit & 31));
    u &= (1u << BITS) - 1u;
    const int gi = e >= split ? 1 : 0;
    if constexpr (MODE == MODE_AFFINE) {
        return s[gi] * (float)u + b[gi];
    } else {
        const int c = (int)(u << (32 - BITS)) >> (32 - BITS);   // two's complement
        return s[gi] * (float)c;
    }
}

// RTG rows per tile: 16, or 4 for a single query of at most 4 heads per kv
// head (a decode with G <= 4), which then costs a quarter of the arithmetic.
template <int QT, int MODE, int BITS, int D, int RTG>
__global__ __launch_bounds__(256) void attn_generic_kernel(AttnLaunch p) {
    constexpr bool STREAM = !fast_format(MODE, BITS, D);
    constexpr int ST = (MODE == MODE_AFFINE) ? QT : DT_F16;  // scale dtype
    constexpr int DPK = D / 8;                               // d per lane (scores)
    // output: OC chunks of DPO d per row, RTG * OC <= 256 threads
    constexpr int OC = D % (256 / RTG) == 0 ? 256 / RTG : 256 / RTG / 2;
    constexpr int DPO = D / OC;
    static_assert(D % OC == 0 && RTG * OC <= 256, "output mapping");
    // softmax: TPR threads per row, KPT keys per thread
    constexpr int KPT = KB * RTG / 256 >= 1 ? KB * RTG / 256 : 1;
    constexpr int TPR = KB / KPT;
    __shared__ float qs[RTG][D];
    __shared__ float sc[RTG][KB];
    __shared__ float vt[KB][D];
    __shared__ float m_s[RTG], l_s[RTG], a_s[RTG];

    const int tid = threadIdx.x;
    const int split = blockIdx.x;
    const int rt = blockIdx.y;
    const int64_t bk = blockIdx.z;
    const int64_t b = bk / p.Hk;
    const int64_t kvh = bk % p.Hk;
    const int r0 = rt * RTG;
    const int nr = min(RTG, p.n_rows - r0);

    // key range of this split, cut at the last key any row of the tile sees
    int64_t j_begin = (int64_t)split * p.chunk;
    int64_t j_end = min(p.L, j_begin + p.chunk);
    if (p.mask_kind == MASK_CAUSAL) {
        const int64_t i_max = (r0 + nr - 1) / p.G;
        j_end = min(j_end, p.L - p.Lq + i_max + 1);
    }

    const int64_t krow0 = b * p.k.sb + kvh * p.k.sh;
    const int64_t vrow0 = b * p.v.sb + kvh * p.v.sh;
    const uint8_t* kc = (const uint8_t*)p.k.codes;
    const uint8_t* vc = (const uint8_t*)p.v.codes;

    // this thread's key of a block and d slice (one quantization group, or
    // up to two for the general formats)
    using Raw = std::conditional_t<STREAM, StreamSlice<MODE, BITS, D>, RawSlice<MODE, BITS, D>>;
    constexpr int ROWB = D * BITS / 8;
    const int kk = tid / 8, part = tid % 8;
    const int NGr = D >> p.gs_log2;
    const int gsl = (part * Raw::DPK) >> p.gs_log2;
    // rows past the range load the range's last row (never used: their scores
    // are -inf and their V entries 0), so the loads need no branch
    const int64_t j_last = max(j_end - 1, (int64_t)0);
    // general formats: the slice's first bit, word and groups
    constexpr int RW = D * BITS / 32;                    // words per row
    const int fbit = part * Raw::DPK * BITS;
    const int w0 = fbit >> 5, sh0 = fbit & 31;
    const int g0 = (part * Raw::DPK) >> p.gs_log2;
    const int g1 = (part * Raw::DPK + Raw::DPK - 1) >> p.gs_log2;
    const int gsplit = ((g0 + 1) << p.gs_log2) - part * Raw::DPK;
    auto load_stream = [&](const uint8_t* base, int64_t r, uint32_t* out) {
        const uint32_t* rw = (const uint32_t*)(base + r * ROWB);
        uint32_t x[Raw::W + 1];
#pragma unroll
        for (int i = 0; i <= Raw::W; ++i) x[i] = rw[min(w0 + i, RW - 1)];
#pragma unroll
        for (int i = 0; i < Raw::W; ++i)
            out[i] = sh0 ? (x[i] >> sh0) | (x[i + 1] << (32 - sh0)) : x[i];
    };
    auto load_raw = [&](int64_t jb, Raw& R) {
        const int64_t j = min(jb + kk, j_last);
        const int64_t kr = krow0 + j * p.k.sl, vr = vrow0 + j * p.v.sl;
        if constexpr (STREAM) {
            load_stream(kc, kr, R.k);
            load_stream(vc, vr, R.v);
            R.split = gsplit;
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                const int gg = t2 ? g1 : g0;
                R.ks[t2] = load_as_f32<ST>(p.k.scales, kr * NGr + gg);
                R.vs[t2] = load_as_f32<ST>(p.v.scales, vr * NGr + gg);
                if constexpr (MODE == MODE_AFFINE) {
                    R.kb[t2] = load_as_f32<ST>(p.k.biases, kr * NGr + gg);
                    R.vb[t2] = load_as_f32<ST>(p.v.biases, vr * NGr + gg);
                } else {
                    R.kb[t2] = R.vb[t2] = 0.0f;
                }
            }
            return;
        } else {
        const uint32_t* kw = (const uint32_t*)(kc + kr * ROWB) + part * Raw::W;
        const uint32_t* vw = (const uint32_t*)(vc + vr * ROWB) + part * Raw::W;
#pragma unroll
        for (int w = 0; w < Raw::W; ++w) { R.k[w] = kw[w]; R.v[w] = vw[w]; }
        R.ks = load_as_f32<ST>(p.k.scales, kr * NGr + gsl);
        R.vs = load_as_f32<ST>(p.v.scales, vr * NGr + gsl);
        if constexpr (MODE == MODE_Q8_0) {
            R.kb = R.vb = 0.0f;
        } else {
            R.kb = load_as_f32<ST>(p.k.biases, kr * NGr + gsl);
            R.vb = load_as_f32<ST>(p.v.biases, vr * NGr + gsl);
        }
        }
    };
    auto k_elem = [&](const Raw& R, int e) -> float {
        if constexpr (STREAM) return stream_elem<MODE, BITS>(R.k, R.ks, R.kb, R.split, e);
        else return slice_elem<MODE, BITS>(R.k, R.ks, R.kb, e);
    };
    auto v_elem = [&](const Raw& R, int e) -> float {
        if constexpr (STREAM) return stream_elem<MODE, BITS>(R.v, R.vs, R.vb, R.split, e);
        else return slice_elem<MODE, BITS>(R.v, R.vs, R.vb, e);
    };
    Raw cur, nxt;
    load_raw(j_begin, cur);

    // queries of the tile, pre-multiplied by the softmax scale (fp32); rows
    // past the tile's last read row 0 and store zeros, so every load is
    // issued before the first wait
    for (int idx = tid; idx < RTG * D; idx += 256) {
        const int r = idx / D, d = idx % D;
        const int pr = r0 + (r < nr ? r : 0);
        const int64_t i = pr / p.G, h = kvh * p.G + pr % p.G;
        const float x = load_as_f32<QT>(p.q, ((b * p.Hq + h) * p.Lq + i) * D + d);
        qs[r][d] = r < nr ? x * p.scale : 0.0f;
    }
    if (tid < RTG) { m_s[tid] = -INFINITY; l_s[tid] = 0.0f; }

    const int orow = tid / OC, ochunk = tid % OC;
    const int orow_c = min(orow, RTG - 1);              // threads past the rows read row RTG - 1
    float o[DPO];
#pragma unroll
    for (int i = 0; i < DPO; ++i) o[i] = 0.0f;
    __syncthreads();

    for (int64_t jb = j_begin; jb < j_end; jb += KB) {
        if (jb + KB < j_end) load_raw(jb + KB, nxt);
        // ---- scores: 8 lanes per key
        {
            const int64_t j = jb + kk;
            const bool valid = j < j_end;
            float acc[RTG];
#pragma unroll
            for (int r = 0; r < RTG; ++r) acc[r] = 0.0f;
            if (valid) {
#pragma unroll
                for (int e = 0; e < DPK; ++e) {
                    const int d = part * DPK + e;
                    const float kv = k_elem(cur, e);
#pragma unroll
                    for (int r = 0; r < RTG; ++r) acc[r] += qs[r][d] * kv;
                }
            }
#pragma unroll
            for (int r = 0; r < RTG; ++r) {
                float a = acc[r];
                a += __shfl_xor(a, 1, 64);
                a += __shfl_xor(a, 2, 64);
                a += __shfl_xor(a, 4, 64);
                acc[r] = a;
            }
            if (part == 0) {
#pragma unroll
                for (int r = 0; r < RTG; ++r) {
                    float z = -INFINITY;
                    if (valid && r < nr) {
                        const int pr = r0 + r;
                        const int64_t i = pr / p.G, h = kvh * p.G + pr % p.G;
                        z = acc[r];
                        if (p.mask_kind == MASK_CAUSAL && j > p.L - p.Lq + i) z = -INFINITY;
                        if (p.mask_kind == MASK_ADDITIVE)
                            z += load_mask(p.mask, p.mask_dtype,
                                           b * p.ms0 + h * p.ms1 + i * p.ms2 + j * p.ms3);
                    }
                    sc[r][kk] = z;
                }
            }
        }
        __syncthreads();
        // ---- online softmax update: TPR lanes per row, KPT keys per lane
        if (tid < RTG * TPR) {                         // whole waves
            const int r = tid / TPR, lt = tid % TPR;
            float z[KPT];
            float mb = -INFINITY;
#pragma unroll
            for (int k = 0; k < KPT; ++k) {
                z[k] = sc[r][lt + k * TPR];
                mb = fmaxf(mb, z[k]);
            }
#pragma unroll
            for (int o2 = 1; o2 < TPR; o2 <<= 1) mb = fmaxf(mb, __shfl_xor(mb, o2, 64));
            const float m_old = m_s[r];
            const float m_new = fmaxf(m_old, mb);
            float pk[KPT], alpha = 1.0f, ps = 0.0f;
#pragma unroll
            for (int k = 0; k < KPT; ++k) pk[k] = 0.0f;
            if (m_new != -INFINITY) {
                alpha = (m_old == -INFINITY) ? 0.0f : fast_exp2((m_old - m_new) * kLog2e);
#pragma unroll
                for (int k = 0; k < KPT; ++k) pk[k] = (z[k] == -INFINITY) ? 0.0f : fast_exp2((z[k] - m_new) * kLog2e);
            }
#pragma unroll
            for (int k = 0; k < KPT; ++k) ps += pk[k];
#pragma unroll
            for (int o2 = 1; o2 < TPR; o2 <<= 1) ps += __shfl_xor(ps, o2, 64);
#pragma unroll
            for (int k = 0; k < KPT; ++k) sc[r][lt + k * TPR] = pk[k];
            if (lt == 0) {
                m_s[r] = m_new;
                l_s[r] = l_s[r] * alpha + ps;
                a_s[r] = alpha;
            }
        }
        // ---- V block -> LDS (fp32; keys past the range hold zeros)
#pragma unroll
        for (int e = 0; e < DPK; ++e)
            vt[kk][part * DPK + e] = (jb + kk < j_end) ? v_elem(cur, e) : 0.0f;
        __syncthreads();
        // ---- o = o * alpha + P V
        {
            const float alpha = a_s[orow_c];
#pragma unroll
            for (int i = 0; i < DPO; ++i) o[i] *= alpha;
            for (int key = 0; key < KB; ++key) {
                const float pk = sc[orow_c][key];
#pragma unroll
                for (int i = 0; i < DPO; ++i) o[i] += pk * vt[key][ochunk * DPO + i];
            }
        }
        __syncthreads();
        cur = nxt;
    }

    const bool row_ok = orow < nr;                       // (nr <= RTG)
    const int pr = r0 + orow;
    const int64_t oi = row_ok ? (int64_t)(pr / p.G) : 0;
    const int64_t oh = row_ok ? kvh * p.G + pr % p.G : 0;
    const int64_t obase = ((b * p.Hq + oh) * p.Lq + oi) * D + ochunk * DPO;

    if (p.S == 1) {
        if (row_ok) {
            const float l = l_s[orow_c];
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
            for (int i = 0; i < DPO; ++i) store_from_f32<QT>(p.out, obase + i, o[i] * inv);
        }
        return;
    }

    // ---- partial state -> workspace, then the last workgroup merges
    const int64_t tile = bk * p.n_rt + rt;
    float* ml = p.part_ml + (tile * p.S + split) * WS_ROWS * 2;
    float* po = p.part_o + (tile * p.S + split) * WS_ROWS * D;
    if (row_ok) {
#pragma unroll
        for (int i = 0; i < DPO; ++i) po[orow * D + ochunk * DPO + i] = o[i];
    }
    if (row_ok && ochunk == 0) {           // the merge works in log2 units
        ml[2 * orow] = m_s[orow] * kLog2e;
        ml[2 * orow + 1] = l_s[orow];
    }
}

template <int QT, int MODE, int BITS, int D>
hipError_t launch_g(int64_t B, const AttnLaunch& p, hipStream_t stream) {
    dim3 grid(p.S, p.n_rt, (unsigned)(B * p.Hk));
    if (p.n_rows <= 4)   // one tile of at most 4 rows (a decode with G <= 4)
        hipLaunchKernelGGL((attn_generic_kernel<QT, MODE, BITS, D, 4>), grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((attn_generic_kernel<QT, MODE, BITS, D, 16>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int QT, int MODE, int BITS>
hipError_t dispatch_d(int D, int64_t B, const AttnLaunch& p, hipStream_t s) {
    switch (D) {
        case 64: return launch_g<QT, MODE, BITS, 64>(B, p, s);
        case 96: return launch_g<QT, MODE, BITS, 96>(B, p, s);
        case 128: return launch_g<QT, MODE, BITS, 128>(B, p, s);
        case 256: return launch_g<QT, MODE, BITS, 256>(B, p, s);
    }
    return hipErrorNotSupported;
}

template <int QT>
hipError_t dispatch_fmt(int mode, int bits, int D, int64_t B, const AttnLaunch& p,
                        hipStream_t s) {
    if (mode == MODE_Q8_0) return dispatch_d<QT, MODE_Q8_0, 8>(D, B, p, s);
    if (mode == MODE_QSYM) {
        if (bits == 4) return dispatch_d<QT, MODE_QSYM, 4>(D, B, p, s);
        if (bits == 5) return dispatch_d<QT, MODE_QSYM, 5>(D, B, p, s);
        return hipErrorNotSupported;
    }
    if (mode != MODE_AFFINE) return hipErrorNotSupported;
    switch (bits) {
        case 2: return dispatch_d<QT, MODE_AFFINE, 2>(D, B, p, s);
        case 3: return dispatch_d<QT, MODE_AFFINE, 3>(D, B, p, s);
        case 4: return dispatch_d<QT, MODE_AFFINE, 4>(D, B, p, s);
        case 5: return dispatch_d<QT, MODE_AFFINE, 5>(D, B, p, s);
        case 6: return dispatch_d<QT, MODE_AFFINE, 6>(D, B, p, s);
        case 8: return dispatch_d<QT, MODE_AFFINE, 8>(D, B, p, s);
    }
    return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_attn_generic(int q_dtype, int mode, int bits, int D, int64_t B,
                               const AttnLaunch& p, hipStream_t stream) {
    switch (q_dtype) {
        case DT_F32: return dispatch_fmt<DT_F32>(mode, bits, D, B, p, stream);
        case DT_F16: return dispatch_fmt<DT_F16>(mode, bits, D, B, p, stream);
        case DT_BF16: return dispatch_fmt<DT_BF16>(mode, bits, D, B, p, stream);
    }
    return hipErrorNotSupported;
}

}  // namespace qkv
