// Unfused attention for one query per head over a quantized KV cache: the
// composition that the MLX page "add fast::quantized_kv_update" gives as the
// fallback of quantized_scaled_dot_product_attention (mlx/fast.cpp: a
// quantized matmul of q against K transposed, plus the mask, a softmax over
// the keys, a quantized matmul of the probabilities with V, query heads
// grouped onto their kv head by a reshape) and that its benchmark
// (sdpa_vector_bench.py, quant_attention) times against the fused kernel.
// Five kernels, each its own pass over memory, so that the fused kernels can
// be measured against it:
//
//   1. unfused_scores_kernel   z[b,h,j] = (scale q[b,h] . K^[b,kvh,j] + mask) log2 e
//      The quantized matrix-vector product (qmv on the MLX 1.0.0 Metal host
//      page): the G query heads of a kv head share every K load.  A row of
//      packed codes is cut into 8-byte slices (4-byte for 16 heads of 4-bit
//      codes), one per lane; the lane keeps the G heads' q values of its
//      slice in registers, so a score is the sum over slices of
//      s_g (q . c) + b_g (sum q), reduced across the row's lanes.
//   2. unfused_softmax_stats_kernel, unfused_softmax_norm_kernel
//      P = 2^(z - max) / sum 2^(z - max), in place: per (row, chunk of keys)
//      the chunk's maximum and sum, then from the row's chunk statistics the
//      probabilities of each chunk (a row with no visible key gives P = 0).
//   3. unfused_pv_kernel       partial[c][b,h,:] = sum_{j in chunk c} P[b,h,j] V^[b,kvh,j,:]
//      The quantized vector-matrix product split over key chunks
//      (qvm_split_k on the MLX 1.0.0 Metal host page): a lane owns 8
//      consecutive d of a key row (inside one quantization group), keeps the
//      G heads' sums of p s c for them and of p b per head, and the waves of
//      a workgroup add their sums in a fixed order.
//   4. unfused_reduce_kernel   out[b,h,:] = sum_c partial[c][b,h,:] in the q dtype.
//
// Workspace: scores [B*Hq][L] fp32, softmax chunk statistics [B*Hq][L/4096]
// (m, l) fp32, then partial [chunks][B*Hq][D] fp32 (each 256-byte aligned).
#include "qkv_device.hpp"
#include "qkv_internal.hpp"

namespace qkv {

namespace {

constexpr int NTHR = 256;
constexpr int kScorePasses = 4;        // keys per lane in the scores kernel
constexpr int kPvSteps = 4;            // key steps whose loads the P V kernel issues together
constexpr int kPvWorkgroups = 256;     // P V chunks are made small enough for this many workgroups

// Codes of element e of a slice of packed words: affine unsigned, Q8_0 signed.
template <int MODE, int BITS>
__device__ __forceinline__ float code_at(const uint32_t* w, int e) {
    if constexpr (MODE == MODE_Q8_0) {
        return (float)(int8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xFFu);
    } else {
        return (float)((w[(e * BITS) >> 5] >> ((e * BITS) & 31)) & ((1u << BITS) - 1u));
    }
}

template <int ST>
__device__ __forceinline__ float load_scale(const void* p, int64_t i) {
    return load_as_f32<ST>(p, i);
}

// -------------------------------------------------------------------- scores
// Bytes of a row slice per lane in the scores kernel: 8, or 4 when the G
// heads' q values of an 8-byte slice would take more than 128 registers.
template <int BITS, int GMAX>
constexpr int scores_slice_bytes() { return GMAX * (64 / BITS) > 128 ? 4 : 8; }

// grid (ceil(L / KPW), Hk, B), 256 threads.  Lane t of a pass: key t / LPK of
// the pass, slice t % LPK of its row; NP passes per workgroup.
template <int QT, int MODE, int BITS, int D, int GMAX>
__global__ __launch_bounds__(NTHR) void unfused_scores_kernel(AttnLaunch p) {
    constexpr int ST = (MODE == MODE_Q8_0) ? DT_F16 : QT;
    constexpr int ROWB = D * BITS / 8;
    constexpr int SB = scores_slice_bytes<BITS, GMAX>();
    constexpr int NSW = SB / 4;                    // words per slice
    constexpr int CPL = SB * 8 / BITS;             // codes per slice
    constexpr int LPK = ROWB / SB;                 // lanes per key row
    static_assert(LPK >= 1 && LPK <= 64 && (LPK & (LPK - 1)) == 0, "whole rows per wave");
    constexpr int KPP = NTHR / LPK;                // keys per pass
    constexpr int NP = kScorePasses;               // passes per workgroup
    constexpr int KPW = KPP * NP;

    const int tid = threadIdx.x;
    const int slice = tid % LPK;
    const int64_t kvh = blockIdx.y, b = blockIdx.z;
    const int G = p.G;
    const int NGr = D >> p.gs_log2;
    const int grp = (slice * CPL) >> p.gs_log2;
    const int64_t krow0 = b * p.k.sb + kvh * p.k.sh;
    const int64_t jw = (int64_t)blockIdx.x * KPW;

    // the lane's packed slices of its NP keys, issued first
    uint32_t w[NP][NSW];
    float s[NP], bi[NP];
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
        const int64_t j = min(jw + pp * KPP + tid / LPK, p.L - 1);
        const int64_t r = krow0 + j * p.k.sl;
        const uint8_t* src = (const uint8_t*)p.k.codes + r * ROWB + slice * SB;
        if constexpr (NSW == 1) {
            w[pp][0] = *(const uint32_t*)src;
        } else {
            const uint2 x = *(const uint2*)src;
            w[pp][0] = x.x;
            w[pp][1] = x.y;
        }
        s[pp] = load_scale<ST>(p.k.scales, r * NGr + grp);
        bi[pp] = MODE == MODE_Q8_0 ? 0.0f : load_scale<ST>(p.k.biases, r * NGr + grp);
    }
    // q of the G heads (rows of the kv head) through LDS, then the slice's
    // values and their sums into registers
    __shared__ float qs[GMAX * D];
    for (int i = tid; i < GMAX * D; i += NTHR) {
        const int h = i / D, d = i % D;
        qs[i] = h < G ? load_as_f32<QT>(p.q, (b * p.Hq + kvh * G + h) * D + d) : 0.0f;
    }
    __syncthreads();
    float q[GMAX][CPL], qsum[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        qsum[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            q[h][e] = qs[h * D + slice * CPL + e];
            qsum[h] += q[h][e];
        }
    }
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
        const int64_t j = jw + pp * KPP + tid / LPK;
        float acc[GMAX];
#pragma unroll
        for (int h = 0; h < GMAX; ++h) acc[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            const float c = code_at<MODE, BITS>(w[pp], e);
#pragma unroll
            for (int h = 0; h < GMAX; ++h) acc[h] += q[h][e] * c;
        }
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            float z = s[pp] * acc[h] + bi[pp] * qsum[h];
#pragma unroll
            for (int o = 1; o < LPK; o <<= 1) z += __shfl_xor(z, o, 64);
            acc[h] = z;
        }
        if (slice == 0 && j < p.L) {
#pragma unroll
            for (int h = 0; h < GMAX; ++h) {
                if (h < G) {
                    const int64_t hq = kvh * G + h;
                    float z = acc[h] * p.scale;
                    if (p.mask_kind == MASK_ADDITIVE)
                        z += load_mask(p.mask, p.mask_dtype, b * p.ms0 + hq * p.ms1 + j * p.ms3);
                    p.un_scores[(b * p.Hq + hq) * p.L + j] = z * kLog2e;
                }
            }
        }
    }
}

// -------------------------------------------------------------------- softmax
// Two passes over the score rows, each spread over every (row, chunk of
// SMC keys): the chunk's maximum and sum of 2^(z - max), then the row's
// maximum and sum from its chunks' and the probabilities of the chunk.
constexpr int SMC = 4096;

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < NTHR / 64; ++i) r = fmaxf(r, red[i]);
    return r;
}
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < NTHR / 64; ++i) r += red[i];
    return r;
}

// grid (chunks, B * Hq): (max, sum 2^(z - max)) of the chunk -> un_stats.
__global__ __launch_bounds__(NTHR) void unfused_softmax_stats_kernel(AttnLaunch p) {
    __shared__ float red[NTHR / 64];
    const int64_t row = blockIdx.y;
    const int64_t j0 = (int64_t)blockIdx.x * SMC;
    const int64_t j1 = min(p.L, j0 + SMC);
    const float* z = p.un_scores + row * p.L;
    float v[SMC / NTHR];
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < SMC / NTHR; ++u) {
        const int64_t j = j0 + threadIdx.x + u * NTHR;
        v[u] = j < j1 ? z[j] : -INFINITY;
        m = fmaxf(m, v[u]);
    }
    m = block_max(m, red);
    float l = 0.0f;
    if (m != -INFINITY) {
#pragma unroll
        for (int u = 0; u < SMC / NTHR; ++u) l += fast_exp2(v[u] - m);
    }
    l = block_sum(l, red);
    if (threadIdx.x == 0) {
        const int64_t si = row * gridDim.x + blockIdx.x;
        p.un_stats[2 * si] = m;
        p.un_stats[2 * si + 1] = l;
    }
}

// grid (chunks, B * Hq): the row's maximum and sum from its chunks (in chunk
// order), then P = 2^(z - max) / sum for the chunk, in place.
__global__ __launch_bounds__(NTHR) void unfused_softmax_norm_kernel(AttnLaunch p) {
    __shared__ float red[NTHR / 64];
    const int64_t row = blockIdx.y;
    const int nc = gridDim.x;
    const float* st = p.un_stats + 2 * row * nc;
    float m = -INFINITY;
    for (int c = threadIdx.x; c < nc; c += NTHR) m = fmaxf(m, st[2 * c]);
    m = block_max(m, red);
    float l = 0.0f;
    if (m != -INFINITY)
        for (int c = threadIdx.x; c < nc; c += NTHR)
            if (st[2 * c] != -INFINITY) l += st[2 * c + 1] * fast_exp2(st[2 * c] - m);
    l = block_sum(l, red);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* z = p.un_scores + row * p.L;
    const int64_t j0 = (int64_t)blockIdx.x * SMC;
    const int64_t j1 = min(p.L, j0 + SMC);
    for (int64_t j = j0 + threadIdx.x; j < j1; j += NTHR)
        z[j] = m == -INFINITY ? 0.0f : fast_exp2(z[j] - m) * inv;
}

// -------------------------------------------------------------------- P V
// grid (chunks, Hk, B), 256 threads.  Lane t of a wave: key t / LPR of the
// wave's KPI keys, d = 8 (t % LPR) .. + 8.  The probabilities of the chunk's
// keys sit in LDS.
template <int QT, int MODE, int BITS, int D, int GMAX>
__global__ __launch_bounds__(NTHR) void unfused_pv_kernel(AttnLaunch p) {
    constexpr int ST = (MODE == MODE_Q8_0) ? DT_F16 : QT;
    constexpr int ROWB = D * BITS / 8;
    constexpr int LPR = D / 8;                     // lanes per row
    constexpr int KPI = 64 / LPR;                  // keys per wave and step
    constexpr int KPS = 4 * KPI;                   // keys per workgroup and step
    constexpr int WB = BITS;                       // bytes of 8 codes
    constexpr int NW = WB >= 4 ? WB / 4 : 1;
    constexpr int PCAP = 16 * 256;                 // LDS floats: P chunk, then the o sums
    static_assert(GMAX * D <= PCAP, "LDS holds the G x D sums");
    __shared__ float lds[PCAP];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int64_t kvh = blockIdx.y, b = blockIdx.z;
    const int G = p.G;
    const int CK = (int)p.un_chunk;
    const int64_t j0 = (int64_t)blockIdx.x * CK;
    const int nk = (int)min((int64_t)CK, p.L - j0);
    const int NGr = D >> p.gs_log2;
    const int dsl = lane % LPR;
    const int grp = (dsl * 8) >> p.gs_log2;
    const int64_t vrow0 = b * p.v.sb + kvh * p.v.sh;

    // probabilities of the chunk: lds[h * CK + k]
    for (int i = tid; i < G * CK; i += NTHR) {
        const int h = i / CK, k = i % CK;
        lds[i] = k < nk ? p.un_scores[(b * p.Hq + kvh * G + h) * p.L + j0 + k] : 0.0f;
    }
    __syncthreads();

    float o[GMAX][8], ob[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        ob[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.0f;
    }
    constexpr int U = kPvSteps;
    for (int k0 = 0; k0 < nk; k0 += U * KPS) {
        uint32_t cw[U][NW];
        float vs[U], vb[U];
        int kk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            kk[u] = k0 + u * KPS + wave * KPI + lane / LPR;
            const int64_t j = j0 + min(kk[u], nk - 1);
            const int64_t r = vrow0 + j * p.v.sl;
            const uint8_t* src = (const uint8_t*)p.v.codes + r * ROWB + dsl * WB;
            if constexpr (NW == 1) cw[u][0] = *(const uint32_t*)src;
            else { const uint2 x = *(const uint2*)src; cw[u][0] = x.x; cw[u][1] = x.y; }
            vs[u] = load_scale<ST>(p.v.scales, r * NGr + grp);
            vb[u] = MODE == MODE_Q8_0 ? 0.0f : load_scale<ST>(p.v.biases, r * NGr + grp);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (kk[u] >= nk) continue;
            float c[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) c[e] = code_at<MODE, BITS>(cw[u], e);
#pragma unroll
            for (int h = 0; h < GMAX; ++h) {
                // heads past G contribute nothing
                const float pr = h < G ? lds[h * CK + kk[u]] : 0.0f;
                const float ps = pr * vs[u];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[h][e] += ps * c[e];
                ob[h] += pr * vb[u];
            }
        }
    }
    // the lanes of one d slice in a wave (KPI keys apart) add up
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = o[h][e] + ob[h];
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
            o[h][e] = x;
        }
    }
    // the four waves add up in wave order through LDS: lds[h * D + d]
    __syncthreads();
    for (int wv = 0; wv < 4; ++wv) {
        if (wave == wv && lane < LPR) {
#pragma unroll
            for (int h = 0; h < GMAX; ++h) {
                if (h < G) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float* dst = &lds[h * D + dsl * 8 + e];
                        *dst = wv == 0 ? o[h][e] : *dst + o[h][e];
                    }
                }
            }
        }
        __syncthreads();
    }
    const int64_t rows = (int64_t)gridDim.z * p.Hq;
    float* part = p.un_partial + ((int64_t)blockIdx.x * rows + b * p.Hq + kvh * G) * D;
    for (int i = tid; i < G * D; i += NTHR) part[i] = lds[i];
}

// -------------------------------------------------------------------- reduce
// grid (ceil(B Hq D / 256)): out = sum over chunks of the partial sums.
template <int QT>
__global__ __launch_bounds__(NTHR) void unfused_reduce_kernel(AttnLaunch p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * NTHR + threadIdx.x;
    if (i >= n) return;
    const int C = p.un_chunks;
    constexpr int U = 8;
    float acc = 0.0f;
    int c = 0;
    for (; c + U <= C; c += U) {
        float x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = p.un_partial[(int64_t)(c + u) * n + i];
#pragma unroll
        for (int u = 0; u < U; ++u) acc += x[u];
    }
    for (; c < C; ++c) acc += p.un_partial[(int64_t)c * n + i];
    store_from_f32<QT>(p.out, i, acc);
}

template <int QT, int MODE, int BITS, int D, int GMAX>
hipError_t launch_all(int64_t B, const AttnLaunch& p, hipStream_t s) {
    constexpr int ROWB = D * BITS / 8;
    constexpr int KPW = NTHR / (ROWB / scores_slice_bytes<BITS, GMAX>()) * kScorePasses;
    if ((int64_t)GMAX * p.un_chunk > 16 * 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL((unfused_scores_kernel<QT, MODE, BITS, D, GMAX>),
                       dim3((unsigned)((p.L + KPW - 1) / KPW), (unsigned)p.Hk, (unsigned)B), dim3(NTHR), 0, s, p);
    const dim3 sm((unsigned)((p.L + SMC - 1) / SMC), (unsigned)(B * p.Hq));
    hipLaunchKernelGGL(unfused_softmax_stats_kernel, sm, dim3(NTHR), 0, s, p);
    hipLaunchKernelGGL(unfused_softmax_norm_kernel, sm, dim3(NTHR), 0, s, p);
    hipLaunchKernelGGL((unfused_pv_kernel<QT, MODE, BITS, D, GMAX>),
                       dim3((unsigned)p.un_chunks, (unsigned)p.Hk, (unsigned)B), dim3(NTHR), 0, s, p);
    const int64_t n = B * p.Hq * D;
    hipLaunchKernelGGL((unfused_reduce_kernel<QT>), dim3((unsigned)((n + NTHR - 1) / NTHR)), dim3(NTHR), 0, s, p, n);
    return hipGetLastError();
}

template <int QT, int MODE, int BITS, int D>
hipError_t dispatch_g(int64_t B, const AttnLaunch& p, hipStream_t s) {
    if (p.G <= 1) return launch_all<QT, MODE, BITS, D, 1>(B, p, s);
    if (p.G <= 2) return launch_all<QT, MODE, BITS, D, 2>(B, p, s);
    if (p.G <= 4) return launch_all<QT, MODE, BITS, D, 4>(B, p, s);
    if (p.G <= 8) return launch_all<QT, MODE, BITS, D, 8>(B, p, s);
    if (p.G <= 16) return launch_all<QT, MODE, BITS, D, 16>(B, p, s);
    return hipErrorNotSupported;
}

template <int QT, int MODE, int BITS>
hipError_t dispatch_d(int D, int64_t B, const AttnLaunch& p, hipStream_t s) {
    switch (D) {
        case 64: return dispatch_g<QT, MODE, BITS, 64>(B, p, s);
        case 128: return dispatch_g<QT, MODE, BITS, 128>(B, p, s);
        case 256: return dispatch_g<QT, MODE, BITS, 256>(B, p, s);
    }
    return hipErrorNotSupported;
}

template <int QT>
hipError_t dispatch_fmt(int mode, int bits, int D, int64_t B, const AttnLaunch& p, hipStream_t s) {
    if (mode == MODE_Q8_0) return dispatch_d<QT, MODE_Q8_0, 8>(D, B, p, s);
    if (bits == 4) return dispatch_d<QT, MODE_AFFINE, 4>(D, B, p, s);
    if (bits == 8) return dispatch_d<QT, MODE_AFFINE, 8>(D, B, p, s);
    return hipErrorNotSupported;
}

}  // namespace

int64_t unfused_stats_floats(int64_t B, int64_t Hq, int64_t L) { return 2 * B * Hq * ((L + SMC - 1) / SMC); }

int unfused_chunk_keys(int64_t B, int64_t Hk, int64_t L, int G) {
    int gp = 1;
    while (gp < G) gp *= 2;
    int ck = 1024;
    while (ck > 64 && (ck * gp > 16 * 256 || ((L + ck - 1) / ck) * B * Hk < kPvWorkgroups)) ck /= 2;
    return ck;
}

hipError_t launch_attn_unfused(int q_dtype, int mode, int bits, int D, int64_t B, const AttnLaunch& p,
                               hipStream_t stream) {
    switch (q_dtype) {
        case DT_F32: return dispatch_fmt<DT_F32>(mode, bits, D, B, p, stream);
        case DT_F16: return dispatch_fmt<DT_F16>(mode, bits, D, B, p, stream);
        case DT_BF16: return dispatch_fmt<DT_BF16>(mode, bits, D, B, p, stream);
    }
    return hipErrorNotSupported;
}

}  // namespace qkv
