/*
 * qkv_oracle.c -- plain, slow CPU oracle for attention over a quantized KV
 * cache.  TEST INFRASTRUCTURE ONLY: the product library never links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.
 *
 * It shares no code with the GPU path (its own half/bfloat16 conversions, its
 * own packing, its own attention).  Every function follows the definition on
 * the source pages step by step, with no blocking, fusion or reordering:
 *
 *   [MLX-KVU]  MLX branch page "add fast::quantized_kv_update"
 *              (kernels/quantized.h affine_quantize / kv_update,
 *               kernels/sdpa_vector.h load_keys / load_values /
 *               quant_sdpa_vector, mlx/fast.cpp
 *               quantized_scaled_dot_product_attention fallback)
 *   [MLX-WIP]  MLX CUDA page "Fixed mma and working dequant"
 *              (quantized.cu affine_quantize / affine_dequantize,
 *               qmm.cu SharedTile::load_quantized)
 *   [LLAMA]    llama.cpp PR page "Metal: Optimize q8_0 KV - #25556"
 *              (Q8_0 KV blocks: 32 signed int8 codes, one fp16 scale)
 *
 * Readings taken where the pages are silent:
 *   - codes of a row form one least-significant-bit-first stream (the 2/4/8-bit
 *     layout of the pages, continued through the 3/5/6-bit packs);
 *   - the Q4_0 / Q5_0 caches the llama.cpp page names: the Q8_0 rule with the
 *     code range of 4 / 5 bits (symmetric blocks of 32, one fp16 scale);
 *   - codes are rounded half-to-even from the STORED (dtype-rounded) scale
 *     and bias, with IEEE fp32 subtract and divide, no fused multiply-add;
 *   - the scale is floored at eps = T(1e-7) before it is stored;
 *   - Q8_0: d = fp16(amax / 127), codes from the stored d, zero block -> 0;
 *   - attention: scale applied in high precision (fp64 here), additive mask,
 *     causal = bottom-right aligned, fully masked row -> zeros.
 *
 * Parity pins live in tests/test_oracle_*.py; every function here has one.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* ------------------------------------------------------------------------ */
/* Scalar formats.  IEEE binary16 and bfloat16, written out from the format  */
/* definitions (sign / exponent / fraction), round-to-nearest-even.          */
/* ------------------------------------------------------------------------ */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

float orc_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0x1f) {
        if (m) return NAN;
        v = INFINITY;
    } else if (e == 0) {
        v = ldexp((double)m, -24);            /* subnormal: m * 2^-24 */
    } else {
        v = ldexp((double)(m + 1024), e - 25); /* (1 + m/1024) * 2^(e-15) */
    }
    return (float)(sign ? -v : v);             /* exact in fp32 */
}

/* Round a finite double to the nearest value of the form k * 2^q (k
 * integer), ties to even k.  Used by both narrowing conversions. */
static double round_to_quantum(double a, int q) {
    double k = ldexp(a, -q);                  /* exact: power-of-two scale */
    double fl = floor(k);
    double frac = k - fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    return ldexp(fl, q);
}

uint16_t orc_f32_to_f16(float f) {
    uint32_t u = f32_to_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
    if (isnan(f)) return (uint16_t)(sign | 0x7e00);
    double a = fabs((double)f);
    if (isinf(f)) return (uint16_t)(sign | 0x7c00);
    if (a == 0.0) return sign;
    /* quantum of binary16 at a's binade; subnormal range has quantum 2^-24 */
    int ex;
    frexp(a, &ex);                            /* a in [2^(ex-1), 2^ex) */
    int q = (ex - 1) - 10;
    if (q < -24) q = -24;
    double r = round_to_quantum(a, q);
    if (r >= 65520.0 || r > 65504.0) return (uint16_t)(sign | 0x7c00);
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -14)) {                /* subnormal */
        return (uint16_t)(sign | (uint16_t)ldexp(r, 24));
    }
    frexp(r, &ex);
    int e = ex - 1;                           /* r in [2^e, 2^(e+1)) */
    int m = (int)(ldexp(r, 10 - e) - 1024.0);
    return (uint16_t)(sign | ((e + 15) << 10) | m);
}

float orc_bf16_to_f32(uint16_t h) { return bits_to_f32(((uint32_t)h) << 16); }

uint16_t orc_f32_to_bf16(float f) {
    uint32_t u = f32_to_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
    if (isnan(f)) return (uint16_t)(sign | 0x7fc0);
    if (isinf(f)) return (uint16_t)(sign | 0x7f80);
    double a = fabs((double)f);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);
    int q = (ex - 1) - 7;                     /* 8 significant bits */
    if (q < -133) q = -133;                   /* subnormal quantum 2^-133 */
    double r = round_to_quantum(a, q);
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7f80);
    /* r is exactly representable as fp32 and has <= 8 significant bits, so
     * its fp32 pattern has zero low 16 bits */
    return (uint16_t)(sign | (f32_to_bits((float)r) >> 16));
}

static float load_elem(const void* p, int dtype, int64_t i) {
    if (dtype == ORC_F32) return ((const float*)p)[i];
    if (dtype == ORC_F16) return orc_f16_to_f32(((const uint16_t*)p)[i]);
    return orc_bf16_to_f32(((const uint16_t*)p)[i]);
}

/* Round an fp32 value to dtype and back (the value as stored in dtype). */
static float round_to_dtype(float v, int dtype) {
    if (dtype == ORC_F32) return v;
    if (dtype == ORC_F16) return orc_f16_to_f32(orc_f32_to_f16(v));
    return orc_bf16_to_f32(orc_f32_to_bf16(v));
}

static void store_elem(void* p, int dtype, int64_t i, float v) {
    if (dtype == ORC_F32) ((float*)p)[i] = v;
    else if (dtype == ORC_F16) ((uint16_t*)p)[i] = orc_f32_to_f16(v);
    else ((uint16_t*)p)[i] = orc_f32_to_bf16(v);
}

/* Round half to even on an fp32 value, as an integer (|v| small). */
static long rne_int(float v) {
    double d = (double)v;                     /* exact */
    double fl = floor(d);
    double frac = d - fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    return (long)fl;
}

/* The scale floor eps = T(1e-7) of the affine quantizer, as fp32
 * ([MLX-KVU] quantized.h, affine_quantize: constexpr T eps = T(1e-7)). */
float orc_affine_eps(int scale_dtype) { return round_to_dtype(1e-7f, scale_dtype); }

/* ------------------------------------------------------------------------ */
/* Code packing.  The codes of a row form one little-endian bit stream:      */
/* element j occupies bits [j*bits, (j+1)*bits), least significant bit      */
/* first.  For 2, 4 and 8 bits this is element j at bits                    */
/* [(j mod (32/bits))*bits, +bits) of uint32 word j / (32/bits)             */
/* ([MLX-KVU] sdpa_vector.h load_keys masks 0x000f, 0x00f0, 0x0f00, 0xf000; */
/* [MLX-WIP] qmm.cu load_quantized shifts); for 3, 5 and 6 bits it packs 8,  */
/* 8 and 4 values into 3, 5 and 3 bytes ([MLX-WIP] quantized_utils.cuh     */
/* get_pack_factor / get_bytes_per_pack), their bit order within a pack     */
/* taken to continue the same least-significant-first stream.               */
/* ------------------------------------------------------------------------ */
static void put_code(uint8_t* row, int64_t j, int bits, uint32_t c) {
    for (int k = 0; k < bits; ++k) {
        int64_t bit = j * bits + k;
        if ((c >> k) & 1u) row[bit >> 3] |= (uint8_t)(1u << (bit & 7));
    }
}

static uint32_t get_code(const uint8_t* row, int64_t j, int bits) {
    uint32_t c = 0;
    for (int k = 0; k < bits; ++k) {
        int64_t bit = j * bits + k;
        c |= (uint32_t)((row[bit >> 3] >> (bit & 7)) & 1u) << k;
    }
    return c;
}

/* ------------------------------------------------------------------------ */
/* Group-wise affine quantization ([MLX-KVU] quantized.h affine_quantize;   */
/* [MLX-WIP] quantized.cu affine_quantize).  Per group of gs elements:       */
/*   s = max((max - min) / (2^bits - 1), eps) stored in T, b = min in T,    */
/*   c = clamp(rne((x - b) / s), 0, 2^bits - 1), packed as above.           */
/* x: rows x D in x_dtype.  codes: rows x (D*bits/8) bytes (D*bits/32       */
/* little-endian words).  scales, biases: rows x (D/gs) in scale_dtype.     */
/* ------------------------------------------------------------------------ */
void orc_quantize_affine(const void* x, int x_dtype, int64_t rows, int64_t D,
                         int bits, int gs, int scale_dtype,
                         uint32_t* codes, void* scales, void* biases) {
    const int64_t bytes_per_row = D * bits / 8;
    const int64_t groups = D / gs;
    const float n_levels = (float)((1 << bits) - 1);
    const float eps = orc_affine_eps(scale_dtype);
    float* xs = (float*)malloc(sizeof(float) * (size_t)gs);
    for (int64_t r = 0; r < rows; ++r) {
        uint8_t* crow = (uint8_t*)codes + r * bytes_per_row;
        memset(crow, 0, (size_t)bytes_per_row);
        for (int64_t g = 0; g < groups; ++g) {
            /* 1. widen the group to fp32 (exact for all three dtypes) */
            for (int i = 0; i < gs; ++i) xs[i] = load_elem(x, x_dtype, r * D + g * gs + i);
            /* 2. min / max */
            float mn = xs[0], mx = xs[0];
            for (int i = 1; i < gs; ++i) {
                if (xs[i] < mn) mn = xs[i];
                if (xs[i] > mx) mx = xs[i];
            }
            /* 3-4. scale in fp32, floored at eps */
            float s32 = (mx - mn) / n_levels;
            if (s32 < eps) s32 = eps;
            /* 5. store scale and bias in T; codes use the stored values */
            store_elem(scales, scale_dtype, r * groups + g, s32);
            store_elem(biases, scale_dtype, r * groups + g, mn);
            const float s = round_to_dtype(s32, scale_dtype);
            const float b = round_to_dtype(mn, scale_dtype);
            /* 6-7. codes and packing */
            for (int i = 0; i < gs; ++i) {
                float t = (xs[i] - b) / s;
                long c = rne_int(t);
                if (c < 0) c = 0;
                if (c > (long)n_levels) c = (long)n_levels;
                put_code(crow, g * gs + i, bits, (uint32_t)c);
            }
        }
    }
    free(xs);
}

/* Affine dequantization x^ = s * c + b in fp32 ([MLX-KVU] quantized.h
 * affine_dequantize "scale * d + bias"; sdpa_vector.h load_values).
 * out: rows x D fp32. */
void orc_dequant_affine(const uint32_t* codes, const void* scales, const void* biases,
                        int scale_dtype, int64_t rows, int64_t D, int bits, int gs,
                        float* out) {
    const int64_t bytes_per_row = D * bits / 8;
    const int64_t groups = D / gs;
    for (int64_t r = 0; r < rows; ++r) {
        const uint8_t* crow = (const uint8_t*)codes + r * bytes_per_row;
        for (int64_t j = 0; j < D; ++j) {
            int64_t g = j / gs;
            uint32_t c = get_code(crow, j, bits);
            float s = load_elem(scales, scale_dtype, r * groups + g);
            float b = load_elem(biases, scale_dtype, r * groups + g);
            float prod = s * (float)c;            /* two roundings, no fma */
            out[r * D + j] = prod + b;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Q8_0 blocks ([LLAMA]: a block of 32 signed int8 codes with one fp16      */
/* scale).  d = fp16(amax / 127); c = clamp(rne(x / d), -127, 127), 0 when  */
/* d == 0.  codes: rows x D int8; d: rows x (D/32) fp16 bit patterns.       */
/* ------------------------------------------------------------------------ */
void orc_quantize_q8_0(const void* x, int x_dtype, int64_t rows, int64_t D,
                       int8_t* codes, uint16_t* dscale) {
    const int64_t blocks = D / 32;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < blocks; ++k) {
            float xs[32];
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                xs[i] = load_elem(x, x_dtype, r * D + k * 32 + i);
                float a = fabsf(xs[i]);
                if (a > amax) amax = a;
            }
            float d32 = amax / 127.0f;
            uint16_t dh = orc_f32_to_f16(d32);
            dscale[r * blocks + k] = dh;
            float d = orc_f16_to_f32(dh);
            for (int i = 0; i < 32; ++i) {
                long c = 0;
                if (d != 0.0f) {
                    c = rne_int(xs[i] / d);
                    if (c < -127) c = -127;
                    if (c > 127) c = 127;
                }
                codes[r * D + k * 32 + i] = (int8_t)c;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Symmetric blocks of 32 at b = 4 or 5 bits: the Q8_0 rule with the code    */
/* range of b bits (the reading taken for the Q4_0 / Q5_0 caches that the   */
/* llama.cpp page names): qmax = 2^(b-1) - 1, d = fp16(amax / qmax),        */
/* c = clamp(rne(x / d), -qmax, qmax) (0 when d == 0), stored as b-bit two's */
/* complement in the row's bit stream.  codes: rows x (D*b/8) bytes.        */
/* ------------------------------------------------------------------------ */
void orc_quantize_qsym(const void* x, int x_dtype, int64_t rows, int64_t D, int bits,
                       uint8_t* codes, uint16_t* dscale) {
    const int64_t blocks = D / 32;
    const int64_t bytes_per_row = D * bits / 8;
    const long qmax = (1L << (bits - 1)) - 1;
    for (int64_t r = 0; r < rows; ++r) {
        uint8_t* crow = codes + r * bytes_per_row;
        memset(crow, 0, (size_t)bytes_per_row);
        for (int64_t k = 0; k < blocks; ++k) {
            float xs[32];
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                xs[i] = load_elem(x, x_dtype, r * D + k * 32 + i);
                float a = fabsf(xs[i]);
                if (a > amax) amax = a;
            }
            float d32 = amax / (float)qmax;
            uint16_t dh = orc_f32_to_f16(d32);
            dscale[r * blocks + k] = dh;
            float d = orc_f16_to_f32(dh);
            for (int i = 0; i < 32; ++i) {
                long c = 0;
                if (d != 0.0f) {
                    c = rne_int(xs[i] / d);
                    if (c < -qmax) c = -qmax;
                    if (c > qmax) c = qmax;
                }
                put_code(crow, k * 32 + i, bits, (uint32_t)c & ((1u << bits) - 1u));
            }
        }
    }
}

void orc_dequant_qsym(const uint8_t* codes, const uint16_t* dscale, int64_t rows, int64_t D,
                      int bits, float* out) {
    const int64_t blocks = D / 32;
    const int64_t bytes_per_row = D * bits / 8;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < D; ++j) {
            uint32_t u = get_code(codes + r * bytes_per_row, j, bits);
            long c = (u >> (bits - 1)) ? (long)u - (1L << bits) : (long)u;   /* two's complement */
            out[r * D + j] = orc_f16_to_f32(dscale[r * blocks + j / 32]) * (float)c;
        }
}

/* Q8_0 dequantization x^ = d * c in fp32. */
void orc_dequant_q8_0(const int8_t* codes, const uint16_t* dscale, int64_t rows, int64_t D,
                      float* out) {
    const int64_t blocks = D / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < D; ++j)
            out[r * D + j] = orc_f16_to_f32(dscale[r * blocks + j / 32]) * (float)codes[r * D + j];
}

/* ------------------------------------------------------------------------ */
/* Attention over the dequantized cache ([MLX-KVU] fast.cpp                  */
/* quantized_scaled_dot_product_attention: the fallback composition         */
/* quantized_matmul(q, K, transpose) -> + mask -> softmax -> quantized_matmul */
/* (P, V), GQA by reshaping q to [B, Hk, Hq/Hk, L, D]; sdpa_vector.h         */
/* quant_sdpa_vector: kv head = q head / (Hq/Hk)).                           */
/*   out[b,h,i,:] = sum_j softmax_j(scale * q.K^_j + m_ij) V^_j              */
/* q: [B,Hq,Lq,D] fp32.  khat, vhat: [B,Hk,L,D] fp32 (dequantized values).   */
/* mask: additive, element (b,h,i,j) at b*ms[0]+h*ms[1]+i*ms[2]+j*ms[3]      */
/* (fp32) or NULL; causal != 0 hides key j from query i when                 */
/* j > L - Lq + i (bottom-right aligned).  out: [B,Hq,Lq,D] fp64.            */
/* A row with every key hidden yields zeros.  All accumulation is fp64.      */
/* ------------------------------------------------------------------------ */
void orc_attention(const float* q, const float* khat, const float* vhat,
                   int64_t B, int64_t Hq, int64_t Hk, int64_t Lq, int64_t L, int64_t D,
                   double scale, const float* mask, const int64_t* ms, int causal,
                   double* out) {
    const int64_t G = Hq / Hk;
    const int64_t nrows = B * Hq * Lq;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t row = 0; row < nrows; ++row) {
        const int64_t i = row % Lq;
        const int64_t h = (row / Lq) % Hq;
        const int64_t b = row / (Lq * Hq);
        const int64_t kh = h / G;
        const float* qr = q + row * D;
        const float* K = khat + (b * Hk + kh) * L * D;
        const float* V = vhat + (b * Hk + kh) * L * D;
        double* o = out + row * D;
        double* z = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        int* vis = (int*)malloc(sizeof(int) * (size_t)(L > 0 ? L : 1));
        double M = -INFINITY;
        for (int64_t j = 0; j < L; ++j) {
            vis[j] = !(causal && j > L - Lq + i);
            if (!vis[j]) { z[j] = -INFINITY; continue; }
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += (double)qr[d] * (double)K[j * D + d];
            z[j] = scale * dot;
            if (mask) z[j] += (double)mask[b * ms[0] + h * ms[1] + i * ms[2] + j * ms[3]];
            if (z[j] == -INFINITY) vis[j] = 0;
            if (vis[j] && z[j] > M) M = z[j];
        }
        for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
        if (M != -INFINITY) {
            double Z = 0.0;
            for (int64_t j = 0; j < L; ++j) {
                if (!vis[j]) continue;
                double w = exp(z[j] - M);
                Z += w;
                for (int64_t d = 0; d < D; ++d) o[d] += w * (double)V[j * D + d];
            }
            for (int64_t d = 0; d < D; ++d) o[d] /= Z;
        }
        free(z);
        free(vis);
    }
}

int orc_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
