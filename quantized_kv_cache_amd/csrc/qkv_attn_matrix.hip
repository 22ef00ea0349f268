// Matrix-core decode for fp16 queries on gfx950: scaled-dot-product attention
// of one query per head over a group-quantized KV cache, with both
// contractions (q K^T and P V) on v_mfma_f32_16x16x32_f16.
//
// What is computed follows the MLX page "add fast::quantized_kv_update"
// (sdpa_vector.h quant_sdpa_vector: scores from packed codes through the
// per-group factorisation  q . (s c + b) = s (q . c) + b (sum q), online
// softmax, merge of partial softmax states) and the llama.cpp page "Metal:
// Optimize q8_0 KV - #25556" (Q8_0 blocks; the query heads of a GQA group
// share every K/V load).  The kernel design is MI355X-specific:
//
//  * One workgroup (8 waves) per (key split, batch x kv head) streams its
//    chunk of packed K/V exactly once; the G query heads of the kv head are
//    the 16 rows of the matrix tiles (rows >= G are zero); each wave reads
//    the query values of its lanes itself, so no wave waits for another
//    before its first tile.  Each wave takes every 8th tile of 32 keys.
//  * A wave's K tile goes straight into LDS (buffer_load ... lds) with loads
//    that read whole key rows, into rows whose 16-byte chunks are
//    XOR-swizzled so that the 16 rows of one fragment read start on distinct
//    banks; the MFMA fragments are read back from there.  Loads that spread
//    one instruction over 16 key rows were measured far slower.  V codes and
//    the scales go to registers.
//  * q K^T: A = queries [16 heads x 32 d], B = key codes [32 d x 16 keys].
//    Folded form (affine caches with G * groups <= 16): codes enter the
//    matrix core unconverted: masking a packed word leaves fp16 subnormals
//    c * 2^-24 (4-bit: the odd nibble of a byte becomes 16 c * 2^-24,
//    compensated by a query pre-divided by 16).  Each K-step of 32 d lies in
//    one quantization group, so every group has its own accumulator and the
//    per-key scale/bias are applied afterwards in fp32:
//    z = sum_g s_g * 2^24 * acc_g + b_g * sum_{d in g} q_d.  Otherwise (Q8_0,
//    wide groups) the key codes are dequantized to fp16 before the matrix
//    core and one accumulator covers all groups.
//  * The 16x16 score tiles go through a per-wave LDS scratch to the layout
//    of the P operand: each lane owns one head and 8 keys, so the running
//    max, the rescale of its accumulators and exp2 are lane-local (the 4
//    lanes of a head agree after two xor-shuffles).  Rescales happen only
//    when a tile raises the running max.
//  * P V, folded form (affine caches with G * groups <= 16): the value codes
//    also enter as fp16 subnormals; the value scale moves into the P operand,
//    whose 16 columns are (head, group) pairs: P'[key][(h, g)] = p_h s_g, so
//    o[h][d] = 2^24 sum_key P'[key][(h, g(d))] c[key][d] + sum_key p_h b_g.
//    Only the (h, group of d) column of each output row is kept.
//  * P V, dequantized form (Q8_0 and wide groups): A = V^ [16 d x 32 keys]
//    (fp16, rounded once by v_pk_fma_f16 / v_pk_mul_f16), B = P [32 keys x
//    16 heads].
//  * The waves merge their softmax states through LDS; with several splits
//    the workgroup writes (m, l, o) to the workspace for the split merge
//    kernel that runs next on the stream.
//  * Every cache access is a raw buffer load: a per-tile buffer resource in
//    SGPRs, bounded at the split's last key (rows past it read as zeros), and
//    a loop-invariant 32-bit lane offset, so the load path costs no vector
//    address arithmetic and needs no clamping.  Each wave keeps one tile in
//    flight and issues the next tile's loads as soon as it is consumed.
#include "qkv_device.hpp"
#include "qkv_internal.hpp"
#include "qkv_merge.hpp"
#include "qkv_mfma.hpp"
#include "qkv_quant_math.hpp"

namespace qkv {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int TK = 32;          // keys per tile
constexpr int NWAVE = 8;
constexpr int NTHR = NWAVE * 64;
constexpr int SROW = 36;        // LDS score row stride (floats)

__device__ __forceinline__ uint32_t perm_b(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}
__device__ __forceinline__ h8 to_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    u4 v = {a, b, c, d};
    return __builtin_bit_cast(h8, v);
}
__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u(h2 h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ float lo_f16(uint32_t u) { return f16_to_f32((uint16_t)(u & 0xffffu)); }
__device__ __forceinline__ float hi_f16(uint32_t u) { return f16_to_f32((uint16_t)(u >> 16)); }

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Format traits -------------------------------------------------------------
template <int MODE, int BITS, int GS, int D>
struct Fmt {
    static constexpr int NG = D / GS;                 // groups per row
    static constexpr int ROWB = D * BITS / 8;         // code bytes per row
    static constexpr int STEPS = D / 32;              // K-steps of q K^T
    static constexpr int SPG = GS / 32;               // K-steps per group
    static constexpr int KCH = GS / 4 * BITS / 8;     // bytes per lane per group (q K^T)
    static constexpr int KW = KCH >= 4 ? KCH / 4 : 1;
    static constexpr int VCODES = D / 16;             // codes per lane per key (P V)
    static constexpr int VBYTES = VCODES * BITS / 8;
    static constexpr int VW = VBYTES >= 4 ? VBYTES / 4 : 1;
    static constexpr int SROWB = NG * 2;              // bytes of one row's scales
    static constexpr int NSW = NG >= 2 ? NG / 2 : 1;  // dwords holding one row's scales
};

// Query half order inside one 8-code K-step chunk of a lane, matching the
// halves produced by unpack_k (position e of the 8 consecutive d values).
template <int BITS>
__device__ __forceinline__ int qpos(int h) {
    if constexpr (BITS == 4) {
        constexpr int p[8] = {0, 4, 1, 5, 2, 6, 3, 7};
        return p[h];
    } else {
        constexpr int p[8] = {0, 2, 1, 3, 4, 6, 5, 7};
        return p[h];
    }
}

// 8 codes of one key (one K-step chunk) -> B operand halves (fp16 subnormals).
template <int MODE, int BITS>
__device__ __forceinline__ h8 unpack_k(const uint32_t* w) {
    if constexpr (BITS == 4) {
        const uint32_t x = w[0];
        const uint32_t t = perm_b(0u, x, 0x0C030C01u);           // bytes 1, 3 -> halves
        return to_h8(x & 0x000F000Fu, x & 0x00F000F0u, t & 0x000F000Fu, t & 0x00F000F0u);
    } else {
        const uint32_t f = (MODE == MODE_Q8_0) ? 0x00800080u : 0u;
        const uint32_t a0 = (w[0] & 0x00FF00FFu) ^ f;
        const uint32_t a1 = perm_b(0u, w[0], 0x0C030C01u) ^ f;
        const uint32_t a2 = (w[1] & 0x00FF00FFu) ^ f;
        const uint32_t a3 = perm_b(0u, w[1], 0x0C030C01u) ^ f;
        return to_h8(a0, a1, a2, a3);
    }
}

// 8 codes of one key (one K-step chunk) -> B operand halves dequantized to
// fp16, in unpack_k's half order: Q8_0 d c, affine s c + b (s2, b2: the
// group's scale and bias in both halves).
template <int MODE, int BITS>
__device__ __forceinline__ h8 dequant_k(const uint32_t* w, uint32_t s2, uint32_t b2) {
    uint32_t a[4];
    if constexpr (BITS == 4) {
        const uint32_t x = w[0];
        const uint32_t t = perm_b(0u, x, 0x0C030C01u);           // bytes 1, 3 -> halves
        a[0] = x & 0x000F000Fu;
        a[1] = (x >> 4) & 0x000F000Fu;
        a[2] = t & 0x000F000Fu;
        a[3] = (t >> 4) & 0x000F000Fu;
    } else {
        a[0] = w[0] & 0x00FF00FFu;
        a[1] = perm_b(0u, w[0], 0x0C030C01u);
        a[2] = w[1] & 0x00FF00FFu;
        a[3] = perm_b(0u, w[1], 0x0C030C01u);
    }
    const h2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    const h2 k1152 = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (MODE == MODE_Q8_0) {
            // byte c (two's complement) -> half 1024 + (c + 128) -> c, times d
            a[i] = as_u((as_h2(a[i] ^ 0x64806480u) - k1152) * as_h2(s2));
        } else {
            a[i] = as_u(__builtin_elementwise_fma(as_h2(a[i] | 0x64006400u) - k1024, as_h2(s2), as_h2(b2)));
        }
    }
    return to_h8(a[0], a[1], a[2], a[3]);
}

// Byte 'byte' of the chunks of two keys -> [key a byte, 0, key b byte, 0].
__device__ __forceinline__ uint32_t pair_bytes(const uint32_t* wa, const uint32_t* wb, int byte) {
    const uint32_t sel = (uint32_t)(byte & 3) | 0x0C00u | ((uint32_t)(4 + (byte & 3)) << 16) |
                         0x0C000000u;
    return perm_b(wb[byte >> 2], wa[byte >> 2], sel);
}

// Code t of the lane's chunk for a pair of keys, as fp16 subnormal halves
// (4-bit odd codes arrive as 16 c).
template <int BITS>
__device__ __forceinline__ uint32_t pair_sub(const uint32_t* wa, const uint32_t* wb, int t) {
    if constexpr (BITS == 4) {
        const uint32_t x = pair_bytes(wa, wb, t >> 1);
        return (t & 1) ? (x & 0x00F000F0u) : (x & 0x000F000Fu);
    } else {
        return pair_bytes(wa, wb, t);
    }
}

// Code t for a pair of keys as (1024 + c) halves (dequantized form).
template <int MODE, int BITS>
__device__ __forceinline__ uint32_t pair_int(const uint32_t* wa, const uint32_t* wb, int t) {
    if constexpr (BITS == 4) {
        return pair_sub<4>(wa, wb, t) | 0x64006400u;
    } else {
        const uint32_t x = pair_bytes(wa, wb, t);              // upper bytes are zero
        return MODE == MODE_Q8_0 ? x ^ 0x64806480u : x | 0x64006400u;
    }
}

// Compiler-only ordering of the per-wave LDS scratch: LDS instructions of one
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

template <int MODE, int BITS, int GS, int D, bool MASK, bool FOLD, bool APPEND = false>
__global__ __launch_bounds__(NTHR) void attn_matrix_decode(AttnLaunch p) {
    using F = Fmt<MODE, BITS, GS, D>;
    constexpr int NG = F::NG;
    constexpr int STEPS = F::STEPS;
    constexpr int NT = D / 16;                    // P V tiles (16 d each)
    constexpr int KW = F::KW;
    constexpr int VW = F::VW;
    constexpr int NSW = F::NSW;
    static_assert(!FOLD || (MODE == MODE_AFFINE && NG <= 2), "folded P V needs <= 2 groups");

    // Per-wave LDS: the score scratch of its tiles while it streams, then its
    // output state for the workgroup merge (written only after its last tile;
    // no other wave touches its scratch).
    // K tiles are staged in LDS (after the score scratch): TK key rows of
    // ROWB bytes, 16-byte chunks XOR-swizzled per row (kswz), filled by
    // direct-to-LDS loads that read whole rows (KPI rows per instruction).
    constexpr int ROWB = F::ROWB;
    constexpr int NCH = ROWB / 16;                // 16-byte chunks per key row
    constexpr int KPI = 1024 / ROWB;              // key rows per load instruction
    constexpr int NKI = TK / KPI;                 // K load instructions per tile
    constexpr int KSTAGE = 16 * SROW;             // float offset of the K stage in a wave's region
    constexpr int WAVE_FLOATS = 64 * (D / 4) > KSTAGE + TK * ROWB / 4 ? 64 * (D / 4) : KSTAGE + TK * ROWB / 4;
    static_assert(NCH >= 2 && NCH <= 16 && TK % KPI == 0, "K stage layout");
    __shared__ __attribute__((aligned(16))) float s_wave[NWAVE][WAVE_FLOATS];
    __shared__ float s_ml[NWAVE][2][16];
    __shared__ float s_bias[NWAVE][16][2];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lane = tid & 63;
    const int n = lane & 15;          // A/B row or column index
    const int kb = lane >> 4;         // K-block of the lane (0..3)
    // grid: x = key split, y = kv head, z = batch
    const int split = blockIdx.x;
    const int64_t kvh = blockIdx.y;
    const int64_t b = blockIdx.z;
    pin_sgpr(p.q); pin_sgpr(p.Hq); pin_sgpr(p.Hk); pin_sgpr(p.G); pin_sgpr(p.L);
    pin_sgpr(p.chunk); pin_sgpr(p.scale);
    pin_sgpr(p.k.codes); pin_sgpr(p.k.scales); pin_sgpr(p.k.biases);
    pin_sgpr(p.k.sb); pin_sgpr(p.k.sh); pin_sgpr(p.k.sl);
    pin_sgpr(p.v.codes); pin_sgpr(p.v.scales); pin_sgpr(p.v.biases);
    pin_sgpr(p.v.sb); pin_sgpr(p.v.sh); pin_sgpr(p.v.sl);
    const int64_t bk = b * p.Hk + kvh;
    const int G = p.G;
    const float sl = p.scale * kLog2e;            // scores kept in log2 units

    // ---------------------------------------------------------------- key range
    const int64_t j0 = (int64_t)split * p.chunk;
    const int64_t j1 = min(p.L, j0 + p.chunk);
    const int ntiles = (int)((j1 - j0 + TK - 1) / TK);

    // Every K/V access is a raw buffer load: a per-tile buffer resource (base at
    // the tile's first row, in SGPRs) and a loop-invariant per-lane byte offset.
    // The resource's size stops at the split's last key, so rows past it read
    // as zeros (they are masked) and tiles need no clamping.
    const int64_t krow0 = b * p.k.sb + kvh * p.k.sh;
    const int64_t vrow0 = b * p.v.sb + kvh * p.v.sh;
    const uint8_t* kc = (const uint8_t*)p.k.codes + krow0 * F::ROWB;
    const uint8_t* vc = (const uint8_t*)p.v.codes + vrow0 * F::ROWB;
    const uint8_t* ksc = (const uint8_t*)p.k.scales + krow0 * F::SROWB;
    const uint8_t* kbi = (const uint8_t*)p.k.biases + krow0 * F::SROWB;
    const uint8_t* vsc = (const uint8_t*)p.v.scales + vrow0 * F::SROWB;
    const uint8_t* vbi = (const uint8_t*)p.v.biases + vrow0 * F::SROWB;
    const uint32_t kcs = (uint32_t)(p.k.sl * F::ROWB);      // byte strides of one key
    const uint32_t vcs = (uint32_t)(p.v.sl * F::ROWB);
    const uint32_t kss = (uint32_t)(p.k.sl * F::SROWB);
    const uint32_t vss = (uint32_t)(p.v.sl * F::SROWB);
    const uint32_t jmax = (uint32_t)(j1 - 1);

    // folded P V: this lane's P' column is (head ch, group cg)
    const int ch = FOLD ? n % G : n;
    const int cg = FOLD ? n / G : 0;
    const bool cvalid = FOLD ? (n < G * NG) : true;
    const int vg = (F::VCODES * n) / GS;          // group of the lane's dequantized P V chunk

    // Registers of one tile.  Only loads write them; every use waits in
    // process().
    // Folded tiles load the scale and bias rows of the tile's 32 keys
    // cooperatively (lane l: key l % 32) and lanes fetch the rows they need
    // with cross-lane shuffles.
    constexpr bool COOP = FOLD;
    // 16-bit loads stay 16-bit here: widened at their use, after the wait
    // for the tile (a widening of the first tile's values would otherwise be
    // placed before the loop and wait for every load of the tile).
    typedef typename std::conditional<NG == 1, uint16_t, uint32_t>::type srow_t;
    struct Tile {
        uint32_t ks[2][NSW];          // key scales (fp16)
        uint32_t kbias[2][NSW];
        uint32_t vw[8][VW];           // P V codes: keys 8 kb + e
        uint16_t vs[8];               // value scale / bias of key 8 kb + e (dequantized form)
        uint16_t vb[8];
        srow_t ksr, kbr, vsr, vbr;    // cooperative scale / bias rows (folded form)
    };
    // K stage: chunk position of chunk c in row r is c ^ kswz(r); the shift
    // makes the 16 rows that one LDS read spans start on distinct banks
    constexpr int SWS = NCH == 16 ? 0 : NCH == 8 ? 1 : NCH == 4 ? 2 : 3;
    auto kswz = [](int r) { return (r >> SWS) & (NCH - 1); };
    uint8_t* kstage = reinterpret_cast<uint8_t*>(&s_wave[wave][KSTAGE]);
    // lane offset of K load instruction i: row KPI i + lane / NCH, position
    // lane % NCH holds the row's chunk (lane % NCH) ^ kswz(row)
    uint32_t o_kl[NKI];
#pragma unroll
    for (int i = 0; i < NKI; ++i) {
        const int r = KPI * i + lane / NCH;
        o_kl[i] = (uint32_t)r * kcs + 16u * (uint32_t)((lane % NCH) ^ kswz(r));
    }
    // nw dwords at byte b (within one 16-byte chunk, or two whole chunks) of
    // staged row r
    auto lds_k = [&](int r, int b, uint32_t* dst, int nw) {
        const int sw = kswz(r);
#pragma unroll
        for (int c0 = 0; c0 < (nw > 4 ? nw / 4 : 1); ++c0) {
            const int bb = b + 16 * c0;
            const uint8_t* src = kstage + r * ROWB + 16 * ((bb >> 4) ^ sw) + (bb & 15);
            if (nw == 1) {
                dst[0] = *(const uint32_t*)src;
            } else if (nw == 2) {
                const uint2 x = *(const uint2*)src;
                dst[0] = x.x; dst[1] = x.y;
            } else {
                const uint4 x = *(const uint4*)src;
                dst[4 * c0] = x.x; dst[4 * c0 + 1] = x.y; dst[4 * c0 + 2] = x.z; dst[4 * c0 + 3] = x.w;
            }
        }
    };
    const uint32_t o_ks0 = (uint32_t)n * kss, o_ks1 = (uint32_t)(16 + n) * kss;
    const uint32_t o_v = (uint32_t)(8 * kb) * vcs + n * F::VBYTES;
    const uint32_t o_vs = (uint32_t)(8 * kb) * vss + 2 * vg;
    const uint32_t o_kr = (uint32_t)(lane & 31) * kss, o_vr = (uint32_t)(lane & 31) * vss;

    auto rsrc = [&](const uint8_t* base, int64_t row0, uint32_t stride, uint32_t rowb) {
        const int64_t rows = min((int64_t)TK, j1 - row0);
        const uint32_t bytes = rows > 0 ? (uint32_t)(rows - 1) * stride + rowb : 0u;
        return __builtin_amdgcn_make_buffer_rsrc((void*)(base + row0 * (int64_t)stride), (short)0,
                                                 (int)bytes, 0x00020000);
    };
    auto ld32 = [](__amdgpu_buffer_rsrc_t r, uint32_t off) -> uint32_t {
        return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    };
    auto ld16 = [](__amdgpu_buffer_rsrc_t r, uint32_t off) -> uint16_t {
        return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    };
    auto ldn = [&](__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* dst, int nw) {
        if (nw == 1) {
            dst[0] = ld32(r, off);
        } else if (nw == 2) {
            auto x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
            dst[0] = x[0]; dst[1] = x[1];
        } else {
#pragma unroll
            for (int q4 = 0; q4 < nw; q4 += 4) {
                auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 4 * q4), 0, 0);
                dst[q4] = x[0]; dst[q4 + 1] = x[1]; dst[q4 + 2] = x[2]; dst[q4 + 3] = x[3];
            }
        }
    };
    auto load_scales = [&](__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* dst) {
        if constexpr (NG == 1) dst[0] = ld16(r, off);
        else ldn(r, off, dst, NSW);
    };
    auto load_tile = [&](int tt, Tile& T) {
        const int64_t row0 = j0 + (int64_t)tt * TK;
        const auto rk = rsrc(kc, row0, kcs, F::ROWB);
        const auto rv = rsrc(vc, row0, vcs, F::ROWB);
#pragma unroll
        for (int i = 0; i < NKI; ++i)
            mf::buf_to_lds16(rk, kstage + 1024 * i, o_kl[i]);
        if constexpr (COOP) {
            auto ldrow = [&](__amdgpu_buffer_rsrc_t r, uint32_t off) -> srow_t {
                if constexpr (NG == 1) return ld16(r, off);
                else return ld32(r, off);
            };
            T.ksr = ldrow(rsrc(ksc, row0, kss, F::SROWB), o_kr);
            T.kbr = ldrow(rsrc(kbi, row0, kss, F::SROWB), o_kr);
            T.vsr = ldrow(rsrc(vsc, row0, vss, F::SROWB), o_vr);
            T.vbr = ldrow(rsrc(vbi, row0, vss, F::SROWB), o_vr);
        } else {
            const auto rks = rsrc(ksc, row0, kss, F::SROWB);
            load_scales(rks, o_ks0, T.ks[0]);
            load_scales(rks, o_ks1, T.ks[1]);
            if constexpr (MODE == MODE_AFFINE) {
                const auto rkb = rsrc(kbi, row0, kss, F::SROWB);
                load_scales(rkb, o_ks0, T.kbias[0]);
                load_scales(rkb, o_ks1, T.kbias[1]);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if constexpr (F::VBYTES == 2) T.vw[e][0] = ld16(rv, o_v + e * vcs);
            else ldn(rv, o_v + e * vcs, T.vw[e], VW);
        }
        if constexpr (!FOLD) {
            const auto rvs = rsrc(vsc, row0, vss, F::SROWB);
#pragma unroll
            for (int e = 0; e < 8; ++e) T.vs[e] = ld16(rvs, o_vs + e * vss);
            if constexpr (MODE == MODE_AFFINE) {
                const auto rvb = rsrc(vbi, row0, vss, F::SROWB);
#pragma unroll
                for (int e = 0; e < 8; ++e) T.vb[e] = ld16(rvb, o_vs + e * vss);
            }
        }
    };

    // Each wave reads the query values its lanes need (row n, the 8
    // consecutive d of every K-step; mostly cache hits, since every wave and
    // workgroup of the kv head reads the same 16 x D block) before it requests
    // its first tile, and nothing in the prologue waits on another wave: a
    // wave starts on its tile as soon as that tile has arrived.  Rows past G
    // read as zeros (the buffer's size stops at row G).
    const auto rq = flat_rsrc((const uint16_t*)p.q + (b * p.Hq + kvh * G) * D, (uint32_t)(G * D * 2));
    const bool q_al16 = (reinterpret_cast<uintptr_t>(p.q) & 15) == 0;   // q only needs 2-byte alignment
    u4 qraw[STEPS];
    auto q_off = [&](int st) {
        const int g = st / F::SPG, u = st % F::SPG;
        return 2u * (uint32_t)(n * D + g * GS + kb * (GS / 4) + 8 * u);
    };
    if (q_al16) {
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
            qraw[st] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)q_off(st), 0, 0);
    } else {
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t h = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rq, (int)(q_off(st) + 2 * i), 0, 0);
                qraw[st][i >> 1] = (i & 1) ? (qraw[st][i >> 1] | (h << 16)) : h;
            }
    }
    // keep the query loads ahead of the tile loads (waiting for q must not
    // wait for the tile)
    __builtin_amdgcn_sched_barrier(0);
    const int my_tiles = wave < ntiles ? (ntiles - wave + NWAVE - 1) / NWAVE : 0;
    // Decode with append: the new K/V token of this (batch, kv head) is pack
    // row L - 1, in the last tile of the last split; the wave that loads that
    // tile first quantizes the two new rows (qm::append_rows), writes them and
    // waits for its stores, so its load of the tile returns them.
    auto append_here = [&](int t) { return APPEND && split == p.S - 1 && t == ntiles - 1; };
    auto append_row = [&]() {
        if constexpr (APPEND && (MODE == MODE_AFFINE || MODE == MODE_Q8_0)) {
            const uint32_t row = (uint32_t)(p.L - 1);
            const int64_t e = b * p.ns0 + kvh * p.ns1;
            qm::append_rows<MODE, BITS, GS, D>(
                (const uint16_t*)p.k_new + e, (const uint16_t*)p.v_new + e, (uint8_t*)kc + row * kcs,
                (uint8_t*)vc + row * vcs, (uint8_t*)ksc + row * kss, (uint8_t*)vsc + row * vss,
                (uint8_t*)kbi + row * kss, (uint8_t*)vbi + row * vss);
            wait_stores();
        }
    };
    Tile cur;
    if (append_here(wave)) append_row();
    load_tile(wave, cur);
    __builtin_amdgcn_sched_barrier(0);

    // ---------------------------------------------------------------- queries
    // A operand of q K^T for every K-step; in the folded form also the
    // per-(head, group) sums of q of the lane's output rows 4 kb + j, taken
    // with lane reads (no LDS access: an LDS access here would wait for the
    // tile's direct-to-LDS loads).
    h8 qa[STEPS];
    float qs[4][NG];                    // (scale log2e) sum q of output rows 4kb + j
    {
        float part[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) part[g] = 0.0f;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const int g = st / F::SPG;
            const u4 raw = qraw[st];
            const uint32_t hw[4] = {raw[0], raw[1], raw[2], raw[3]};
            _Float16 hv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                hv[e] = __builtin_bit_cast(_Float16, (uint16_t)(hw[e >> 1] >> (16 * (e & 1))));
            uint32_t w[4];
#pragma unroll
            for (int hh = 0; hh < 4; ++hh) {
                _Float16 v0 = hv[qpos<BITS>(2 * hh)], v1 = hv[qpos<BITS>(2 * hh + 1)];
                if constexpr (FOLD) part[g] += (float)v0 + (float)v1;
                if constexpr (BITS == 4 && FOLD) {   // raw odd nibbles arrive as 16 c
                    if (hh & 1) { v0 = v0 * (_Float16)0.0625f; v1 = v1 * (_Float16)0.0625f; }
                }
                w[hh] = (uint32_t)__builtin_bit_cast(uint16_t, v0) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
            }
            qa[st] = to_h8(w[0], w[1], w[2], w[3]);
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if constexpr (FOLD) {
                const float s = sum4(part[g]) * sl;          // head n's group sum, in lanes n + 16 kb
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), j));
                    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 4 + j));
                    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 8 + j));
                    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 12 + j));
                    qs[j][g] = kb == 0 ? r0 : kb == 1 ? r1 : kb == 2 ? r2 : r3;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) qs[j][g] = 0.0f;
            }
        }
    }

    // ---------------------------------------------------------------- main loop
    f4 acc_o[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc_o[t] = f4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;
    float bsum[2] = {0.0f, 0.0f};     // folded: sum_key p b_g of the softmax head, per group
    float* sw = s_wave[wave];
    const float kscale = 16777216.0f * sl;        // 2^24 undoes the subnormal code scale

    auto process = [&](const Tile& cur, int tt) {
        const uint32_t base = (uint32_t)(j0 + (int64_t)tt * TK);
        // this lane's K codes from the stage: key 16 hf + n, per group the
        // KCH bytes at kb KCH (the B operand of every K-step)
        uint32_t kw[2][NG][KW];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int g = 0; g < NG; ++g) lds_k(16 * hf + n, g * (GS * BITS / 8) + kb * F::KCH, kw[hf][g], KW);

        // ---- scores of 2 x 16 keys
        uint32_t krow_s[2] = {0u, 0u}, krow_b[2] = {0u, 0u};
        if constexpr (COOP) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                krow_s[hf] = (uint32_t)__shfl((int)cur.ksr, 16 * hf + n, 64);
                krow_b[hf] = (uint32_t)__shfl((int)cur.kbr, 16 * hf + n, 64);
            }
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            float z[4];
            if constexpr (!FOLD) {
                // keys dequantized to fp16 per element (one accumulator for all
                // groups; the group scale and bias are in the operand)
                f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const uint32_t sw2 = cur.ks[hf][g >> 1];
                    const uint32_t s2 = perm_b(sw2, sw2, (g & 1) ? 0x03020302u : 0x01000100u);
                    uint32_t b2 = 0u;
                    if constexpr (MODE == MODE_AFFINE) {
                        const uint32_t bw2 = cur.kbias[hf][g >> 1];
                        b2 = perm_b(bw2, bw2, (g & 1) ? 0x03020302u : 0x01000100u);
                    }
#pragma unroll
                    for (int u = 0; u < F::SPG; ++u) {
                        const h8 kop = dequant_k<MODE, BITS>(&kw[hf][g][u * (BITS == 4 ? 1 : 2)], s2, b2);
                        acc = mfma(qa[g * F::SPG + u], kop, acc);
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) z[j] = acc[j] * sl;
            } else
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < F::SPG; ++u) {
                    const h8 kbop = unpack_k<MODE, BITS>(&kw[hf][g][u * (BITS == 4 ? 1 : 2)]);
                    acc = mfma(qa[g * F::SPG + u], kbop, acc);
                }
                const uint32_t sw2 = COOP ? krow_s[hf] : cur.ks[hf][g >> 1];
                const float s = (g & 1) ? hi_f16(sw2) : lo_f16(sw2);
                if constexpr (MODE == MODE_AFFINE) {
                    const uint32_t bw2 = COOP ? krow_b[hf] : cur.kbias[hf][g >> 1];
                    const float sc = s * kscale;
                    const float bb = (g & 1) ? hi_f16(bw2) : lo_f16(bw2);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float t = __builtin_fmaf(bb, qs[j][g], sc * acc[j]);
                        z[j] = g == 0 ? t : z[j] + t;
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float t = s * __builtin_fmaf(kscale, acc[j], -128.0f * qs[j][g]);
                        z[j] = g == 0 ? t : z[j] + t;
                    }
                }
            }
            const uint32_t j = base + 16 * hf + n;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                float v = z[jj];
                if (j > jmax) v = -INFINITY;
                else if constexpr (MASK) {
                    const int h = 4 * kb + jj;
                    if (h < G)
                        v += kLog2e * load_mask(p.mask, p.mask_dtype,
                                                b * p.ms0 + (kvh * G + h) * p.ms1 + j * p.ms3);
                }
                sw[(4 * kb + jj) * SROW + 16 * hf + n] = v;
            }
        }
        lds_order();

        // ---- online softmax: lane = (head n, keys 8 kb .. 8 kb + 7)
        float zz[8];
        {
            const float4 a = *(const float4*)&sw[n * SROW + 8 * kb];
            const float4 c = *(const float4*)&sw[n * SROW + 8 * kb + 4];
            zz[0] = a.x; zz[1] = a.y; zz[2] = a.z; zz[3] = a.w;
            zz[4] = c.x; zz[5] = c.y; zz[6] = c.z; zz[7] = c.w;
        }
        lds_order();
        float mx = fmaxf(fmaxf(fmaxf(zz[0], zz[1]), fmaxf(zz[2], zz[3])),
                         fmaxf(fmaxf(zz[4], zz[5]), fmaxf(zz[6], zz[7])));
        mx = max4(mx);
        const float m_new = fmaxf(m_run, mx);
        const bool grow = m_new > m_run;
        if (__ballot(grow) != 0ull) {
            const float alpha = grow ? (m_run == -INFINITY ? 0.0f : fast_exp2(m_run - m_new)) : 1.0f;
            l_run *= alpha;
            bsum[0] *= alpha;
            bsum[1] *= alpha;
            const float ac = FOLD ? __shfl(alpha, ch + 16 * kb, 64) : alpha;
#pragma unroll
            for (int t = 0; t < NT; ++t) acc_o[t] *= ac;
            m_run = m_new;
        }
        float pf[8];
        float ps = 0.0f;
        // while the head has seen no visible key (m_run = -inf) all its scores
        // are -inf, and 2^(-inf - 0) = 0: one select per lane, not per score
        const float m_sub = m_run == -INFINITY ? 0.0f : m_run;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pf[e] = fast_exp2(zz[e] - m_sub);
            ps += pf[e];
        }
        l_run += ps;
        uint32_t pb[4];
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
            h2 hp = {(_Float16)pf[2 * q2], (_Float16)pf[2 * q2 + 1]};
            pb[q2] = as_u(hp);
        }

        if constexpr (FOLD) {
            uint32_t vrs[8], vrb[8];      // scale / bias rows of keys 8 kb + e
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                vrs[e] = (uint32_t)__shfl((int)cur.vsr, 8 * kb + e, 64);
                vrb[e] = (uint32_t)__shfl((int)cur.vbr, 8 * kb + e, 64);
            }
            // bias sums of the softmax head, per group
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bsum[0] = __builtin_fmaf(pf[e], lo_f16(vrb[e]), bsum[0]);
                if constexpr (NG == 2) bsum[1] = __builtin_fmaf(pf[e], hi_f16(vrb[e]), bsum[1]);
            }
            // P' column (ch, cg): p of head ch (from its softmax lane) times the scale of cg
            uint32_t pp[4];
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
                const uint32_t src = (uint32_t)__shfl((int)pb[q2], ch + 16 * kb, 64);
                const uint32_t sa = vrs[2 * q2], sb2 = vrs[2 * q2 + 1];
                const uint32_t spair = (NG == 2 && cg == 1) ? perm_b(sb2, sa, 0x07060302u)
                                                            : perm_b(sb2, sa, 0x05040100u);
                pp[q2] = cvalid ? as_u(as_h2(src) * as_h2(spair)) : 0u;
            }
            const h8 pop = to_h8(pp[0], pp[1], pp[2], pp[3]);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                uint32_t a[4];
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2)
                    a[q2] = pair_sub<BITS>(cur.vw[2 * q2], cur.vw[2 * q2 + 1], t);
                acc_o[t] = mfma(to_h8(a[0], a[1], a[2], a[3]), pop, acc_o[t]);
            }
        } else {
            const h8 pop = to_h8(pb[0], pb[1], pb[2], pb[3]);
            uint32_t sp[4], bp[4];
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
                sp[q2] = perm_b(cur.vs[2 * q2 + 1], cur.vs[2 * q2], 0x05040100u);
                bp[q2] = MODE == MODE_AFFINE ? perm_b(cur.vb[2 * q2 + 1], cur.vb[2 * q2], 0x05040100u)
                                             : 0u;
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                uint32_t a[4];
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) {
                    const uint32_t x = pair_int<MODE, BITS>(cur.vw[2 * q2], cur.vw[2 * q2 + 1], t);
                    if constexpr (MODE == MODE_AFFINE) {
                        h2 c = as_h2(x) - (h2){(_Float16)1024.0f, (_Float16)1024.0f};
                        h2 s = as_h2(sp[q2]);
                        if constexpr (BITS == 4) {
                            if (t & 1) s = s * (h2){(_Float16)0.0625f, (_Float16)0.0625f};
                        }
                        a[q2] = as_u(__builtin_elementwise_fma(c, s, as_h2(bp[q2])));
                    } else {
                        h2 c = as_h2(x) - (h2){(_Float16)1152.0f, (_Float16)1152.0f};
                        a[q2] = as_u(c * as_h2(sp[q2]));
                    }
                }
                acc_o[t] = mfma(to_h8(a[0], a[1], a[2], a[3]), pop, acc_o[t]);
            }
        }
    };

    // One register tile per wave: the next tile's loads are issued as soon as
    // a tile is consumed (deeper register rings measured no faster: with every
    // CU streaming they only lengthen the memory queues).  Loads past the
    // split read zeros, so the loop needs no clamping and its waits are exact.
    for (int i = 0; i < my_tiles; ++i) {
        process(cur, wave + i * NWAVE);
        __builtin_amdgcn_sched_barrier(0);
        // no loads after the last tile: they would hold the wave (and the
        // workgroup merge behind it) until the CU's memory queue drains
        if (i + 1 < my_tiles) {
            if (append_here(wave + (i + 1) * NWAVE)) append_row();
            load_tile(wave + (i + 1) * NWAVE, cur);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---------------------------------------------------------------- merge waves
    // Every wave leaves its unscaled state in LDS; after one barrier each
    // thread combines the waves' states for its output elements.
    l_run = sum4(l_run);
    if constexpr (FOLD) {
        bsum[0] = sum4(bsum[0]);
        bsum[1] = sum4(bsum[1]);
    }
    if (kb == 0) {
        s_ml[wave][0][n] = m_run;
        s_ml[wave][1][n] = l_run;
        s_bias[wave][n][0] = bsum[0];
        s_bias[wave][n][1] = bsum[1];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) *(f4*)&s_wave[wave][(t * 64 + lane) * 4] = acc_o[t];   // [t][lane][4]
    __syncthreads();

    // ---------------------------------------------------------------- output
    // Item i -> (j, head oh, kbb, tc), j fastest: the P V values of the 4
    // consecutive d = DPT (4 kbb + j) + 4 tc + 0..3 sit in lane 16 kbb +
    // column, register j, of tiles 4 tc .. 4 tc + 3 (column = oh, or oh + G g
    // in the folded form; DPT = D / 16).  Consecutive threads read
    // consecutive LDS words; each item is one 16-byte (or 8-byte) store.
    constexpr int DPT = D / 16;
    static_assert(DPT % 4 == 0, "4 consecutive d per output item");
    float* ml = p.part_ml + (bk * p.S + split) * 32;
    float* po = p.part_o + (bk * p.S + split) * 16 * D;
    const int64_t obase = (b * p.Hq + kvh * G) * D;
    int cur_h = -1;
    float fw[NWAVE], Mh = 0.0f, Lh = 0.0f, bias_h[2] = {0.0f, 0.0f};
    for (int i = tid; i < G * D / 4; i += NTHR) {
        const int j = i & 3;
        const int oh = (i >> 2) % G;
        const int rest = (i >> 2) / G;
        const int kbb = rest & 3, tc = rest >> 2;
        const int d0 = DPT * (4 * kbb + j) + 4 * tc;
        if (oh != cur_h) {                // per-head wave factors (once per head)
            cur_h = oh;
            Mh = -INFINITY;
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) Mh = fmaxf(Mh, s_ml[w][0][oh]);
            Lh = 0.0f;
            bias_h[0] = bias_h[1] = 0.0f;
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) {
                const float mw = s_ml[w][0][oh];
                fw[w] = (mw == -INFINITY) ? 0.0f : fast_exp2(mw - Mh);
                Lh += fw[w] * s_ml[w][1][oh];
                bias_h[0] += fw[w] * s_bias[w][oh][0];
                bias_h[1] += fw[w] * s_bias[w][oh][1];
            }
        }
        const int g = FOLD ? d0 / GS : 0;             // 4 consecutive d share a group
        const int slot = (kbb * 16 + oh + (FOLD ? G * g : 0)) * 4 + j;
        float o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t = 4 * tc + q;
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) v += fw[w] * s_wave[w][t * 256 + slot];
            if constexpr (FOLD) {
                const float sc = (BITS == 4 && (q & 1)) ? 16777216.0f * 0.0625f : 16777216.0f;
                v = v * sc + (g ? bias_h[1] : bias_h[0]);
            }
            o[q] = v;
        }
        if (p.S == 1) {
            const float inv = Lh > 0.0f ? 1.0f / Lh : 0.0f;
            uint16_t* dst = (uint16_t*)p.out + obase + oh * D + d0;
            const uint16_t h[4] = {f32_to_f16(o[0] * inv), f32_to_f16(o[1] * inv),
                                   f32_to_f16(o[2] * inv), f32_to_f16(o[3] * inv)};
            if ((reinterpret_cast<uintptr_t>(p.out) & 7) == 0) {   // out only needs 2-byte alignment
                *(uint2*)dst = uint2{(uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                     (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) dst[q] = h[q];
            }
        } else {
            *(float4*)(po + oh * D + d0) = float4{o[0], o[1], o[2], o[3]};
            if (d0 == 0) {
                ml[2 * oh] = Mh;
                ml[2 * oh + 1] = Lh;
            }
        }
    }
}

template <int MODE, int BITS, int GS, int D, bool FOLD>
hipError_t launch_m(int64_t B, const AttnLaunch& p, hipStream_t stream) {
    dim3 grid(p.S, (unsigned)p.Hk, (unsigned)B);
    if (p.append) {
        // the decode with append: no additive mask
        if (p.mask_kind == MASK_ADDITIVE) return hipErrorNotSupported;
        hipLaunchKernelGGL((attn_matrix_decode<MODE, BITS, GS, D, false, FOLD, true>), grid, dim3(NTHR), 0,
                           stream, p);
        return hipGetLastError();
    }
    if (p.mask_kind == MASK_ADDITIVE)
        hipLaunchKernelGGL((attn_matrix_decode<MODE, BITS, GS, D, true, FOLD>), grid, dim3(NTHR), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((attn_matrix_decode<MODE, BITS, GS, D, false, FOLD>), grid, dim3(NTHR), 0,
                           stream, p);
    return hipGetLastError();
}

template <int MODE, int BITS, int GS, int D>
hipError_t by_fold(int64_t B, const AttnLaunch& p, hipStream_t s) {
    constexpr int NG = D / GS;
    if constexpr (MODE == MODE_AFFINE && NG <= 2) {
        if (p.G * NG <= 16) return launch_m<MODE, BITS, GS, D, true>(B, p, s);
    }
    return launch_m<MODE, BITS, GS, D, false>(B, p, s);
}

template <int MODE, int BITS, int GS>
hipError_t by_d(int D, int64_t B, const AttnLaunch& p, hipStream_t s) {
    switch (D) {
        case 64: if constexpr (GS <= 64) return by_fold<MODE, BITS, GS, 64>(B, p, s); else break;
        case 128: return by_fold<MODE, BITS, GS, 128>(B, p, s);
        case 256: return by_fold<MODE, BITS, GS, 256>(B, p, s);
    }
    return hipErrorNotSupported;
}

}  // namespace

bool matrix_supported(int q_dtype, int mode, int bits, int group_size, int D, int G, int64_t Lq) {
    if (q_dtype != DT_F16 || Lq < 1 || G < 1) return false;
    if (D != 64 && D != 128 && D != 256) return false;
    if (mode == MODE_DENSE) return true;
    if (!fast_format(mode, bits, D)) return false;
    if (mode == MODE_Q8_0) return true;
    if (bits != 4 && bits != 8) return false;
    if (group_size != 32 && group_size != 64 && group_size != 128) return false;
    return D % group_size == 0;
}

int decode_matrix_key_quantum() { return TK * NWAVE; }

bool decode_matrix_supported(int q_dtype, int mode, int bits, int group_size, int D, int G,
                             int64_t Lq) {
    return mode != MODE_DENSE && Lq == 1 && G <= 16 && matrix_supported(q_dtype, mode, bits, group_size, D, G, Lq);
}

hipError_t launch_attn_matrix(int mode, int bits, int D, int64_t B, const AttnLaunch& p,
                              hipStream_t stream) {
    const int gs = 1 << p.gs_log2;
    if (mode == MODE_Q8_0) return by_d<MODE_Q8_0, 8, 32>(D, B, p, stream);
    if (bits == 4) {
        if (gs == 32) return by_d<MODE_AFFINE, 4, 32>(D, B, p, stream);
        if (gs == 64) return by_d<MODE_AFFINE, 4, 64>(D, B, p, stream);
        if (gs == 128) return by_d<MODE_AFFINE, 4, 128>(D, B, p, stream);
    } else if (bits == 8) {
        if (gs == 32) return by_d<MODE_AFFINE, 8, 32>(D, B, p, stream);
        if (gs == 64) return by_d<MODE_AFFINE, 8, 64>(D, B, p, stream);
        if (gs == 128) return by_d<MODE_AFFINE, 8, 128>(D, B, p, stream);
    }
    return hipErrorNotSupported;
}

}  // namespace qkv
