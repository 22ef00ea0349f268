// Matrix-core prefill for fp16 queries on gfx950: attention of Lq > 1 queries
// per head over a group-quantized KV cache, optionally causal (bottom-right)
// or with an additive mask.
//
// Semantics as the decode kernels (MLX page "add fast::quantized_kv_update",
// fast.cpp quantized_scaled_dot_product_attention: the GQA reshape and the
// composition quantized_matmul -> + mask -> softmax -> quantized_matmul).
// The prefill design follows the llama.cpp page "Metal: Optimize q8_0 KV -
// #25556" in dequantizing K/V once per tile for a block of query rows, and
// the tile loop of the MLX CUDA page "Fixed mma and working dequant"
// (qmm.cu: dequantize a tile into shared memory, then matrix multiply), laid
// out for gfx950:
//
//  * A workgroup owns 128 (or, for few rows, 64) GQA-packed rows (row
//    p = query i * G + head g of one kv head) and streams key tiles of 64.
//    Its 512 threads dequantize the next K and V tile (fp16, row-major, in
//    LDS, double buffered) while the current one is consumed; the stores of
//    each 8-lane group hit distinct LDS banks.
//  * 8 waves, two per SIMD (one hides the other's LDS and matrix latencies).
//    With 128 rows each wave takes a 16-row block over all 64 keys of a
//    tile; with 64 rows waves w and w + 4 share the 16-row block w % 4 and
//    take the two 32-key halves, keeping separate softmax states that are
//    merged through LDS at the end.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_f16 (A = K rows from LDS, B = the
//    wave's queries in registers), so each lane holds 4 keys x its row per
//    16-key subtile: the online softmax of a row is lane-local plus a 4-lane
//    reduction (v_permlane*_swap).
//  * O^T = V^T P^T: A = V^T read straight from the row-major V tile with
//    ds_read_b64_tr_b16 (4 consecutive keys at one d per lane), B = P^T from
//    the score accumulators (the key order of both operands is the same
//    permutation), so the output rows stay in the lanes of their softmax
//    state and rescaling is lane-local.
//  * Causal/additive masking is applied per (row, key) only on tiles that
//    cross a row's last visible key; fully hidden tiles are skipped.
//  * With several key splits the rows' (m, l, o) go to the workspace for the
//    split merge kernel.
//  * A dense fp16 cache (the unquantized baseline, or the fp16 copies of the
//    dequantize-first strategy of the llama.cpp page) takes the same path
//    with its rows staged into LDS as loaded.
#include "qkv_internal.hpp"
#include "qkv_mfma.hpp"

namespace qkv {

namespace {

using namespace mf;

constexpr int BN = 64;          // keys per tile
constexpr int PW = 8;           // waves
constexpr int PNTHR = PW * 64;
constexpr float kLazy = 8.0f;   // running-maximum slack (log2 units)

// Dequantize 16 consecutive codes of a row (one uint4) into 8 fp16 pairs.
// Affine: s * c + b rounded once (v_pk_fma_f16); Q8_0: d * c (c exact in fp16).
template <int MODE, int BITS>
__device__ __forceinline__ void dequant16(uint4 w, uint32_t s2, uint32_t b2, uint32_t out[8]) {
    const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (MODE == MODE_Q8_0) {
            // bytes c -> halves 1024 + (c + 128), minus 1152, times d
            const uint32_t u = x[i] ^ 0x80808080u;
            const h2 c0 = as_h2(perm_b(0x64646464u, u, 0x04010400u)) - (h2){(_Float16)1152.0f, (_Float16)1152.0f};
            const h2 c1 = as_h2(perm_b(0x64646464u, u, 0x04030402u)) - (h2){(_Float16)1152.0f, (_Float16)1152.0f};
            out[2 * i] = as_u(c0 * as_h2(s2));
            out[2 * i + 1] = as_u(c1 * as_h2(s2));
        } else {
            const h2 c0 = as_h2(perm_b(0x64646464u, x[i], 0x04010400u)) - (h2){(_Float16)1024.0f, (_Float16)1024.0f};
            const h2 c1 = as_h2(perm_b(0x64646464u, x[i], 0x04030402u)) - (h2){(_Float16)1024.0f, (_Float16)1024.0f};
            out[2 * i] = as_u(__builtin_elementwise_fma(c0, as_h2(s2), as_h2(b2)));
            out[2 * i + 1] = as_u(__builtin_elementwise_fma(c1, as_h2(s2), as_h2(b2)));
        }
    }
}

// 4-bit: 8 consecutive codes (one dword) into 4 fp16 pairs.
__device__ __forceinline__ void dequant8_4bit(uint32_t w, uint32_t s2, uint32_t b2, uint32_t out[4]) {
    // element e sits in bits [4e, 4e + 4)
    const uint32_t a = perm_b(0u, w, 0x0C010C00u);             // [b0, 0, b1, 0]: (c0|c1<<4, c2|c3<<4)
    const uint32_t c = perm_b(0u, w, 0x0C030C02u);             // bytes 2, 3
    const h2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    const h2 lo0 = as_h2((a & 0x000F000Fu) | 0x64006400u) - k1024;          // c0, c2
    const h2 hi0 = as_h2(((a >> 4) & 0x000F000Fu) | 0x64006400u) - k1024;   // c1, c3
    const h2 lo1 = as_h2((c & 0x000F000Fu) | 0x64006400u) - k1024;          // c4, c6
    const h2 hi1 = as_h2(((c >> 4) & 0x000F000Fu) | 0x64006400u) - k1024;   // c5, c7
    const h2 v02 = __builtin_elementwise_fma(lo0, as_h2(s2), as_h2(b2));
    const h2 v13 = __builtin_elementwise_fma(hi0, as_h2(s2), as_h2(b2));
    const h2 v46 = __builtin_elementwise_fma(lo1, as_h2(s2), as_h2(b2));
    const h2 v57 = __builtin_elementwise_fma(hi1, as_h2(s2), as_h2(b2));
    // back to element order: (v0, v1), (v2, v3), (v4, v5), (v6, v7)
    out[0] = perm_b(as_u(v13), as_u(v02), 0x05040100u);
    out[1] = perm_b(as_u(v13), as_u(v02), 0x07060302u);
    out[2] = perm_b(as_u(v57), as_u(v46), 0x05040100u);
    out[3] = perm_b(as_u(v57), as_u(v46), 0x07060302u);
}

// RB 16-row blocks per workgroup: RB = 4 (64 rows; waves w and w + 4 take
// the two 32-key halves of each tile) or RB = 8 (128 rows; every wave takes
// all 64 keys, so each dequantized tile serves twice the rows).
template <int MODE, int BITS, int GS, int D, int RB>
__global__ __launch_bounds__(PNTHR) void attn_matrix_prefill(AttnLaunch p) {
    static_assert(RB == 4 || RB == 8, "64 or 128 rows per workgroup");
    constexpr int KH = PW / RB;                    // key parts per tile (2 or 1)
    constexpr int BMR = 16 * RB;                   // rows per workgroup
    constexpr int KPW = BN / KH;                   // keys per wave and tile
    constexpr int NSUB = KPW / 16;                 // 16-key subtiles per wave
    constexpr int NG = D / GS;
    constexpr int ROWB = D * BITS / 8;             // code bytes per row
    constexpr int LDROW = D + 16;                  // LDS row stride in halves (pad 32 B)
    constexpr int STEPS = D / 32;                  // K-steps of S^T
    constexpr int NT = D / 16;                     // output d-tiles
    constexpr int TPR = D / 16 < 8 ? D / 16 : 8;   // dequant threads per key row
    constexpr int DPT = D / TPR;                   // d per dequant thread (16 or 32: one group)
    constexpr int CB = DPT * BITS / 8;             // code bytes per dequant thread
    constexpr int NCH = CB / 16 > 0 ? CB / 16 : 1; // uint4 loads per dequant thread
    static_assert(DPT % 16 == 0 && DPT <= GS, "a dequant thread covers whole 16-d steps of one group");

    __shared__ __attribute__((aligned(16))) _Float16 s_k[2][BN * LDROW];
    __shared__ __attribute__((aligned(16))) _Float16 s_v[2][BN * LDROW];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rb = wave % RB;                      // 16-row block
    const int kh = wave / RB;                      // key part of each tile
    const int lane = tid & 63;
    const int n = lane & 15;
    const int kb = lane >> 4;
    const int split = blockIdx.x;
    const int rt = blockIdx.y;                     // row tile
    pin_sgpr(p.q); pin_sgpr(p.Hq); pin_sgpr(p.Hk); pin_sgpr(p.G); pin_sgpr(p.L); pin_sgpr(p.Lq);
    pin_sgpr(p.chunk); pin_sgpr(p.scale); pin_sgpr(p.mask_kind); pin_sgpr(p.n_rows);
    pin_sgpr(p.k.codes); pin_sgpr(p.k.scales); pin_sgpr(p.k.biases);
    pin_sgpr(p.k.sb); pin_sgpr(p.k.sh); pin_sgpr(p.k.sl);
    pin_sgpr(p.v.codes); pin_sgpr(p.v.scales); pin_sgpr(p.v.biases);
    pin_sgpr(p.v.sb); pin_sgpr(p.v.sh); pin_sgpr(p.v.sl);
    // z = batch x kv head (below 2^16: 32-bit division)
    const uint32_t bk32 = blockIdx.z, hk32 = (uint32_t)p.Hk;
    const int64_t bk = bk32;
    const int64_t b = bk32 / hk32;
    const int64_t kvh = bk32 - (uint32_t)b * hk32;
    const int G = p.G;
    const float sl = p.scale * kLog2e;

    // this lane's row (the B column of S^T and of O^T); a wave whose 16-row
    // block lies past the last row (decode, ragged last tile) only loads and
    // stages tiles for the others
    const bool rb_live = rt * BMR + rb * 16 < p.n_rows;
    const int row = rt * BMR + rb * 16 + n;
    const bool row_ok = row < p.n_rows;
    const int rowc = row_ok ? row : p.n_rows - 1;
    const int64_t qi = rowc / G;
    const int64_t qh = kvh * G + rowc % G;
    const int64_t last_vis = (p.mask_kind == MASK_CAUSAL) ? p.L - p.Lq + qi : p.L - 1;

    // key range: the split's chunk, cut at the last key any row of the tile sees
    const int64_t j_begin = (int64_t)split * p.chunk;
    int64_t j_end = min(p.L, j_begin + p.chunk);
    if (p.mask_kind == MASK_CAUSAL) {
        const int last_row = min(rt * BMR + BMR, p.n_rows) - 1;
        j_end = min(j_end, p.L - p.Lq + last_row / G + 1);
    }
    const int ntile = j_end > j_begin ? (int)((j_end - j_begin + BN - 1) / BN) : 0;
    // first key hidden from some row of the tile (tiles before it need no mask)
    const int first_row = rt * BMR;
    const int64_t lo_vis = (p.mask_kind == MASK_CAUSAL) ? p.L - p.Lq + first_row / G : p.L - 1;

    // ---- queries: B operand of S^T = K Q^T (row n, d = 32 st + 8 kb .. + 7)
    h8 qb[STEPS];
    {
        const _Float16* qrow = (const _Float16*)p.q + ((b * p.Hq + qh) * p.Lq + qi) * D;
        // the loads are at multiples of 16 bytes from q
        const bool q_al16 = (reinterpret_cast<uintptr_t>(p.q) & 15) == 0;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const uint4 raw = load_h8((const uint16_t*)(qrow + 32 * st + 8 * kb), q_al16);
            u4 v = {row_ok ? raw.x : 0u, row_ok ? raw.y : 0u, row_ok ? raw.z : 0u, row_ok ? raw.w : 0u};
            qb[st] = __builtin_bit_cast(h8, v);
        }
    }

    // ---- dequantization of a K/V tile into LDS.  Thread -> (key row drow,
    // slice dq of DPT d): lane l of wave w takes row 8 w + l % 8 and slice
    // l / 8, so the 8 lanes of each store group write 8 consecutive rows.  The
    // row stride is 8 dwords modulo the 32 LDS banks, so rows r and r + 4 of a
    // group would collide; rows 4..7 of each group store their 16-byte chunks
    // in swapped pairs (the pair's codes are swapped before dequantization),
    // which puts the group's 8 stores on distinct banks.
    const int64_t krow0 = b * p.k.sb + kvh * p.k.sh;
    const int64_t vrow0 = b * p.v.sb + kvh * p.v.sh;
    const int drow = 8 * wave + (lane & 7);        // key row of the tile
    const int dq = lane >> 3;                      // slice of the row
    const bool dq_on = dq < TPR;
    const int dgrp = (dq * DPT) / GS;              // its quantization group
    const bool swap = (drow >> 2) & 1;
    constexpr int SROWB = NG * 2;                  // scale bytes per row
    const uint8_t* kcb = (const uint8_t*)p.k.codes + krow0 * ROWB;
    const uint8_t* vcb = (const uint8_t*)p.v.codes + vrow0 * ROWB;
    const uint8_t* ksb = (const uint8_t*)p.k.scales + krow0 * SROWB;
    const uint8_t* vsb = (const uint8_t*)p.v.scales + vrow0 * SROWB;
    const uint8_t* kbb = (const uint8_t*)p.k.biases + krow0 * SROWB;
    const uint8_t* vbb = (const uint8_t*)p.v.biases + vrow0 * SROWB;
    const uint32_t kcs = (uint32_t)(p.k.sl * ROWB), vcs = (uint32_t)(p.v.sl * ROWB);
    const uint32_t kss = (uint32_t)(p.k.sl * SROWB), vss = (uint32_t)(p.v.sl * SROWB);
    const uint32_t o_kc = (uint32_t)drow * kcs + dq * CB, o_vc = (uint32_t)drow * vcs + dq * CB;
    const uint32_t o_ks = (uint32_t)drow * kss + 2 * dgrp, o_vs = (uint32_t)drow * vss + 2 * dgrp;
    struct Raw {
        uint4 kc[NCH], vc[NCH];
        uint32_t ks, kbias, vs, vbias;             // fp16 scale / bias of the slice's group
    };
    // rows past the split's end read as zeros (buffer bounds): their scores are
    // masked and their zero values add nothing
    auto load_raw = [&](int t, Raw& R) {
        const int64_t r0 = j_begin + (int64_t)t * BN;
        const auto rk = rows_rsrc(kcb, r0, j_end, BN, kcs, ROWB);
        const auto rv = rows_rsrc(vcb, r0, j_end, BN, vcs, ROWB);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if constexpr (CB >= 16) {
                const auto x = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(o_kc + 16 * c), 0, 0);
                const auto y = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(o_vc + 16 * c), 0, 0);
                R.kc[c] = uint4{x[0], x[1], x[2], x[3]};
                R.vc[c] = uint4{y[0], y[1], y[2], y[3]};
            } else {
                const auto x = __builtin_amdgcn_raw_buffer_load_b64(rk, (int)o_kc, 0, 0);
                const auto y = __builtin_amdgcn_raw_buffer_load_b64(rv, (int)o_vc, 0, 0);
                R.kc[c] = uint4{x[0], x[1], 0u, 0u};
                R.vc[c] = uint4{y[0], y[1], 0u, 0u};
            }
        }
        if constexpr (MODE == MODE_DENSE) {
            R.ks = R.vs = 0u;
        } else {
            R.ks = buf16(rows_rsrc(ksb, r0, j_end, BN, kss, SROWB), o_ks);
            R.vs = buf16(rows_rsrc(vsb, r0, j_end, BN, vss, SROWB), o_vs);
        }
        if constexpr (MODE == MODE_AFFINE) {
            R.kbias = buf16(rows_rsrc(kbb, r0, j_end, BN, kss, SROWB), o_ks);
            R.vbias = buf16(rows_rsrc(vbb, r0, j_end, BN, vss, SROWB), o_vs);
        } else {
            R.kbias = R.vbias = 0u;
        }
    };
    // one 16-d step: 16 codes (one uint4 of 8-bit codes, or two dwords of 4-bit
    // codes) -> the slice's chunks 2 c16 and 2 c16 + 1 in LDS, in swapped order
    // on swapping rows (codes swapped first, so the stores need no selects)
    auto store_step = [&](uint4 w, uint32_t s2, uint32_t b2, _Float16* dst, int c16) {
        uint32_t o[8];
        if constexpr (BITS == 4) {
            const uint32_t lo = swap ? w.y : w.x, hi = swap ? w.x : w.y;
            dequant8_4bit(lo, s2, b2, o);
            dequant8_4bit(hi, s2, b2, o + 4);
        } else {
            const uint4 x = swap ? uint4{w.z, w.w, w.x, w.y} : w;
            dequant16<MODE, BITS>(x, s2, b2, o);
        }
        const int c0 = 2 * c16 + (swap ? 1 : 0), c1 = 2 * c16 + (swap ? 0 : 1);
        *(uint4*)(dst + 8 * c0) = uint4{o[0], o[1], o[2], o[3]};
        *(uint4*)(dst + 8 * c1) = uint4{o[4], o[5], o[6], o[7]};
    };
    // the K (or V) half of a tile: the slice's codes -> fp16 rows in LDS
    auto store_half = [&](const uint4* codes, uint32_t sc, uint32_t bi, _Float16* dst) {
        if constexpr (MODE == MODE_DENSE) {
            // fp16 values: the chunks as loaded, the pair's order swapped on
            // swapping rows as for the dequantized chunks
            // (a mask, not a select: a select of the two chunks becomes an
            // indexed access through scratch memory)
            const uint32_t m = swap ? 0xffffffffu : 0u;
#pragma unroll
            for (int c16 = 0; c16 < DPT / 16; ++c16) {
                const uint4 a = codes[2 * c16], c = codes[2 * c16 + 1];
                const uint4 x = {a.x ^ c.x, a.y ^ c.y, a.z ^ c.z, a.w ^ c.w};
                const uint4 first = {a.x ^ (x.x & m), a.y ^ (x.y & m), a.z ^ (x.z & m), a.w ^ (x.w & m)};
                const uint4 second = {c.x ^ (x.x & m), c.y ^ (x.y & m), c.z ^ (x.z & m), c.w ^ (x.w & m)};
                const int c0 = 2 * c16 + (swap ? 1 : 0), c1 = 2 * c16 + (swap ? 0 : 1);
                *(uint4*)(dst + 8 * c0) = first;
                *(uint4*)(dst + 8 * c1) = second;
            }
            return;
        }
        const uint32_t s2 = sc | (sc << 16), b2 = bi | (bi << 16);
#pragma unroll
        for (int c16 = 0; c16 < DPT / 16; ++c16) {
            uint4 w;
            if constexpr (BITS == 4) {
                const uint4 x = codes[c16 / 2];
                w = (c16 & 1) ? uint4{x.z, x.w, 0u, 0u} : uint4{x.x, x.y, 0u, 0u};
            } else {
                w = codes[c16];
            }
            store_step(w, s2, b2, dst, c16);
        }
    };
    auto store_k = [&](const Raw& R, int buf) {
        store_half(R.kc, R.ks, R.kbias, &s_k[buf][drow * LDROW + dq * DPT]);
    };
    auto store_v = [&](const Raw& R, int buf) {
        store_half(R.vc, R.vs, R.vbias, &s_v[buf][drow * LDROW + dq * DPT]);
    };

    // ---- main loop
    f4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    // Raw codes are loaded two tiles ahead into two register sets that
    // alternate between iterations (iter(t, cur): cur holds tile t + 1 and is
    // refilled with tile t + 3 once dequantized).
    Raw raw0, raw1;
    if (ntile > 0 && dq_on) {
        load_raw(0, raw0);
        store_k(raw0, 0);
        store_v(raw0, 0);
        if (ntile > 1) load_raw(1, raw0);
        if (ntile > 2) load_raw(2, raw1);
    }
    __syncthreads();

    auto iter = [&](int t, Raw& cur) {
        const int buf = t & 1;
        const int64_t j0 = j_begin + (int64_t)t * BN + KPW * kh;  // first key of this wave's part
        const _Float16* kt = s_k[buf];
        const _Float16* vt = s_v[buf];
        if (rb_live) {

        // S^T for the part's subtiles of 16 keys: lane holds keys 16 u + 4 kb + jj of row n
        float sc[NSUB][4];
#pragma unroll
        for (int u = 0; u < NSUB; ++u) {
            f4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < STEPS; ++st) {
                const h8 ka = *(const h8*)(kt + (KPW * kh + 16 * u + n) * LDROW + 32 * st + 8 * kb);
                s = mfma16(ka, qb[st], s);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) sc[u][jj] = s[jj] * sl;
        }
        // masking: only parts reaching past the first row's last visible key,
        // the ragged end of the split, or with an additive mask
        const bool edge = (j0 + KPW - 1 > lo_vis) || (j0 + KPW > j_end) || p.mask_kind == MASK_ADDITIVE;
        if (edge) {
#pragma unroll
            for (int u = 0; u < NSUB; ++u)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int64_t j = j0 + 16 * u + 4 * kb + jj;
                    float v = sc[u][jj];
                    if (j >= j_end || j > last_vis || !row_ok) v = -INFINITY;
                    else if (p.mask_kind == MASK_ADDITIVE)
                        v += kLog2e * load_mask(p.mask, p.mask_dtype,
                                                b * p.ms0 + qh * p.ms1 + qi * p.ms2 + j * p.ms3);
                    sc[u][jj] = v;
                }
        }
        // online softmax of row n over the part (4 NSUB keys in this lane, x4 lanes)
        float mx = sc[0][0];
#pragma unroll
        for (int u = 0; u < NSUB; ++u)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) mx = fmaxf(mx, sc[u][jj]);
        mx = max4(mx);
        // lazy maximum: raised only when a score exceeds it by kLazy (log2
        // units), so p = 2^(s - m) <= 2^kLazy stays well inside fp16
        const bool grow = mx > m_run + kLazy;
        const float m_new = grow ? fmaxf(m_run, mx) : m_run;
        if (__ballot(grow) != 0ull) {
            const float alpha = grow ? (m_run == -INFINITY ? 0.0f : fast_exp2(m_run - m_new)) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int t2 = 0; t2 < NT; ++t2) acc[t2] *= alpha;
            m_run = m_new;
        }
        // while the row has seen no visible key (m_run = -inf) all its scores
        // are -inf, and 2^(-inf - 0) = 0: one select per lane, not per score
        const float m_sub = m_run == -INFINITY ? 0.0f : m_run;
        uint32_t pp[NSUB][2];     // P^T operand halves: keys (16u + 4kb + jj) in pairs
        float ps = 0.0f;
#pragma unroll
        for (int u = 0; u < NSUB; ++u) {
            float e[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                e[jj] = fast_exp2(sc[u][jj] - m_sub);
                ps += e[jj];
            }
            h2 a = {(_Float16)e[0], (_Float16)e[1]}, c = {(_Float16)e[2], (_Float16)e[3]};
            pp[u][0] = as_u(a);
            pp[u][1] = as_u(c);
        }
        l_run += ps;
        // O^T += V^T P^T over the part, 32 keys (two subtiles) per step: the
        // lane's 8 keys are 4 kb .. 4 kb + 3 of each subtile, in the order of pp
#pragma unroll
        for (int sp = 0; sp < NSUB / 2; ++sp) {
            const h8 pb = to_h8(pp[2 * sp][0], pp[2 * sp][1], pp[2 * sp + 1][0], pp[2 * sp + 1][1]);
            const int k0a = KPW * kh + 32 * sp + 4 * kb;   // subtile 2 sp, keys 4kb..
            const int k0b = k0a + 16;                     // subtile 2 sp + 1
#pragma unroll
            for (int t2 = 0; t2 < NT; ++t2) {
                // lane (s = n within its 16-lane group) points at V[k0 + s/4][16 t2 + 4 (s%4)];
                // the transpose read returns V[k0 .. k0+3][16 t2 + n]
                const _Float16* pa = vt + (k0a + (n >> 2)) * LDROW + 16 * t2 + 4 * (n & 3);
                const _Float16* pb2 = vt + (k0b + (n >> 2)) * LDROW + 16 * t2 + 4 * (n & 3);
                const s4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s4*)(pa));
                const s4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s4*)(pb2));
                const h8 aop = __builtin_bit_cast(h8, (short __attribute__((ext_vector_type(8)))){
                    va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]});
                acc[t2] = mfma16(aop, pb, acc[t2]);
            }
        }
        }
        // next tile -> the other buffer, then one barrier per tile
        if (t + 1 < ntile && dq_on) {
            store_k(cur, buf ^ 1);
            store_v(cur, buf ^ 1);
            if (t + 3 < ntile) load_raw(t + 3, cur);
        }
        __syncthreads();
    };
    for (int t = 0; t < ntile; t += 2) {
        iter(t, raw0);
        if (t + 1 < ntile) iter(t + 1, raw1);
    }

    // ---- merge the two key halves of each row block through LDS (the tile
    // buffers are free after the loop's last barrier)
    l_run = sum4(l_run);
    if constexpr (KH == 2) {
    float* xo = (float*)&s_k[0][0];                // [rb][t][lane][4] floats
    float* xml = (float*)&s_v[0][0];               // [rb][lane][2]
    if (kh == 1) {
#pragma unroll
        for (int t2 = 0; t2 < NT; ++t2) *(f4*)&xo[((rb * NT + t2) * 64 + lane) * 4] = acc[t2];
        xml[(rb * 64 + lane) * 2] = m_run;
        xml[(rb * 64 + lane) * 2 + 1] = l_run;
    }
    __syncthreads();
    if (kh == 1) return;
    {
        const float m1 = xml[(rb * 64 + lane) * 2], l1 = xml[(rb * 64 + lane) * 2 + 1];
        const float M = fmaxf(m_run, m1);
        const float f0 = m_run == -INFINITY ? 0.0f : fast_exp2(m_run - M);
        const float f1 = m1 == -INFINITY ? 0.0f : fast_exp2(m1 - M);
#pragma unroll
        for (int t2 = 0; t2 < NT; ++t2)
            acc[t2] = acc[t2] * f0 + *(const f4*)&xo[((rb * NT + t2) * 64 + lane) * 4] * f1;
        l_run = l_run * f0 + l1 * f1;
        m_run = M;
    }
    }

    // ---- output: lane holds O^T[d = 16 t + 4 kb + jj][row n]
    if (!row_ok) return;
    if (p.S == 1) {
        const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
        _Float16* op = (_Float16*)p.out + ((b * p.Hq + qh) * p.Lq + qi) * D;
        const bool out_al8 = (reinterpret_cast<uintptr_t>(p.out) & 7) == 0;
#pragma unroll
        for (int t2 = 0; t2 < NT; ++t2) {
            h4 o4 = {(_Float16)(acc[t2][0] * inv), (_Float16)(acc[t2][1] * inv),
                     (_Float16)(acc[t2][2] * inv), (_Float16)(acc[t2][3] * inv)};
            if (out_al8) {                             // out only needs 2-byte alignment
                *(h4*)(op + 16 * t2 + 4 * kb) = o4;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) op[16 * t2 + 4 * kb + e] = o4[e];
            }
        }
        return;
    }
    // partial state for the split merge: 16-row tile index of this row
    const int64_t tile16 = bk * p.n_rt + row / 16;
    const int r16 = row % 16;
    float* ml = p.part_ml + ((tile16 * p.S + split) * 16 + r16) * 2;
    float* po = p.part_o + ((tile16 * p.S + split) * 16 + r16) * D;
#pragma unroll
    for (int t2 = 0; t2 < NT; ++t2)
        *(float4*)(po + 16 * t2 + 4 * kb) = float4{acc[t2][0], acc[t2][1], acc[t2][2], acc[t2][3]};
    if (kb == 0) { ml[0] = m_run; ml[1] = l_run; }
}

template <int MODE, int BITS, int GS, int D>
hipError_t launch_p(int64_t B, const AttnLaunch& p, hipStream_t s) {
    const int bm = p.wg_rows;
    const int nwg = (p.n_rows + bm - 1) / bm;
    dim3 grid(p.S, nwg, (unsigned)(B * p.Hk));
    if (bm == 128)
        hipLaunchKernelGGL((attn_matrix_prefill<MODE, BITS, GS, D, 8>), grid, dim3(PNTHR), 0, s, p);
    else if (bm == 64)
        hipLaunchKernelGGL((attn_matrix_prefill<MODE, BITS, GS, D, 4>), grid, dim3(PNTHR), 0, s, p);
    else
        return hipErrorNotSupported;
    return hipGetLastError();
}

template <int MODE, int BITS, int GS>
hipError_t by_d(int D, int64_t B, const AttnLaunch& p, hipStream_t s) {
    switch (D) {
        case 64: if constexpr (GS <= 64) return launch_p<MODE, BITS, GS, 64>(B, p, s); else break;
        case 128: return launch_p<MODE, BITS, GS, 128>(B, p, s);
        case 256: return launch_p<MODE, BITS, GS, 256>(B, p, s);
    }
    return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_prefill_matrix(int mode, int bits, int D, int64_t B, const AttnLaunch& p,
                                 hipStream_t stream) {
    const int gs = 1 << p.gs_log2;
    if (mode == MODE_DENSE) {
        switch (D) {
            case 64: return launch_p<MODE_DENSE, 16, 64, 64>(B, p, stream);
            case 128: return launch_p<MODE_DENSE, 16, 128, 128>(B, p, stream);
            case 256: return launch_p<MODE_DENSE, 16, 256, 256>(B, p, stream);
        }
        return hipErrorNotSupported;
    }
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
