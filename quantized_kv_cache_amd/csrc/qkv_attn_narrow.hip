// Matrix-core decode for narrow GQA groups (G = Hq/Hk <= 4) with fp16
// queries: one query per head over a group-quantized KV cache.
//
// What is computed follows the MLX page "add fast::quantized_kv_update"
// (sdpa_vector.h quant_sdpa_vector: scores from packed codes through the
// per-group factorisation  q . (s c + b) = s (q . c) + b (sum q), online
// softmax, merge of partial softmax states) and the llama.cpp page "Metal:
// Optimize q8_0 KV - #25556" (Q8_0 blocks; the heads of a GQA group share
// every K/V load).  With only G <= 4 query rows per kv head, a 16-row matrix
// tile would leave 12 rows idle in the scores and the softmax, so this kernel
// lays the work out differently:
//
//  * q K^T on v_mfma_f32_4x4x4_16b_f16: 16 blocks, block b = keys 4b..4b+3 of
//    a 64-key tile, 4 rows = the G heads, contraction over 4 d per step.  The
//    result leaves lane l with the G scores of key l, so the key's scale and
//    bias are lane-local and the softmax runs on real scores only.  The q
//    operand of all blocks is broadcast from one block (CBSZ / ABID), so
//    16 steps of q fit in one register pair per lane: lane 4a + i holds head
//    i's 4 values of step a of the bank.
//  * Codes enter the matrix core unconverted (masking a packed word leaves
//    fp16 subnormals c * 2^-24; 4-bit odd nibbles arrive as 16 c against a q
//    pre-divided by 16; Q8_0 codes have the sign bit flipped, c + 128); each
//    step lies in one quantization group and the groups have separate
//    accumulators, so  z = sum_g s_g 2^24 acc_g + b_g sum_{d in g} q_d.
//    The symmetric 4-bit blocks (the q4_0 reading of the llama.cpp page's
//    merged #27390 text: d c with c a 4-bit two's complement code) are the
//    affine 4-bit form of the same block: flipping each nibble's top bit
//    gives c + 8, and d c = d (c + 8) + (-8 d), so they run as affine codes
//    with the bias -8 d derived from the scale (no bias plane).
//  * Online softmax with a lazy maximum: the running maxima change (and the
//    wave reduces, rescales) only when a tile holds a score 8 (log2 units)
//    above them, or any larger score for keys with a large value scale.
//  * P V folded into the matrix core as in the 16-head kernel: the value
//    scale moves into P', whose 16 columns are (head, group) pairs, the bias
//    term sum_key p b_g is accumulated per lane.  Each lane writes its key's
//    row of P' to a per-wave LDS tile, and ds_read_b64_tr_b16 reads it back
//    transposed as the B operand (8 keys of one column per lane).
//  * K/V stream through raw buffer loads with per-tile resources bounded at
//    the split's last key (rows past it read as zeros, so no clamping).  Each
//    wave keeps one tile in registers and issues the next tile's loads as
//    soon as it has consumed one; wave w takes tiles w, w + 8, ... (a fixed
//    order, so the result is the same on every call).
//  * The 8 waves' states merge after one barrier; each thread then writes 4
//    consecutive output d.  With several key splits the workgroup stores
//    its state at device scope and takes a ticket; the one that takes the
//    last ticket of its (batch, kv head) merges the splits (merge_last).
#include "qkv_internal.hpp"
#include "qkv_merge.hpp"
#include "qkv_mfma.hpp"
#include "qkv_quant_math.hpp"

namespace qkv {

namespace {

using namespace mf;

constexpr int NTK = 64;         // keys per tile (one per lane)
constexpr int NW = 8;           // waves per workgroup
constexpr int NTH = NW * 64;
constexpr float kLazy = 8.0f;                  // running-maximum slack (log2 units)
constexpr uint32_t kLazyBigScale = 0x5800u;    // fp16 128 = 2^(15 - kLazy)

// SA: the scale (and bias) rows are aligned to their size (up to 16 bytes),
// so a row is read in dwords; otherwise (possible only for the symmetric blocks, whose scale
// planes need 2-byte alignment) it is read in 16-bit pieces.
template <int MODE, int BITS, int GS, int D, bool MASK, int GP, bool SA, bool APPEND = false>
__global__ __launch_bounds__(NTH) void attn_decode_narrow(AttnLaunch p) {
    constexpr int NG = D / GS;
    constexpr int ROWB = D * BITS / 8;            // code bytes of a row
    constexpr int KWORDS = ROWB / 4;
    constexpr int QS = D / 4;                     // q K^T steps (4 d each)
    constexpr int NBANK = QS / 16;                // q registers pairs (16 steps each)
    constexpr int NT = D / 16;                    // P V output tiles
    constexpr int VB = D / 16 * BITS / 8;         // P V code bytes per lane and key
    constexpr int VW = VB >= 4 ? VB / 4 : 1;
    constexpr int SROWB = NG * 2;                 // bytes of a row of scales
    constexpr int NSW = SROWB >= 4 ? SROWB / 4 : 1;
    static_assert(NG <= 4 && NBANK >= 1, "narrow kernel: <= 4 groups, D >= 64");
    static_assert(GP * NG <= 16, "P' has 16 columns");
    static_assert(MODE != MODE_QSYM || (BITS == 4 && GS == 32), "symmetric blocks: 4-bit codes, blocks of 32");
    // symmetric codes: the nibbles' top bits flipped (c + 8) and the bias -8 d;
    // Q8_0: the bias of its sign-flipped codes (c + 128) is -128 d
    constexpr uint32_t kFlip = MODE == MODE_QSYM ? 0x88888888u : 0u;
    constexpr float kCodeBias = MODE == MODE_QSYM ? -8.0f : -128.0f;

    // Per-wave LDS: the P' rows of its tiles while it streams, then its
    // output state for the workgroup merge (a wave writes the latter only
    // after its last tile, and no other wave touches its P' rows).
    constexpr int WAVE_FLOATS = 64 * (D / 4) > NTK * 8 ? 64 * (D / 4) : NTK * 8;
    __shared__ __attribute__((aligned(16))) float s_wave[NW][WAVE_FLOATS];
    __shared__ float s_ml[NW][2][4];
    __shared__ bool s_last;                       // this workgroup merges the splits
    __shared__ float s_bias[NW][4][4];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int n = lane & 15;
    const int kb = lane >> 4;
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
    const float sl = p.scale * kLog2e;            // scores in log2 units

    const int64_t j0 = (int64_t)split * p.chunk;
    const int64_t j1 = min(p.L, j0 + p.chunk);
    const int ntiles = (int)((j1 - j0 + NTK - 1) / NTK);
    const int64_t jmax = j1 - 1;

    const int64_t krow0 = b * p.k.sb + kvh * p.k.sh;
    const int64_t vrow0 = b * p.v.sb + kvh * p.v.sh;
    const uint8_t* kc = (const uint8_t*)p.k.codes + krow0 * ROWB;
    const uint8_t* vc = (const uint8_t*)p.v.codes + vrow0 * ROWB;
    const uint8_t* ksc = (const uint8_t*)p.k.scales + krow0 * SROWB;
    const uint8_t* kbi = (const uint8_t*)p.k.biases + krow0 * SROWB;
    const uint8_t* vsc = (const uint8_t*)p.v.scales + vrow0 * SROWB;
    const uint8_t* vbi = (const uint8_t*)p.v.biases + vrow0 * SROWB;
    const uint32_t kcs = (uint32_t)(p.k.sl * ROWB), vcs = (uint32_t)(p.v.sl * ROWB);
    const uint32_t kss = (uint32_t)(p.k.sl * SROWB), vss = (uint32_t)(p.v.sl * SROWB);

    // ------------------------------------------------------------ queries
    // lane 4a + i holds, in bank c, head i's q at the 4 d of step 16c + a, in
    // the order the codes of that step are unpacked (odd 4-bit nibbles / 16)
    const int qi = lane & 3, qa = lane >> 2;
    const uint16_t* qrow = (const uint16_t*)p.q + (b * p.Hq + kvh * G + min(qi, G - 1)) * D;
    // every q load below is at a multiple of 16 (8-bit codes: 8) bytes from q
    const bool q_al16 = (reinterpret_cast<uintptr_t>(p.q) & 15) == 0;
    const bool q_al8 = (reinterpret_cast<uintptr_t>(p.q) & 7) == 0;
    auto step_d = [](int u, int e) -> int {       // d of half e of step u
        if constexpr (BITS == 4) {
            constexpr int o0[4] = {0, 4, 1, 5}, o1[4] = {2, 6, 3, 7};
            return 8 * (u >> 1) + ((u & 1) ? o1[e] : o0[e]);
        } else {
            constexpr int o[4] = {0, 2, 1, 3};
            return 4 * u + o[e];
        }
    };
    // raw q chunk of each bank (4-bit: the 8 d of the step's code dword,
    // 8-bit: its 4 d); the halves are picked after the tile loads are issued
    constexpr int QCH = BITS == 4 ? 4 : 2;        // dwords per chunk
    uint32_t qraw[NBANK][QCH];
#pragma unroll
    for (int c = 0; c < NBANK; ++c) {
        const int u = 16 * c + qa;
        const int d0 = BITS == 4 ? 8 * (u >> 1) : 4 * u;
        if constexpr (BITS == 4) {
            const uint4 x = load_h8(qrow + d0, q_al16);
            qraw[c][0] = x.x; qraw[c][1] = x.y; qraw[c][2] = x.z; qraw[c][3] = x.w;
        } else {
            const uint2 x = load_h4(qrow + d0, q_al8);
            qraw[c][0] = x.x; qraw[c][1] = x.y;
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ------------------------------------------------------------ K/V tiles
    struct Tile {
        uint32_t k[KWORDS];           // the lane's key row (q K^T)
        uint32_t ks[NSW], kbias[NSW]; // its scales / biases
        uint32_t vs[NSW], vbias[NSW]; // its value scales / biases (P' and the bias sums)
        uint32_t v[2][8][VW];         // P V codes: key 32 c + 8 kb + e, chunk n
    };
    const uint32_t o_k = (uint32_t)lane * kcs;
    const uint32_t o_ks = (uint32_t)lane * kss, o_vs = (uint32_t)lane * vss;
    const uint32_t o_v = (uint32_t)(8 * kb) * vcs + (uint32_t)n * VB;
    auto load_rows16 = [&](__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* dst) {
        if constexpr (NG == 1) {
            dst[0] = buf16(r, off);
        } else if constexpr (!SA) {
            uint32_t h[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) h[g] = buf16(r, off + 2 * g);
#pragma unroll
            for (int w = 0; w < NSW; ++w) dst[w] = h[2 * w] | (h[2 * w + 1] << 16);
        } else {
            bufn(r, off, dst, NSW);
        }
    };
    auto load_tile = [&](int tt, Tile& T) {
        const int64_t row0 = j0 + (int64_t)tt * NTK;
        const auto rk = rows_rsrc(kc, row0, j1, NTK, kcs, ROWB);
        bufn(rk, o_k, T.k, KWORDS);
        load_rows16(rows_rsrc(ksc, row0, j1, NTK, kss, SROWB), o_ks, T.ks);
        if constexpr (MODE == MODE_AFFINE)
            load_rows16(rows_rsrc(kbi, row0, j1, NTK, kss, SROWB), o_ks, T.kbias);
        load_rows16(rows_rsrc(vsc, row0, j1, NTK, vss, SROWB), o_vs, T.vs);
        if constexpr (MODE == MODE_AFFINE)
            load_rows16(rows_rsrc(vbi, row0, j1, NTK, vss, SROWB), o_vs, T.vbias);
        const auto rv = rows_rsrc(vc, row0, j1, NTK, vcs, ROWB);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t off = o_v + (uint32_t)(32 * c + e) * vcs;
                if constexpr (VB == 2) T.v[c][e][0] = buf16(rv, off);
                else bufn(rv, off, T.v[c][e], VW);
            }
    };
    // Decode with append: the new K/V token of this (batch, kv head) is pack
    // row L - 1, in the last tile of the last split.  The wave that loads
    // that tile first quantizes the two new rows with the quantize kernel's
    // arithmetic (qm::append_rows), writes them into the packs and waits for
    // its stores, so its load of the tile returns them.  No other workgroup
    // reads the row.
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
    // An opaque zero, defined after the tile loads (the memory clobber keeps
    // them ahead of it): the q arithmetic below depends on it, so the wait for
    // the q loads cannot be placed before the tile loads are issued.
    uint32_t after_loads;
    __asm__ __volatile__("s_mov_b32 %0, 0" : "=s"(after_loads) : : "memory");

    // q banks and the per-(head, group) sums of q (scale log2e applied)
    h4 qb[NBANK];
    float qs[4][NG];
    {
        float part[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) part[g] = 0.0f;
#pragma unroll
        for (int c = 0; c < NBANK; ++c) {
            _Float16 hv[4];
            const int u = 16 * c + qa;
            const int d0 = BITS == 4 ? 8 * (u >> 1) : 4 * u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int dd = step_d(u, e) - d0;       // 0 .. 2 QCH - 1
                uint32_t w = qraw[c][0];
#pragma unroll
                for (int k2 = 1; k2 < QCH; ++k2)
                    if ((dd >> 1) == k2) w = qraw[c][k2];
                w ^= after_loads;
                const _Float16 x = __builtin_bit_cast(_Float16, (uint16_t)((dd & 1) ? (w >> 16) : (w & 0xffffu)));
                part[d0 / GS] += (float)x;
                const bool sixteenth = BITS == 4 && e >= 2;
                hv[e] = qi < G ? (sixteenth ? x * (_Float16)0.0625f : x) : (_Float16)0.0f;
            }
            qb[c] = (h4){hv[0], hv[1], hv[2], hv[3]};
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            float s = part[g];
#pragma unroll
            for (int o = 4; o < 64; o <<= 1) s += __shfl_xor(s, o, 64);
#pragma unroll
            for (int h = 0; h < 4; ++h)
                qs[h][g] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), h)) * sl;
        }
    }

    // ------------------------------------------------------------ main loop
    f4 acc_o[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc_o[t] = f4{0.f, 0.f, 0.f, 0.f};
    float m_h[4], l_h[4], bs[4][NG];              // m uniform; l, bs per-lane partial sums
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        m_h[h] = -INFINITY;
        l_h[h] = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g) bs[h][g] = 0.0f;
    }
    _Float16* pw = (_Float16*)s_wave[wave];        // [key][16] P' rows
    const float kscale = 16777216.0f * sl;       // 2^24 undoes the subnormal code scale
    // P' column of this lane: (head ch, group cg); the column layout uses GP
    // (2 or 4) head slots per group, G <= GP of them real
    const int ch = n % GP;

    auto process = [&](const Tile& T, int tt) {
        const int64_t row0 = j0 + (int64_t)tt * NTK;
        // ---- q K^T: scores of key row0 + lane for the 4 heads
        f4 acc[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[g] = f4{0.f, 0.f, 0.f, 0.f};
        static_for<0, QS>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            uint32_t b0, b1;
            if constexpr (BITS == 4) {
                const uint32_t x = T.k[u >> 1] ^ kFlip;
                if constexpr (u & 1) {
                    const uint32_t t = perm_b(0u, x, 0x0C030C01u);
                    b0 = t & 0x000F000Fu;
                    b1 = t & 0x00F000F0u;
                } else {
                    b0 = x & 0x000F000Fu;
                    b1 = x & 0x00F000F0u;
                }
            } else {
                const uint32_t f = MODE == MODE_Q8_0 ? 0x00800080u : 0u;
                const uint32_t x = T.k[u];
                b0 = (x & 0x00FF00FFu) ^ f;
                b1 = perm_b(0u, x, 0x0C030C01u) ^ f;
            }
            constexpr int g = (BITS == 4 ? 8 * (u >> 1) : 4 * u) / GS;
            acc[g] = mfma4_bcast<u & 15>(qb[u >> 4], to_h4(b0, b1), acc[g]);
        });
        float z[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) z[h] = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const uint32_t sw = T.ks[g >> 1];
            const float s = (g & 1) ? hi_f16(sw) : lo_f16(sw);
            const float S = s * kscale;
            if constexpr (MODE == MODE_AFFINE) {
                const uint32_t bw = T.kbias[g >> 1];
                const float bb = (g & 1) ? hi_f16(bw) : lo_f16(bw);
#pragma unroll
                for (int h = 0; h < 4; ++h) z[h] = __builtin_fmaf(bb, qs[h][g], __builtin_fmaf(acc[g][h], S, z[h]));
            } else {
                const float Tq = kCodeBias * s;
#pragma unroll
                for (int h = 0; h < 4; ++h) z[h] = __builtin_fmaf(Tq, qs[h][g], __builtin_fmaf(acc[g][h], S, z[h]));
            }
        }
        const int64_t j = row0 + lane;
        if (row0 + NTK - 1 > jmax) {              // tile crosses the end of the split
            if (j > jmax) {
#pragma unroll
                for (int h = 0; h < 4; ++h) z[h] = -INFINITY;
            }
        }
        if constexpr (MASK) {
            if (j <= jmax) {
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    if (h < G)
                        z[h] += kLog2e * load_mask(p.mask, p.mask_dtype,
                                                   b * p.ms0 + (kvh * G + h) * p.ms1 + j * p.ms3);
            }
        }
#pragma unroll
        for (int h = 0; h < 4; ++h)
            if (h >= G) z[h] = -INFINITY;

        // ---- online softmax, lazy maximum: the running maximum is raised only
        // when a score exceeds it by kLazy (log2 units), so p = 2^(z - m) <= 2^kLazy
        // and P' = p s_v stays in fp16 range for |s_v| < 2^(15 - kLazy); a key with
        // a larger value scale raises it as soon as its score exceeds it
        bool big_sv = false;
#pragma unroll
        for (int q = 0; q < NSW; ++q) {
            const uint32_t a = T.vs[q] & 0x7FFF7FFFu;
            big_sv |= (a & 0xFFFFu) >= kLazyBigScale || (a >> 16) >= kLazyBigScale;
        }
        const float slack = big_sv ? 0.0f : kLazy;
        bool grow = false;
#pragma unroll
        for (int h = 0; h < 4; ++h) grow |= z[h] > m_h[h] + slack;
        if (__ballot(grow) != 0ull) {
            float alpha[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float mn = fmaxf(m_h[h], wave_max(z[h]));
                alpha[h] = (m_h[h] == -INFINITY) ? 0.0f : fast_exp2(m_h[h] - mn);
                m_h[h] = mn;
                l_h[h] *= alpha[h];
#pragma unroll
                for (int g = 0; g < NG; ++g) bs[h][g] *= alpha[h];
            }
            const float ac = ch == 0 ? alpha[0] : ch == 1 ? alpha[1] : ch == 2 ? alpha[2] : alpha[3];
#pragma unroll
            for (int t = 0; t < NT; ++t) acc_o[t] *= ac;
        }
        float pr[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            pr[h] = m_h[h] == -INFINITY ? 0.0f : fast_exp2(z[h] - m_h[h]);
            l_h[h] += pr[h];
        }
        // ---- P' row of this key (column h + G g = p_h s_g) and the bias sums
        _Float16 prow[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) prow[q] = (_Float16)0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const uint32_t sw = T.vs[g >> 1];
            const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)((g & 1) ? (sw >> 16) : (sw & 0xffffu)));
            float bv;
            if constexpr (MODE == MODE_AFFINE) {
                const uint32_t bw = T.vbias[g >> 1];
                bv = (g & 1) ? hi_f16(bw) : lo_f16(bw);
            } else {
                bv = kCodeBias * (float)sv;
            }
#pragma unroll
            for (int h = 0; h < GP; ++h) prow[h + GP * g] = (_Float16)pr[h] * sv;
#pragma unroll
            for (int h = 0; h < 4; ++h) bs[h][g] = __builtin_fmaf(pr[h], bv, bs[h][g]);
        }
        {
            uint32_t w[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                w[q] = (uint32_t)__builtin_bit_cast(uint16_t, prow[2 * q]) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, prow[2 * q + 1]) << 16);
            uint4* dst = (uint4*)(pw + lane * 16);
            dst[0] = uint4{w[0], w[1], w[2], w[3]};
            dst[1] = uint4{w[4], w[5], w[6], w[7]};
        }
        lds_order();
        // ---- P V: two 32-key steps; B = P'^T by the LDS transpose read
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int k0 = 32 * c + 8 * kb;
            const _Float16* pa = pw + (k0 + (n >> 2)) * 16 + 4 * (n & 3);
            const s4 ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(pa));
            const s4 rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(pa + 4 * 16));
            const h8 pop = __builtin_bit_cast(h8, (short __attribute__((ext_vector_type(8)))){
                ra[0], ra[1], ra[2], ra[3], rb[0], rb[1], rb[2], rb[3]});
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                uint32_t a[4];
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) {
                    uint32_t x;
                    if constexpr (MODE == MODE_QSYM) {
                        uint32_t wa[VW], wb[VW];
#pragma unroll
                        for (int i = 0; i < VW; ++i) {
                            wa[i] = T.v[c][2 * q2][i] ^ kFlip;
                            wb[i] = T.v[c][2 * q2 + 1][i] ^ kFlip;
                        }
                        x = pair_sub_byte<BITS>(wa, wb, t);
                    } else {
                        x = pair_sub_byte<BITS>(T.v[c][2 * q2], T.v[c][2 * q2 + 1], t);
                    }
                    if constexpr (MODE == MODE_Q8_0) x ^= 0x00800080u;
                    a[q2] = x;
                }
                acc_o[t] = mfma16(to_h8(a[0], a[1], a[2], a[3]), pop, acc_o[t]);
            }
        }
        lds_order();
    };

    // One register tile per wave: the next tile's loads are issued as soon as
    // a tile is consumed.  Deeper register rings measured slower (with every
    // CU streaming they only lengthen the memory queues; 64K-context 4-bit
    // decode with this loop: 2 tiles 24.5 us, 1 tile 22.5 us per call).  Wave
    // w takes tiles w, w + NW, ...: with tiles handed out by an LDS counter
    // the partition (and so the rounding) changed from call to call, for no
    // measurable gain.
    int tt = wave;
    while (tt < ntiles) {
        const int nxt = tt + NW;
        process(cur, tt);
        __builtin_amdgcn_sched_barrier(0);
        // no loads after the last tile: they would hold the wave (and the
        // workgroup merge behind it) until the CU's memory queue drains
        if (nxt < ntiles) {
            if (append_here(nxt)) append_row();
            load_tile(nxt, cur);
        }
        __builtin_amdgcn_sched_barrier(0);
        tt = nxt;
    }

    // ------------------------------------------------------------ merge waves
    // Every wave leaves its unscaled state in LDS; after one barrier each
    // thread combines the 8 waves' states for its output elements (a single
    // synchronisation: the tail after the slowest wave stays short).
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        l_h[h] = wave_sum(l_h[h]);
#pragma unroll
        for (int g = 0; g < NG; ++g) bs[h][g] = wave_sum(bs[h][g]);
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            s_ml[wave][0][h] = m_h[h];
            s_ml[wave][1][h] = l_h[h];
#pragma unroll
            for (int g = 0; g < NG; ++g) s_bias[wave][h][g] = bs[h][g];
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) *(f4*)&s_wave[wave][(t * 64 + lane) * 4] = acc_o[t];   // [t][lane][4]
    __syncthreads();

    // ------------------------------------------------------------ output
    // Item -> (jj, head oh, kbb, tc), jj fastest: the P V values of the 4
    // consecutive d = DPT (4 kbb + jj) + 4 tc + 0..3 sit in lane
    // 16 kbb + (oh + GP g), register jj, of tiles 4 tc .. 4 tc + 3
    // (DPT = D / 16).  The 4 lanes of a quad share an item: lane 'sub' of the
    // quad combines waves sub and sub + 4, and two quad exchanges add the
    // lanes' sums in a fixed order.  Consecutive quads read consecutive LDS
    // words; each item is one 16-byte (or 8-byte) store.
    constexpr int DPT = D / 16;
    static_assert(DPT % 4 == 0, "4 consecutive d per output item");
    static_assert(NW == 8, "two waves per quad lane");
    // with several splits: this split's state, stored at device scope for the
    // fused merge ([16 rows][D] o and [16 rows][2] (m, l); rows = heads)
    const auto rml = flat_rsrc(p.part_ml + (bk * p.S + split) * 32, 32 * 4);
    const auto rpo = flat_rsrc(p.part_o + (bk * p.S + split) * 16 * D, 16 * D * 4);
    const int64_t obase = (b * p.Hq + kvh * G) * D;
    for (int i = tid; i < G * D; i += NTH) {          // G D is a multiple of 4: whole quads
        const int sub = i & 3;
        const int item = i >> 2;
        const int jj = item & 3;
        const int oh = (item >> 2) % G;
        const int rest = (item >> 2) / G;
        const int kbb = rest & 3, tc = rest >> 2;
        const int d0 = DPT * (4 * kbb + jj) + 4 * tc;
        const int g = d0 / GS;                        // 4 consecutive d share a group
        const int w0 = sub, w1 = sub + 4;
        const float m0 = s_ml[w0][0][oh], m1 = s_ml[w1][0][oh];
        float Mh = fmaxf(m0, m1);
        Mh = fmaxf(Mh, dpp_f<0xB1>(Mh));
        Mh = fmaxf(Mh, dpp_f<0x4E>(Mh));
        const float f0 = (m0 == -INFINITY) ? 0.0f : fast_exp2(m0 - Mh);
        const float f1 = (m1 == -INFINITY) ? 0.0f : fast_exp2(m1 - Mh);
        float part[6];
        part[4] = f0 * s_ml[w0][1][oh] + f1 * s_ml[w1][1][oh];
        part[5] = f0 * s_bias[w0][oh][g] + f1 * s_bias[w1][oh][g];
        const int slot = (kbb * 16 + oh + GP * g) * 4 + jj;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            part[q] = f0 * s_wave[w0][(4 * tc + q) * 256 + slot] + f1 * s_wave[w1][(4 * tc + q) * 256 + slot];
#pragma unroll
        for (int k = 0; k < 6; ++k) {
            part[k] += dpp_f<0xB1>(part[k]);          // quad_perm [1, 0, 3, 2]
            part[k] += dpp_f<0x4E>(part[k]);          // quad_perm [2, 3, 0, 1]
        }
        if (sub != 0) continue;
        const float Lh = part[4], bias = part[5];
        float o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // 4-bit odd d: the tile of its code's whole byte minus the even d's tile
            const float x = (BITS == 4 && (q & 1)) ? (part[q] - part[q - 1]) * 0.0625f : part[q];
            o[q] = x * 16777216.0f + bias;
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
            const u4 ov = {__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                           __float_as_uint(o[3])};
            __builtin_amdgcn_raw_buffer_store_b128(ov, rpo, (oh * D + d0) * 4, 0, kScopeDevice);
            if (d0 == 0) {
                const u2 mv = {__float_as_uint(Mh), __float_as_uint(Lh)};
                __builtin_amdgcn_raw_buffer_store_b64(mv, rml, 2 * oh * 4, 0, kScopeDevice);
            }
        }
    }
    if (p.S == 1) return;

    // ------------------------------------------------------------ fused split merge
    // The workgroup's state stores are complete (device scope) before its
    // ticket; the workgroup that takes the last ticket of this (batch, kv head)
    // combines the S states (all stored before their tickets) and writes out.
    wait_stores();
    __syncthreads();
    if (tid == 0) s_last = take_last_ticket(p.tickets + bk, p.S);
    __syncthreads();
    if (!s_last) return;
    merge_last<NTH, D, GP>(p, b, kvh, bk, &s_wave[0][0]);
}

template <int MODE, int BITS, int GS, int D, int GP>
hipError_t launch_g(int64_t B, const AttnLaunch& p, hipStream_t stream) {
    dim3 grid(p.S, (unsigned)p.Hk, (unsigned)B);
    constexpr int SROWB = D / GS * 2;
    constexpr uintptr_t kAlign = (SROWB >= 16 ? 16 : SROWB) - 1;   // a scale row's own alignment
    const bool sa = SROWB < 4 ||
                    ((reinterpret_cast<uintptr_t>(p.k.scales) | reinterpret_cast<uintptr_t>(p.v.scales)) & kAlign) == 0;
    if constexpr (MODE == MODE_QSYM) {
        if (!sa) {
            if (p.mask_kind == MASK_ADDITIVE)
                hipLaunchKernelGGL((attn_decode_narrow<MODE, BITS, GS, D, true, GP, false>), grid, dim3(NTH), 0, stream, p);
            else
                hipLaunchKernelGGL((attn_decode_narrow<MODE, BITS, GS, D, false, GP, false>), grid, dim3(NTH), 0, stream, p);
            return hipGetLastError();
        }
    } else if (!sa) {
        return hipErrorInvalidValue;               // the host checks guarantee aligned rows
    }
    if (p.append) {
        // the decode with append: affine and Q8_0 codes, no additive mask
        if constexpr (MODE == MODE_AFFINE || MODE == MODE_Q8_0) {
            if (p.mask_kind == MASK_ADDITIVE) return hipErrorNotSupported;
            hipLaunchKernelGGL((attn_decode_narrow<MODE, BITS, GS, D, false, GP, true, true>), grid, dim3(NTH), 0,
                               stream, p);
            return hipGetLastError();
        } else {
            return hipErrorNotSupported;
        }
    }
    if (p.mask_kind == MASK_ADDITIVE)
        hipLaunchKernelGGL((attn_decode_narrow<MODE, BITS, GS, D, true, GP, true>), grid, dim3(NTH), 0, stream, p);
    else
        hipLaunchKernelGGL((attn_decode_narrow<MODE, BITS, GS, D, false, GP, true>), grid, dim3(NTH), 0, stream, p);
    return hipGetLastError();
}

template <int MODE, int BITS, int GS, int D>
hipError_t launch_n(int64_t B, const AttnLaunch& p, hipStream_t stream) {
    if (p.G <= 2) return launch_g<MODE, BITS, GS, D, 2>(B, p, stream);
    return launch_g<MODE, BITS, GS, D, 4>(B, p, stream);
}

// The instantiated shapes: D <= 128, and 8-bit codes with at most 2 groups
// per row (larger rows exceed the register budget of one tile).
template <int BITS, int GS, int D>
constexpr bool narrow_shape() {
    return D <= 128 && D % GS == 0 && D / GS <= 4 && (BITS == 4 || D / GS <= 2);
}

template <int MODE, int BITS, int GS>
hipError_t by_d(int D, int64_t B, const AttnLaunch& p, hipStream_t s) {
    switch (D) {
        case 64: if constexpr (narrow_shape<BITS, GS, 64>()) return launch_n<MODE, BITS, GS, 64>(B, p, s); else break;
        case 128: if constexpr (narrow_shape<BITS, GS, 128>()) return launch_n<MODE, BITS, GS, 128>(B, p, s); else break;
    }
    return hipErrorNotSupported;
}

}  // namespace

bool narrow_decode_supported(int q_dtype, int mode, int bits, int group_size, int D, int G,
                             int64_t Lq) {
    if (q_dtype != DT_F16 || Lq != 1 || G < 1 || G > 4) return false;
    if (D != 64 && D != 128) return false;
    if (mode == MODE_QSYM) return bits == 4 && group_size == 32;
    if (!fast_format(mode, bits, D)) return false;
    const int gs = mode == MODE_Q8_0 ? 32 : group_size;
    if (mode == MODE_AFFINE && (bits != 4 && bits != 8)) return false;
    if (gs != 32 && gs != 64 && gs != 128) return false;
    if (D % gs) return false;
    const int ng = D / gs;
    return ng <= 4 && (bits == 4 || ng <= 2);
}

// Splits are whole tiles, not whole rounds of the 8 waves: with a key count
// that is not a multiple of 8 tiles per split the spare tiles fall to the
// first waves of every workgroup, instead of a shorter last split idling the
// XCDs that hold it (16,448 keys in 4 splits: 65/65/65/62 tiles against
// 72/72/72/41).
int narrow_decode_key_quantum() { return NTK; }

hipError_t launch_attn_narrow(int mode, int bits, int D, int64_t B, const AttnLaunch& p,
                              hipStream_t stream) {
    const int gs = 1 << p.gs_log2;
    if (mode == MODE_Q8_0) return by_d<MODE_Q8_0, 8, 32>(D, B, p, stream);
    if (mode == MODE_QSYM) return bits == 4 && gs == 32 ? by_d<MODE_QSYM, 4, 32>(D, B, p, stream) : hipErrorNotSupported;
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
