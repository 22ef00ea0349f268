// C-ABI entry points of libqkv.so (declared in include/qkv.h): argument
// validation, kernel selection and launch on the caller's stream.  Every check
// runs before anything is enqueued, so a non-OK status leaves all buffers
// untouched.  The library never allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/qkv.h"
#include "../../include/qkv_measure.h"
#include "qkv_internal.hpp"

namespace qkv {
// Plain streaming read of a device buffer (qkv_measure.hip).
hipError_t launch_measure_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink,
                               hipStream_t stream);
hipError_t launch_measure_read_config(const void* buf, size_t bytes, int workgroups, int threads, int in_flight,
                                      int width, uint32_t* sink, hipStream_t stream);
}  // namespace qkv
#include "qkv_merge.hpp"

static_assert(QKV_TICKET_BYTES == qkv::kTicketBytes, "ticket header size of the ABI");

namespace {

thread_local std::string g_last_error;

qkv_status fail(qkv_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

qkv_status ok() {
    g_last_error.clear();
    return QKV_OK;
}

qkv_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(QKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_dtype(int32_t d) { return d == QKV_F32 || d == QKV_F16 || d == QKV_BF16; }
size_t dtype_size(int32_t d) { return d == QKV_F32 ? 4 : 2; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int ilog2(int v) {
    int r = 0;
    while ((1 << r) < v) ++r;
    return r;
}

// Byte extent of a pack's rows (for overlap checks).
struct Range {
    uintptr_t lo, hi;
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int64_t max_row(const qkv_pack* p) {
    return (p->B - 1) * p->stride_b + (p->H - 1) * p->stride_h + (p->L_cap - 1) * p->stride_l;
}
int64_t row_bytes(const qkv_pack* p) { return p->D * p->bits / 8; }
int64_t groups_per_row(const qkv_pack* p) { return p->D / p->group_size; }

Range codes_range(const qkv_pack* p) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p->codes);
    return {lo, lo + (uintptr_t)((max_row(p) + 1) * row_bytes(p))};
}
Range scales_range(const qkv_pack* p, const void* base) {
    if (!base) return {0, 0};
    uintptr_t lo = reinterpret_cast<uintptr_t>(base);
    return {lo, lo + (uintptr_t)((max_row(p) + 1) * groups_per_row(p) * dtype_size(p->scale_dtype))};
}

qkv_status check_pack(const qkv_pack* p, const char* name) {
    if (!p) return fail(QKV_EINVAL, "%s: null pack", name);
    if (p->mode != QKV_AFFINE && p->mode != QKV_Q8_0 && p->mode != QKV_DENSE && p->mode != QKV_QSYM)
        return fail(QKV_EINVAL, "%s: unknown mode %d", name, p->mode);
    if (p->B < 1 || p->H < 1 || p->L_cap < 1 || p->D < 1)
        return fail(QKV_EINVAL, "%s: B, H, L_cap and D must be >= 1", name);
    if (p->stride_b < 0 || p->stride_h < 0 || p->stride_l < 0)
        return fail(QKV_EINVAL, "%s: negative stride", name);
    if (!p->codes) return fail(QKV_EINVAL, "%s: null codes", name);
    if (p->mode == QKV_DENSE) {
        if (p->bits != 16 || p->scale_dtype != QKV_F16 || p->group_size != p->D)
            return fail(QKV_EINVAL, "%s: a dense pack holds fp16 values (bits 16, group_size D, scale dtype fp16)",
                        name);
        if (p->scales || p->biases) return fail(QKV_EINVAL, "%s: a dense pack takes no scales or biases", name);
        if (p->D != 64 && p->D != 128 && p->D != 256)
            return fail(QKV_EUNSUPPORTED, "%s: head size D=%lld not in {64, 128, 256}", name, (long long)p->D);
        if (!aligned(p->codes, 16)) return fail(QKV_EINVAL, "%s: codes not 16-byte aligned", name);
        return QKV_OK;
    }
    if (!p->scales) return fail(QKV_EINVAL, "%s: null scales", name);
    if (p->mode == QKV_AFFINE) {
        if (p->bits != 2 && p->bits != 3 && p->bits != 4 && p->bits != 5 && p->bits != 6 && p->bits != 8)
            return fail(QKV_EUNSUPPORTED, "%s: bits %d not in {2, 3, 4, 5, 6, 8}", name, p->bits);
        if (p->group_size != 32 && p->group_size != 64 && p->group_size != 128)
            return fail(QKV_EUNSUPPORTED, "%s: group_size %d not in {32, 64, 128}", name, p->group_size);
        if (p->D % p->group_size)
            return fail(QKV_EINVAL, "%s: D=%lld is not a multiple of group_size=%d", name,
                        (long long)p->D, p->group_size);
        if (!valid_dtype(p->scale_dtype)) return fail(QKV_EINVAL, "%s: bad scale dtype", name);
        if (!p->biases) return fail(QKV_EINVAL, "%s: affine pack needs biases", name);
    } else if (p->mode == QKV_QSYM) {
        if ((p->bits != 4 && p->bits != 5) || p->group_size != 32)
            return fail(QKV_EINVAL, "%s: symmetric blocks need bits 4 or 5, group_size 32", name);
        if (p->scale_dtype != QKV_F16) return fail(QKV_EINVAL, "%s: symmetric block scales are fp16", name);
        if (p->biases) return fail(QKV_EINVAL, "%s: symmetric blocks take no biases", name);
        if (p->D % 32) return fail(QKV_EINVAL, "%s: D must be a multiple of 32", name);
    } else {
        if (p->bits != 8 || p->group_size != 32)
            return fail(QKV_EINVAL, "%s: Q8_0 needs bits=8, group_size=32", name);
        if (p->scale_dtype != QKV_F16) return fail(QKV_EINVAL, "%s: Q8_0 scales are fp16", name);
        if (p->biases) return fail(QKV_EINVAL, "%s: Q8_0 pack takes no biases", name);
        if (p->D % 32) return fail(QKV_EINVAL, "%s: D must be a multiple of 32", name);
    }
    if (p->D != 64 && p->D != 96 && p->D != 128 && p->D != 256)
        return fail(QKV_EUNSUPPORTED, "%s: head size D=%lld not in {64, 96, 128, 256}", name, (long long)p->D);
    if (!aligned(p->codes, 16)) return fail(QKV_EINVAL, "%s: codes not 16-byte aligned", name);
    // scale and bias planes: for the matrix-core formats aligned to one row of
    // them (up to 16 bytes), the width of those kernels' row loads; the
    // general paths read them one element at a time
    const size_t ss = dtype_size(p->scale_dtype);
    const size_t ra = qkv::fast_format(p->mode, p->bits, (int)p->D)
                          ? std::min<size_t>(16, (size_t)(p->D / p->group_size) * ss) : ss;
    if (!aligned(p->scales, ra) || (p->biases && !aligned(p->biases, ra)))
        return fail(QKV_EINVAL, "%s: scales/biases misaligned (need %zu-byte alignment)", name, ra);
    return QKV_OK;
}

bool same_format(const qkv_pack* a, const qkv_pack* b) {
    return a->mode == b->mode && a->bits == b->bits && a->group_size == b->group_size &&
           a->scale_dtype == b->scale_dtype && a->B == b->B && a->H == b->H && a->D == b->D;
}

qkv::QuantJob make_job(const void* x, const int64_t xs[3], const qkv_pack* p) {
    qkv::QuantJob j;
    j.x = x;
    j.xs0 = xs[0];
    j.xs1 = xs[1];
    j.xs2 = xs[2];
    j.codes = p->codes;
    j.scales = p->scales;
    j.biases = p->biases;
    j.sb = p->stride_b;
    j.sh = p->stride_h;
    j.sl = p->stride_l;
    return j;
}

qkv_status check_source(const void* x, int32_t dtype, const int64_t xs[3], const qkv_pack* p,
                        const char* name) {
    if (!x) return fail(QKV_EINVAL, "%s: null source", name);
    if (!valid_dtype(dtype)) return fail(QKV_EINVAL, "%s: bad dtype %d", name, dtype);
    if (!xs) return fail(QKV_EINVAL, "%s: null strides", name);
    for (int i = 0; i < 3; ++i)
        if (xs[i] < 0 || xs[i] % 8) return fail(QKV_EINVAL, "%s: strides must be >= 0 and multiples of 8", name);
    if (!aligned(x, 16)) return fail(QKV_EINVAL, "%s: source not 16-byte aligned", name);
    if (p->mode == QKV_AFFINE && dtype != p->scale_dtype)
        return fail(QKV_EUNSUPPORTED, "%s: affine scale dtype must equal the source dtype", name);
    if (p->mode == QKV_DENSE && dtype != QKV_F16)
        return fail(QKV_EUNSUPPORTED, "%s: a dense pack takes fp16 values", name);
    return QKV_OK;
}

// The quantize kernels address a pass of rows with 32-bit offsets from a
// per-pass base: a source row stride and a pack row stride below 2^27 bytes.
qkv_status check_row_strides(const int64_t xs[3], int32_t dtype, const qkv_pack* p, const char* name) {
    const int64_t lim = int64_t(1) << 27;
    if (xs[2] * (int64_t)dtype_size(dtype) >= lim || p->stride_l * row_bytes(p) >= lim)
        return fail(QKV_EUNSUPPORTED, "%s: a row stride of 2^27 bytes or more is not supported", name);
    return QKV_OK;
}

// One append of T new K/V tokens at row offset (qkv_update_append's checks).
qkv_status check_append(const char* name, const void* k_new, const void* v_new, int32_t dtype,
                        const int64_t new_strides[3], int64_t T, int64_t offset, const qkv_pack* k_cache,
                        const qkv_pack* v_cache) {
    qkv_status st;
    if ((st = check_pack(k_cache, name)) != QKV_OK) return st;
    if ((st = check_pack(v_cache, name)) != QKV_OK) return st;
    if (!same_format(k_cache, v_cache)) return fail(QKV_EINVAL, "%s: K and V packs differ in format or shape", name);
    if ((st = check_source(k_new, dtype, new_strides, k_cache, name)) != QKV_OK) return st;
    if ((st = check_source(v_new, dtype, new_strides, v_cache, name)) != QKV_OK) return st;
    if (T < 1) return fail(QKV_EINVAL, "%s: T must be >= 1", name);
    if (offset < 0 || offset + T > k_cache->L_cap || offset + T > v_cache->L_cap)
        return fail(QKV_EINVAL, "%s: rows [%lld, %lld) exceed the capacity", name, (long long)offset,
                    (long long)(offset + T));
    if (overlap(codes_range(k_cache), codes_range(v_cache)))
        return fail(QKV_EINVAL, "%s: K and V codes overlap", name);
    if ((st = check_row_strides(new_strides, dtype, k_cache, name)) != QKV_OK) return st;
    if ((st = check_row_strides(new_strides, dtype, v_cache, name)) != QKV_OK) return st;
    return QKV_OK;
}

qkv::QuantLaunch append_launch(const void* k_new, const void* v_new, const int64_t new_strides[3], int64_t T,
                               int64_t offset, const qkv_pack* k_cache, const qkv_pack* v_cache) {
    qkv::QuantLaunch p{};
    p.job[0] = make_job(k_new, new_strides, k_cache);
    p.job[1] = make_job(v_new, new_strides, v_cache);
    p.H = k_cache->H;
    p.T = T;
    p.offset = offset;
    p.BH = k_cache->B * k_cache->H;
    p.rows = p.BH * T;
    return p;
}

// The new token of a decode with append (one row per (batch, kv head), in the
// query dtype, written at row L - 1 before the decode attends rows [0, L)).
struct AppendArgs {
    const void* k_new;
    const void* v_new;
    const int64_t* strides;
};

// ---------------------------------------------------------------- attention plans
struct Plan {
    bool unfused;                   // the four-kernel composition (QKV_ALGO_UNFUSED)
    bool prepass;                   // dense fp16 copies first (QKV_ALGO_DEQUANT_F16)
    size_t dense_bytes;             // bytes of each dense copy in the workspace
    bool matrix;
    bool prefill;                   // tiled matrix kernel
    int wg_rows;                    // its rows per workgroup
    bool narrow;                    // single-query kernel for GQA factors <= 4
    bool stream;                    // single-query VALU kernel for the bit-stream formats
    int RT, n_rt, S;
    int64_t chunk;
    size_t ws_bytes;
};

size_t ws_for(int64_t B, int64_t Hk, int n_rt, int S, int RT, int64_t D) {
    if (S <= 1) return 0;
    return qkv::kTicketBytes +
           (size_t)(B * Hk * n_rt) * (size_t)S * (size_t)RT * (size_t)(D + 2) * 4;  // ml + o
}

// Element extent [lo, hi) of a strided 4-d view in bytes.
Range strided_range(const void* base, size_t esize, const int64_t n[4], const int64_t st[4]) {
    int64_t last = 0;
    for (int i = 0; i < 4; ++i) last += (n[i] - 1) * st[i];
    uintptr_t lo = reinterpret_cast<uintptr_t>(base);
    return {lo, lo + (uintptr_t)((last + 1) * (int64_t)esize)};
}

bool overlaps_pack(Range r, const qkv_pack* p) {
    return overlap(r, codes_range(p)) || overlap(r, scales_range(p, p->scales)) ||
           (p->biases && overlap(r, scales_range(p, p->biases)));
}

size_t unfused_scores_bytes(int64_t B, int64_t Hq, int64_t L) {
    return ((size_t)(B * Hq * L) * 4 + 255) / 256 * 256;
}
size_t unfused_stats_bytes(int64_t B, int64_t Hq, int64_t L) {
    return ((size_t)qkv::unfused_stats_floats(B, Hq, L) * 4 + 255) / 256 * 256;
}

// Split count: enough workgroups to cover the CUs about twice, each split at
// least min_keys long, and at most kMaxSplits (the merge keeps per-split
// weights in LDS).
int auto_splits(int64_t base_wgs, int64_t L, int64_t min_keys, int64_t target) {
    int64_t want = (target + base_wgs - 1) / base_wgs;
    int64_t cap = std::max<int64_t>(1, L / min_keys);
    return (int)std::max<int64_t>(1, std::min<int64_t>({want, cap, 256}));
}

qkv::DequantLaunch dequant_job(const qkv_pack* src, const qkv_pack* dst, int64_t L) {
    qkv::DequantLaunch j{};
    j.codes = src->codes;
    j.scales = src->scales;
    j.biases = src->biases;
    j.sb = src->stride_b;
    j.sh = src->stride_h;
    j.sl = src->stride_l;
    j.out = dst->codes;
    j.db = dst->stride_b;
    j.dh = dst->stride_h;
    j.dl = dst->stride_l;
    j.H = src->H;
    j.L = L;
    j.rows = src->B * src->H * L;
    j.gs = src->mode == QKV_Q8_0 ? 32 : src->group_size;
    return j;
}

// A dense fp16 pack of rows [0, L) of every (b, h) of k at 'codes' (the
// dequantize-first strategy's copies).
qkv_pack dense_copy_of(const qkv_pack* k, int64_t L, void* codes) {
    qkv_pack d{};
    d.mode = QKV_DENSE;
    d.bits = 16;
    d.group_size = (int32_t)k->D;
    d.scale_dtype = QKV_F16;
    d.B = k->B;
    d.H = k->H;
    d.L_cap = L;
    d.D = k->D;
    d.codes = codes;
    d.stride_b = k->H * L;
    d.stride_h = L;
    d.stride_l = 1;
    return d;
}

size_t dense_copy_bytes(const qkv_pack* k, int64_t L) {
    return ((size_t)(k->B * k->H * L * k->D) * 2 + 255) / 256 * 256;
}

Plan make_plan(int64_t B, int64_t Hq, int64_t Lq, int64_t D, int64_t L, const qkv_pack* k,
               int32_t q_dtype, const qkv_attn_opts* opts) {
    if (opts && opts->algo == QKV_ALGO_DEQUANT_F16) {
        // the dense plan over the copies, after them in the workspace
        const qkv_pack d = dense_copy_of(k, L, nullptr);
        qkv_attn_opts o2 = *opts;
        o2.algo = QKV_ALGO_AUTO;
        Plan pl = make_plan(B, Hq, Lq, D, L, &d, q_dtype, &o2);
        pl.prepass = true;
        pl.dense_bytes = dense_copy_bytes(k, L);
        pl.ws_bytes += 2 * pl.dense_bytes;
        return pl;
    }
    Plan pl{};
    const int64_t Hk = k->H;
    const int G = (int)(Hq / Hk);
    const int algo = opts ? opts->algo : QKV_ALGO_AUTO;
    const int bits = k->bits;
    if (algo == QKV_ALGO_UNFUSED) {
        // scores [B Hq][L], then the P V sums of every key chunk
        pl.unfused = true;
        pl.RT = 16;
        pl.n_rt = 1;
        pl.wg_rows = 0;
        pl.chunk = qkv::unfused_chunk_keys(B, Hk, L, G);
        pl.S = (int)((L + pl.chunk - 1) / pl.chunk);
        pl.ws_bytes = unfused_scores_bytes(B, Hq, L) + unfused_stats_bytes(B, Hq, L) +
                      (size_t)pl.S * (size_t)(B * Hq * D) * 4;
        return pl;
    }
    pl.matrix = false;
    pl.prefill = false;
    pl.narrow = false;
    pl.stream = false;
    // the matrix kernels address a kv head's rows with 32-bit offsets
    const int64_t span = (k->L_cap - 1) * k->stride_l * row_bytes(k) + row_bytes(k);
    // the narrow decode also takes the symmetric 4-bit blocks, which the
    // other matrix kernels do not
    const bool narrow_ok = qkv::narrow_decode_supported(q_dtype, k->mode, bits, k->group_size, (int)D, G, Lq);
    if (algo != QKV_ALGO_GENERIC && span < (int64_t(1) << 31) &&
        (narrow_ok || qkv::matrix_supported(q_dtype, k->mode, bits, k->group_size, (int)D, G, Lq))) {
        pl.matrix = true;
        pl.narrow = narrow_ok;
        pl.prefill = !pl.narrow &&
                     !qkv::decode_matrix_supported(q_dtype, k->mode, bits, k->group_size, (int)D, G, Lq);
    }
    if (!pl.matrix && algo != QKV_ALGO_GENERIC && algo != QKV_ALGO_MATRIX && span < (int64_t(1) << 31) &&
        qkv::stream_decode_supported(q_dtype, k->mode, bits, k->group_size, k->scale_dtype, (int)D, G, Lq))
        pl.stream = true;
    const int64_t n_rows = (int64_t)G * Lq;
    pl.wg_rows = n_rows >= qkv::kPrefillWideMinRows ? qkv::kPrefillRowsWide : qkv::kPrefillRows;
    if (pl.prefill) {
        // grid rows (row tiles) and (batch, kv head) pairs within the y/z grid limits
        const int64_t tiles = (n_rows + pl.wg_rows - 1) / pl.wg_rows;
        if (tiles > 65535 || B * Hk > 65535) pl.matrix = pl.prefill = false;
    }
    pl.RT = 16;
    pl.n_rt = (int)((n_rows + pl.RT - 1) / pl.RT);
    int S;
    if (opts && opts->num_splits > 0) {
        S = std::min(opts->num_splits, 256);
    } else if (pl.prefill && Lq == 1) {
        // a decode on the tiled kernel (dense caches, GQA beyond 16): it streams
        // the cache like the decode kernels, so it wants two workgroups per CU
        // (the LDS of the tiles allows it) and splits down to two tiles
        const int64_t wgs = B * Hk * ((n_rows + pl.wg_rows - 1) / pl.wg_rows);
        S = auto_splits(wgs, L, 128, 512);
    } else if (pl.prefill) {
        // one workgroup per CU fits the largest tiles; split only short row counts
        const int64_t wgs = B * Hk * ((n_rows + pl.wg_rows - 1) / pl.wg_rows);
        S = auto_splits(wgs, L, 1024, 256);
    } else {
        // the generic kernel walks a split serially in 32-key blocks (one
        // memory round trip each), so even single-block splits pay off for
        // small caches (256 keys: 10.5 us with 8 splits, 12.9 us with 4), and
        // long ones want four workgroups per CU (64K keys, 3-bit, 8 kv heads:
        // 199 us with 64 splits, 136 us with 128)
        // the bit-stream decode: a workgroup of 4 waves takes at least one
        // 64-key tile per wave, about 1024 workgroups in all
        S = pl.matrix ? auto_splits(B * Hk * pl.n_rt, L, 256, 256)
            : pl.stream ? auto_splits(B * Hk, L, qkv::stream_decode_key_quantum(), 1024)
                        : auto_splits(B * Hk * pl.n_rt, L, 32, 1024);
    }
    // the narrow decode's in-kernel merge keeps one ticket per (batch, kv
    // head) in the fixed header: a batch beyond it runs unsplit
    if (pl.narrow && B * Hk > (int64_t)qkv::kTicketWords) S = 1;
    int64_t chunk = (L + S - 1) / S;
    const int64_t gran = pl.stream ? qkv::stream_decode_key_quantum()
                         : !pl.matrix ? 32
                         : pl.prefill ? 64
                         : pl.narrow  ? qkv::narrow_decode_key_quantum()
                                      : qkv::decode_matrix_key_quantum();
    // whole granules per split: rounding the chunk up can nearly halve the
    // splits when it is a few granules long (257 keys -> 512 with 256-key
    // granules: the 16-row decode of 20481 keys would get 41 splits instead
    // of 80), so it is rounded down when that keeps the split count within
    // an eighth above the one asked for
    const int64_t up = (chunk + gran - 1) / gran * gran;
    const int64_t dn = std::max<int64_t>(gran, chunk / gran * gran);
    const int64_t s_up = (L + up - 1) / up, s_dn = (L + dn - 1) / dn;
    chunk = (s_up < S && s_dn <= std::min<int64_t>(qkv::kMaxSplits, S + S / 8)) ? dn : up;
    S = (int)((L + chunk - 1) / chunk);
    pl.S = S;
    pl.chunk = chunk;
    pl.ws_bytes = ws_for(B, Hk, pl.n_rt, S, pl.RT, D);
    return pl;
}

qkv_status attention(const char* name, const void* q, int32_t q_dtype, int64_t B, int64_t Hq,
                     int64_t Lq, int64_t D, const qkv_pack* k, const qkv_pack* v, int64_t L,
                     float scale, int32_t mask_kind, const void* mask, int32_t mask_dtype,
                     const int64_t ms[4], void* out, void* workspace, size_t workspace_bytes,
                     const qkv_attn_opts* opts, void* stream, bool static_ws = false,
                     const AppendArgs* app = nullptr) {
    qkv_status st;
    if ((st = check_pack(k, "k")) != QKV_OK) return st;
    if ((st = check_pack(v, "v")) != QKV_OK) return st;
    if (!same_format(k, v)) return fail(QKV_EINVAL, "%s: K and V packs differ in format or shape", name);
    if (!q || !out) return fail(QKV_EINVAL, "%s: null q or out", name);
    if (!valid_dtype(q_dtype)) return fail(QKV_EINVAL, "%s: bad q dtype", name);
    if (B != k->B || D != k->D) return fail(QKV_EINVAL, "%s: q shape does not match the packs", name);
    if (Hq < 1 || Hq % k->H) return fail(QKV_EINVAL, "%s: Hq=%lld is not a multiple of Hk=%lld", name,
                                         (long long)Hq, (long long)k->H);
    if (Lq < 1) return fail(QKV_EINVAL, "%s: Lq must be >= 1", name);
    if (L < 1 || L > k->L_cap || L > v->L_cap)
        return fail(QKV_EINVAL, "%s: L=%lld outside [1, L_cap]", name, (long long)L);
    const int64_t G = Hq / k->H;
    if (G > 64) return fail(QKV_EUNSUPPORTED, "%s: GQA factor %lld > 64", name, (long long)G);
    if (k->mode == QKV_AFFINE && k->scale_dtype != q_dtype)
        return fail(QKV_EUNSUPPORTED, "%s: affine scale dtype must equal the query dtype", name);
    if (mask_kind != QKV_MASK_NONE && mask_kind != QKV_MASK_CAUSAL && mask_kind != QKV_MASK_ADDITIVE)
        return fail(QKV_EINVAL, "%s: bad mask kind", name);
    if (mask_kind == QKV_MASK_ADDITIVE) {
        if (!mask || !ms) return fail(QKV_EINVAL, "%s: additive mask needs data and strides", name);
        if (!valid_dtype(mask_dtype)) return fail(QKV_EINVAL, "%s: bad mask dtype", name);
        for (int i = 0; i < 4; ++i)
            if (ms[i] < 0) return fail(QKV_EINVAL, "%s: negative mask stride", name);
        if (!aligned(mask, dtype_size(mask_dtype))) return fail(QKV_EINVAL, "%s: mask misaligned", name);
    }
    if (mask_kind == QKV_MASK_CAUSAL && L < Lq)
        return fail(QKV_EINVAL, "%s: causal mask needs L >= Lq", name);
    if (opts && (opts->num_splits < 0 || opts->algo < 0 || opts->algo > QKV_ALGO_DEQUANT_F16))
        return fail(QKV_EINVAL, "%s: bad options", name);
    const int algo = opts ? opts->algo : QKV_ALGO_AUTO;
    if (k->mode == QKV_DENSE && (q_dtype != QKV_F16 || (algo != QKV_ALGO_AUTO && algo != QKV_ALGO_MATRIX)))
        return fail(QKV_EUNSUPPORTED, "%s: attention over dense packs takes fp16 queries on the matrix-core "
                    "kernel", name);
    if (algo == QKV_ALGO_DEQUANT_F16 &&
        (q_dtype != QKV_F16 || k->mode == QKV_DENSE || (k->mode == QKV_AFFINE && k->scale_dtype != QKV_F16)))
        return fail(QKV_EUNSUPPORTED, "%s: the dequantize-first strategy takes fp16 queries and a quantized "
                    "cache with fp16 scales", name);
    if ((algo == QKV_ALGO_UNFUSED || algo == QKV_ALGO_DEQUANT_F16 || algo == QKV_ALGO_MATRIX) &&
        k->mode != QKV_DENSE && !qkv::fast_format(k->mode, k->bits, (int)D))
        return fail(QKV_EUNSUPPORTED, "%s: this algorithm takes affine 4/8-bit or Q8_0 caches with D a "
                    "multiple of 64", name);
    if (opts && opts->algo == QKV_ALGO_UNFUSED && (Lq != 1 || G > 16 || B * Hq > 65535))
        return fail(QKV_EUNSUPPORTED, "%s: the unfused composition takes one query per head, a GQA "
                    "factor of at most 16 and B x Hq below 65536", name);
    const size_t qe = dtype_size(q_dtype);
    if (!aligned(q, qe) || !aligned(out, qe)) return fail(QKV_EINVAL, "%s: q/out misaligned", name);
    const size_t qbytes = (size_t)(B * Hq * Lq * D) * qe;
    Range ro{reinterpret_cast<uintptr_t>(out), reinterpret_cast<uintptr_t>(out) + qbytes};
    Range rq{reinterpret_cast<uintptr_t>(q), reinterpret_cast<uintptr_t>(q) + qbytes};
    if (overlap(ro, rq)) return fail(QKV_EINVAL, "%s: out overlaps q", name);
    const qkv_pack* packs[2] = {k, v};
    for (const qkv_pack* p : packs)
        if (overlaps_pack(ro, p)) return fail(QKV_EINVAL, "%s: out overlaps a pack", name);
    // a decode with append reads the new tokens while the call writes out,
    // the workspace and the packs' new rows
    Range rn[2] = {{0, 0}, {0, 0}};
    if (app) {
        const int64_t nn[4] = {B, k->H, 1, D};
        const int64_t ns[4] = {app->strides[0], app->strides[1], app->strides[2], 1};
        rn[0] = strided_range(app->k_new, qe, nn, ns);
        rn[1] = strided_range(app->v_new, qe, nn, ns);
        for (const Range& r : rn) {
            if (overlap(r, ro)) return fail(QKV_EINVAL, "%s: out overlaps a new token", name);
            for (const qkv_pack* p : packs)
                if (overlaps_pack(r, p)) return fail(QKV_EINVAL, "%s: a new token overlaps a pack", name);
        }
    }
    Range rm{0, 0};
    if (mask_kind == QKV_MASK_ADDITIVE) {
        const int64_t mn[4] = {B, Hq, Lq, L};
        rm = strided_range(mask, dtype_size(mask_dtype), mn, ms);
        if (overlap(ro, rm)) return fail(QKV_EINVAL, "%s: out overlaps the mask", name);
    }
    if (opts && opts->algo == QKV_ALGO_MATRIX &&
        !qkv::matrix_supported(q_dtype, k->mode, k->bits, k->group_size, (int)D, (int)G, Lq))
        return fail(QKV_EUNSUPPORTED, "%s: no matrix-core kernel for these arguments", name);

    Plan pl = make_plan(B, Hq, Lq, D, L, k, q_dtype, opts);
    if (B * k->H > 65535 || (!pl.prefill && pl.n_rt > 65535) || pl.S > 65535)
        return fail(QKV_EUNSUPPORTED, "%s: batch x kv heads or row tiles beyond the launch grid", name);
    if ((k->mode == QKV_DENSE || pl.prepass) && !pl.prefill)
        return fail(QKV_EUNSUPPORTED, "%s: no matrix-core kernel for a dense cache of this size", name);
    if (pl.ws_bytes > 0 && static_ws) {
        // the library's own device array; checked last, since resolving it
        // may enqueue the zero fill of its ticket header
        if (pl.ws_bytes > QKV_STATIC_SCRATCH_BYTES)
            return fail(QKV_EWORKSPACE, "%s: the plan needs %zu bytes of workspace, the static one holds %zu",
                        name, pl.ws_bytes, (size_t)QKV_STATIC_SCRATCH_BYTES);
        hipError_t se = qkv::static_scratch(static_cast<hipStream_t>(stream), &workspace);
        if (se != hipSuccess) return hip_status(se, name);
        workspace_bytes = QKV_STATIC_SCRATCH_BYTES;
    } else if (pl.ws_bytes > 0) {
        if (!workspace || workspace_bytes < pl.ws_bytes)
            return fail(QKV_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", name,
                        pl.ws_bytes, workspace ? workspace_bytes : (size_t)0);
        if (!aligned(workspace, 256)) return fail(QKV_EINVAL, "%s: workspace not 256-byte aligned", name);
        Range rw{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + pl.ws_bytes};
        if (overlap(ro, rw)) return fail(QKV_EINVAL, "%s: out overlaps the workspace", name);
        if (overlap(rq, rw)) return fail(QKV_EINVAL, "%s: q overlaps the workspace", name);
        for (const qkv_pack* p : packs)
            if (overlaps_pack(rw, p)) return fail(QKV_EINVAL, "%s: the workspace overlaps a pack", name);
        if (mask_kind == QKV_MASK_ADDITIVE && overlap(rm, rw))
            return fail(QKV_EINVAL, "%s: the mask overlaps the workspace", name);
        if (app && (overlap(rn[0], rw) || overlap(rn[1], rw)))
            return fail(QKV_EINVAL, "%s: a new token overlaps the workspace", name);
    }

    // the dequantize-first strategy attends dense fp16 copies at the start of
    // the workspace; the split states follow them
    const qkv_pack* kx = k;
    const qkv_pack* vx = v;
    qkv_pack kd{}, vd{};
    if (pl.prepass) {
        uint8_t* w8 = static_cast<uint8_t*>(workspace);
        kd = dense_copy_of(k, L, w8);
        vd = dense_copy_of(v, L, w8 + pl.dense_bytes);
        kx = &kd;
        vx = &vd;
        workspace = w8 + 2 * pl.dense_bytes;
    }

    qkv::AttnLaunch a{};
    a.q = q;
    a.out = out;
    a.k = {kx->codes, kx->scales, kx->biases, kx->stride_b, kx->stride_h, kx->stride_l};
    a.v = {vx->codes, vx->scales, vx->biases, vx->stride_b, vx->stride_h, vx->stride_l};
    a.Hq = Hq;
    a.Hk = k->H;
    a.Lq = Lq;
    a.L = L;
    a.G = (int32_t)G;
    a.gs_log2 = ilog2(kx->group_size);
    a.scale = scale;
    a.mask_kind = mask_kind;
    a.mask = mask_kind == QKV_MASK_ADDITIVE ? mask : nullptr;
    a.mask_dtype = mask_dtype;
    if (mask_kind == QKV_MASK_ADDITIVE) {
        a.ms0 = ms[0]; a.ms1 = ms[1]; a.ms2 = ms[2]; a.ms3 = ms[3];
    }
    a.S = pl.S;
    a.chunk = pl.chunk;
    a.n_rows = (int32_t)(G * Lq);
    a.n_rt = pl.n_rt;
    a.wg_rows = pl.wg_rows;
    a.RT = pl.RT;
    if (pl.unfused) {
        uint8_t* w8 = static_cast<uint8_t*>(workspace);
        a.un_scores = reinterpret_cast<float*>(w8);
        a.un_stats = reinterpret_cast<float*>(w8 + unfused_scores_bytes(B, Hq, L));
        a.un_partial = reinterpret_cast<float*>(w8 + unfused_scores_bytes(B, Hq, L) +
                                                unfused_stats_bytes(B, Hq, L));
        a.un_chunks = pl.S;
        a.un_chunk = pl.chunk;
    } else if (pl.ws_bytes > 0) {
        const int64_t tiles = B * k->H * pl.n_rt;
        a.tickets = static_cast<uint32_t*>(workspace);
        a.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + qkv::kTicketBytes);
        a.part_o = a.part_ml + (size_t)tiles * (size_t)pl.S * 16 * 2;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    // a decode with append: on the narrow and the 16-row decode (affine or
    // Q8_0 codes, no additive mask) the kernel quantizes the new rows itself;
    // otherwise the append kernel runs first
    hipError_t e = hipSuccess;
    if (app) {
        const bool fused = (pl.narrow || (pl.matrix && !pl.prefill)) && !pl.unfused && !pl.prepass &&
                           mask_kind != QKV_MASK_ADDITIVE && (k->mode == QKV_AFFINE || k->mode == QKV_Q8_0);
        if (fused) {
            a.append = 1;
            a.k_new = app->k_new;
            a.v_new = app->v_new;
            a.ns0 = app->strides[0];
            a.ns1 = app->strides[1];
        } else {
            e = qkv::launch_quantize(q_dtype, k->mode, k->bits, k->group_size, (int)D,
                                     append_launch(app->k_new, app->v_new, app->strides, 1, L - 1, k, v), 2, s);
            if (e != hipSuccess) return hip_status(e, name);
        }
    }
    const bool timed = opts && opts->timing_events[0] && opts->timing_events[1];
    if (timed) {
        hipError_t te = hipEventRecord(static_cast<hipEvent_t>(opts->timing_events[0]), s);
        if (te != hipSuccess) return hip_status(te, name);
    }
    if (pl.prepass) {
        for (int i = 0; i < 2 && e == hipSuccess; ++i) {
            const qkv_pack* src = i == 0 ? k : v;
            const qkv_pack& dst = i == 0 ? kd : vd;
            e = qkv::launch_dequantize(src->mode, src->bits, src->group_size, (int)D,
                                       dequant_job(src, &dst, L), s);
        }
    }
    if (e == hipSuccess)
        e = pl.unfused     ? qkv::launch_attn_unfused(q_dtype, k->mode, k->bits, (int)D, B, a, s)
                   : pl.prefill  ? qkv::launch_prefill_matrix(kx->mode, kx->bits, (int)D, B, a, s)
                   : pl.narrow ? qkv::launch_attn_narrow(k->mode, k->bits, (int)D, B, a, s)
                   : pl.matrix ? qkv::launch_attn_matrix(k->mode, k->bits, (int)D, B, a, s)
                   : pl.stream ? qkv::launch_attn_stream(k->mode, k->bits, (int)D, B, a, s)
                               : qkv::launch_attn_generic(q_dtype, k->mode, k->bits, (int)D, B, a, s);
    if (e == hipSuccess && timed) e = hipEventRecord(static_cast<hipEvent_t>(opts->timing_events[1]), s);
    // the narrow decode kernel merges its splits itself
    if (e == hipSuccess && pl.S > 1 && !pl.narrow && !pl.unfused) e = qkv::launch_merge(q_dtype, (int)D, B, a, s);
    return hip_status(e, name);
}

}  // namespace

extern "C" {

qkv_status qkv_quantize(const void* x, int32_t x_dtype, const int64_t x_strides[3], int64_t L,
                        const qkv_pack* dst, void* stream) {
    qkv_status st;
    if ((st = check_pack(dst, "qkv_quantize")) != QKV_OK) return st;
    if ((st = check_source(x, x_dtype, x_strides, dst, "qkv_quantize")) != QKV_OK) return st;
    if (L < 0 || L > dst->L_cap) return fail(QKV_EINVAL, "qkv_quantize: L=%lld outside [0, L_cap]", (long long)L);
    if (L == 0) return ok();
    if ((st = check_row_strides(x_strides, x_dtype, dst, "qkv_quantize")) != QKV_OK) return st;
    qkv::QuantLaunch p{};
    p.job[0] = make_job(x, x_strides, dst);
    p.job[1] = p.job[0];
    p.H = dst->H;
    p.T = L;
    p.offset = 0;
    p.BH = dst->B * dst->H;
    p.rows = p.BH * L;
    hipError_t e = qkv::launch_quantize(x_dtype, dst->mode, dst->bits, dst->group_size, (int)dst->D, p,
                                        1, static_cast<hipStream_t>(stream));
    return hip_status(e, "qkv_quantize");
}

qkv_status qkv_update_append(const void* k_new, const void* v_new, int32_t dtype,
                             const int64_t new_strides[3], int64_t T, int64_t offset,
                             const qkv_pack* k_cache, const qkv_pack* v_cache, void* stream) {
    qkv_status st;
    if ((st = check_append("qkv_update_append", k_new, v_new, dtype, new_strides, T, offset, k_cache, v_cache)) !=
        QKV_OK)
        return st;
    hipError_t e = qkv::launch_quantize(dtype, k_cache->mode, k_cache->bits, k_cache->group_size,
                                        (int)k_cache->D,
                                        append_launch(k_new, v_new, new_strides, T, offset, k_cache, v_cache), 2,
                                        static_cast<hipStream_t>(stream));
    return hip_status(e, "qkv_update_append");
}

qkv_status qkv_dequantize(const qkv_pack* src, int64_t L, const qkv_pack* dst, void* stream) {
    qkv_status st;
    if ((st = check_pack(src, "qkv_dequantize(src)")) != QKV_OK) return st;
    if ((st = check_pack(dst, "qkv_dequantize(dst)")) != QKV_OK) return st;
    if (src->mode == QKV_DENSE) return fail(QKV_EINVAL, "qkv_dequantize: the source is not quantized");
    if (dst->mode != QKV_DENSE) return fail(QKV_EINVAL, "qkv_dequantize: the destination must be a dense pack");
    if ((src->mode == QKV_AFFINE && src->scale_dtype != QKV_F16) ||
        !qkv::fast_format(src->mode, src->bits, (int)src->D))
        return fail(QKV_EUNSUPPORTED, "qkv_dequantize: affine 4/8-bit packs with fp16 scales, or Q8_0, "
                    "with D a multiple of 64");
    if (src->B != dst->B || src->H != dst->H || src->D != dst->D)
        return fail(QKV_EINVAL, "qkv_dequantize: source and destination differ in B, H or D");
    if (L < 0 || L > src->L_cap || L > dst->L_cap)
        return fail(QKV_EINVAL, "qkv_dequantize: L=%lld outside [0, capacity]", (long long)L);
    if (overlaps_pack(codes_range(dst), src))
        return fail(QKV_EINVAL, "qkv_dequantize: source and destination overlap");
    if (L == 0) return ok();
    return hip_status(qkv::launch_dequantize(src->mode, src->bits, src->group_size, (int)src->D,
                                             dequant_job(src, dst, L), static_cast<hipStream_t>(stream)),
                      "qkv_dequantize");
}

size_t qsdpa_workspace_bytes(int64_t B, int64_t Hq, int64_t Lq, int64_t D, int64_t L,
                             const qkv_pack* k, int32_t q_dtype, const qkv_attn_opts* opts) {
    if (!k || k->H < 1 || B < 1 || Hq < 1 || Lq < 1 || L < 1 || Hq % k->H) return 0;
    return make_plan(B, Hq, Lq, D, L, k, q_dtype, opts).ws_bytes;
}

qkv_status qsdpa_plan(int64_t B, int64_t Hq, int64_t Lq, int64_t D, int64_t L, const qkv_pack* k,
                      int32_t q_dtype, const qkv_attn_opts* opts, qkv_attn_plan* plan) {
    if (!k || !plan) return fail(QKV_EINVAL, "qsdpa_plan: null pack or plan");
    if (k->H < 1 || B < 1 || Hq < 1 || Lq < 1 || L < 1 || Hq % k->H)
        return fail(QKV_EINVAL, "qsdpa_plan: bad sizes");
    Plan pl = make_plan(B, Hq, Lq, D, L, k, q_dtype, opts);
    plan->algo = pl.unfused   ? QKV_ALGO_UNFUSED
                 : pl.prepass ? QKV_ALGO_DEQUANT_F16
                 : pl.matrix  ? QKV_ALGO_MATRIX
                              : QKV_ALGO_GENERIC;
    plan->num_splits = pl.S;
    plan->row_tile = pl.prefill ? pl.wg_rows : pl.RT;
    plan->kernel = pl.unfused   ? QKV_KERNEL_UNFUSED
                   : pl.stream  ? QKV_KERNEL_DECODE_STREAM
                   : !pl.matrix ? QKV_KERNEL_GENERIC
                   : pl.prefill ? QKV_KERNEL_PREFILL
                   : pl.narrow  ? QKV_KERNEL_DECODE_NARROW
                                : QKV_KERNEL_DECODE;
    plan->keys_per_split = pl.chunk;
    plan->workspace_bytes = pl.ws_bytes;
    return ok();
}

qkv_status qsdpa_decode(const void* q, int32_t q_dtype, int64_t B, int64_t Hq, int64_t D,
                        const qkv_pack* k, const qkv_pack* v, int64_t L, float scale,
                        const void* mask, int32_t mask_dtype, const int64_t mask_strides[4],
                        void* out, void* workspace, size_t workspace_bytes,
                        const qkv_attn_opts* opts, void* stream) {
    return attention("qsdpa_decode", q, q_dtype, B, Hq, 1, D, k, v, L, scale,
                     mask ? QKV_MASK_ADDITIVE : QKV_MASK_NONE, mask, mask_dtype, mask_strides, out,
                     workspace, workspace_bytes, opts, stream);
}

qkv_status qsdpa_decode_static(const void* q, int32_t q_dtype, int64_t B, int64_t Hq, int64_t D,
                               const qkv_pack* k, const qkv_pack* v, int64_t L, float scale,
                               const void* mask, int32_t mask_dtype, const int64_t mask_strides[4],
                               void* out, const qkv_attn_opts* opts, void* stream) {
    return attention("qsdpa_decode_static", q, q_dtype, B, Hq, 1, D, k, v, L, scale,
                     mask ? QKV_MASK_ADDITIVE : QKV_MASK_NONE, mask, mask_dtype, mask_strides, out,
                     nullptr, 0, opts, stream, true);
}

qkv_status qsdpa_decode_append(const void* q, int32_t q_dtype, int64_t B, int64_t Hq, int64_t D,
                               const void* k_new, const void* v_new, const int64_t new_strides[3],
                               int64_t offset, const qkv_pack* k_cache, const qkv_pack* v_cache, float scale,
                               const void* mask, int32_t mask_dtype, const int64_t mask_strides[4], void* out,
                               void* workspace, size_t workspace_bytes, const qkv_attn_opts* opts, void* stream) {
    qkv_status st;
    if ((st = check_append("qsdpa_decode_append", k_new, v_new, q_dtype, new_strides, 1, offset, k_cache,
                           v_cache)) != QKV_OK)
        return st;
    const AppendArgs app{k_new, v_new, new_strides};
    return attention("qsdpa_decode_append", q, q_dtype, B, Hq, 1, D, k_cache, v_cache, offset + 1, scale,
                     mask ? QKV_MASK_ADDITIVE : QKV_MASK_NONE, mask, mask_dtype, mask_strides, out, workspace,
                     workspace_bytes, opts, stream, false, &app);
}

qkv_status qsdpa_prefill(const void* q, int32_t q_dtype, int64_t B, int64_t Hq, int64_t Lq,
                         int64_t D, const qkv_pack* k, const qkv_pack* v, int64_t L, float scale,
                         int32_t mask_kind, const void* mask, int32_t mask_dtype,
                         const int64_t mask_strides[4], void* out, void* workspace,
                         size_t workspace_bytes, const qkv_attn_opts* opts, void* stream) {
    return attention("qsdpa_prefill", q, q_dtype, B, Hq, Lq, D, k, v, L, scale, mask_kind, mask,
                     mask_dtype, mask_strides, out, workspace, workspace_bytes, opts, stream);
}

qkv_status qsdpa_workspace_reset(void* workspace, size_t workspace_bytes, void* stream) {
    if (!workspace) return fail(QKV_EINVAL, "qsdpa_workspace_reset: null workspace");
    if (!aligned(workspace, 256)) return fail(QKV_EINVAL, "qsdpa_workspace_reset: workspace not 256-byte aligned");
    if (workspace_bytes < qkv::kTicketBytes)
        return fail(QKV_EINVAL, "qsdpa_workspace_reset: %zu bytes is less than the %zu-byte ticket header",
                    workspace_bytes, qkv::kTicketBytes);
    return hip_status(qkv::launch_fill_zero(workspace, qkv::kTicketBytes, static_cast<hipStream_t>(stream)),
                      "qsdpa_workspace_reset");
}

qkv_status qkv_measure_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                            void* stream) {
    if (!buf || !sink) return fail(QKV_EINVAL, "qkv_measure_read: null pointer");
    if (bytes == 0 || bytes % 16 || !aligned(buf, 16))
        return fail(QKV_EINVAL, "qkv_measure_read: bytes must be a nonzero multiple of 16 at a 16-byte aligned address");
    if (workgroups < 1 || workgroups > QKV_MEASURE_MAX_WORKGROUPS)
        return fail(QKV_EINVAL, "qkv_measure_read: workgroups=%d outside [1, %d]", workgroups,
                    QKV_MEASURE_MAX_WORKGROUPS);
    return hip_status(qkv::launch_measure_read(buf, bytes, workgroups, sink, static_cast<hipStream_t>(stream)),
                      "qkv_measure_read");
}

qkv_status qkv_measure_read_config(const void* buf, size_t bytes, int32_t workgroups, int32_t threads,
                                   int32_t in_flight, int32_t width, uint32_t* sink, void* stream) {
    if (!buf || !sink) return fail(QKV_EINVAL, "qkv_measure_read_config: null pointer");
    if (width != 4 && width != 8 && width != 16)
        return fail(QKV_EINVAL, "qkv_measure_read_config: width %d not in {4, 8, 16}", width);
    if (bytes == 0 || bytes % (size_t)width || !aligned(buf, (size_t)width))
        return fail(QKV_EINVAL, "qkv_measure_read_config: bytes and buf must be multiples of the width");
    if (threads < 64 || threads > 1024 || threads % 64)
        return fail(QKV_EINVAL, "qkv_measure_read_config: threads=%d not a multiple of 64 in [64, 1024]", threads);
    if (in_flight != 1 && in_flight != 2 && in_flight != 4 && in_flight != 8 && in_flight != 16)
        return fail(QKV_EINVAL, "qkv_measure_read_config: in_flight=%d not in {1, 2, 4, 8, 16}", in_flight);
    if (workgroups < 1 || workgroups > QKV_MEASURE_MAX_WORKGROUPS)
        return fail(QKV_EINVAL, "qkv_measure_read_config: workgroups=%d outside [1, %d]", workgroups,
                    QKV_MEASURE_MAX_WORKGROUPS);
    return hip_status(qkv::launch_measure_read_config(buf, bytes, workgroups, threads, in_flight, width, sink,
                                                      static_cast<hipStream_t>(stream)),
                      "qkv_measure_read_config");
}

const char* qkv_last_error(void) { return g_last_error.c_str(); }

int32_t qkv_abi_version(void) { return QKV_ABI_VERSION; }

}  // extern "C"
