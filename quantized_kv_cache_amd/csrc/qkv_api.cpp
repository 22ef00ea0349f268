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
}  // namespace qkv
#include "qkv_merge.hpp"

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
    uintptr_t lo = reinterpret_cast<uintptr_t>(base);
    return {lo, lo + (uintptr_t)((max_row(p) + 1) * groups_per_row(p) * dtype_size(p->scale_dtype))};
}

qkv_status check_pack(const qkv_pack* p, const char* name) {
    if (!p) return fail(QKV_EINVAL, "%s: null pack", name);
    if (p->mode != QKV_AFFINE && p->mode != QKV_Q8_0)
        return fail(QKV_EINVAL, "%s: unknown mode %d", name, p->mode);
    if (p->B < 1 || p->H < 1 || p->L_cap < 1 || p->D < 1)
        return fail(QKV_EINVAL, "%s: B, H, L_cap and D must be >= 1", name);
    if (p->stride_b < 0 || p->stride_h < 0 || p->stride_l < 0)
        return fail(QKV_EINVAL, "%s: negative stride", name);
    if (!p->codes || !p->scales) return fail(QKV_EINVAL, "%s: null codes or scales", name);
    if (p->mode == QKV_AFFINE) {
        if (p->bits != 4 && p->bits != 8) return fail(QKV_EUNSUPPORTED, "%s: bits %d not in {4, 8}", name, p->bits);
        if (p->group_size != 32 && p->group_size != 64 && p->group_size != 128)
            return fail(QKV_EUNSUPPORTED, "%s: group_size %d not in {32, 64, 128}", name, p->group_size);
        if (p->D % p->group_size)
            return fail(QKV_EINVAL, "%s: D=%lld is not a multiple of group_size=%d", name,
                        (long long)p->D, p->group_size);
        if (!valid_dtype(p->scale_dtype)) return fail(QKV_EINVAL, "%s: bad scale dtype", name);
        if (!p->biases) return fail(QKV_EINVAL, "%s: affine pack needs biases", name);
    } else {
        if (p->bits != 8 || p->group_size != 32)
            return fail(QKV_EINVAL, "%s: Q8_0 needs bits=8, group_size=32", name);
        if (p->scale_dtype != QKV_F16) return fail(QKV_EINVAL, "%s: Q8_0 scales are fp16", name);
        if (p->biases) return fail(QKV_EINVAL, "%s: Q8_0 pack takes no biases", name);
        if (p->D % 32) return fail(QKV_EINVAL, "%s: D must be a multiple of 32", name);
    }
    if (p->D != 64 && p->D != 128 && p->D != 256)
        return fail(QKV_EUNSUPPORTED, "%s: head size D=%lld not in {64, 128, 256}", name, (long long)p->D);
    if (!aligned(p->codes, 16)) return fail(QKV_EINVAL, "%s: codes not 16-byte aligned", name);
    // scale and bias planes: aligned to one row of them (up to 16 bytes), the
    // width of the kernels' row loads
    const size_t ss = dtype_size(p->scale_dtype);
    const size_t ra = std::min<size_t>(16, (size_t)(p->D / p->group_size) * ss);
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
    return QKV_OK;
}

// ---------------------------------------------------------------- attention plans
struct Plan {
    bool matrix;
    bool prefill;                   // tiled matrix kernel
    int wg_rows;                    // its rows per workgroup
    bool narrow;                    // single-query kernel for GQA factors <= 4
    int RT, n_rt, S;
    int64_t chunk;
    size_t ws_bytes;
};

size_t ws_for(int64_t B, int64_t Hk, int n_rt, int S, int RT, int64_t D) {
    if (S <= 1) return 0;
    return qkv::ticket_bytes(B * Hk * n_rt) +
           (size_t)(B * Hk * n_rt) * (size_t)S * (size_t)RT * (size_t)(D + 2) * 4;  // ml + o
}

// Split count: enough workgroups to cover the CUs about twice, each split at
// least min_keys long, and at most kMaxSplits (the merge keeps per-split
// weights in LDS).
int auto_splits(int64_t base_wgs, int64_t L, int64_t min_keys, int64_t target) {
    int64_t want = (target + base_wgs - 1) / base_wgs;
    int64_t cap = std::max<int64_t>(1, L / min_keys);
    return (int)std::max<int64_t>(1, std::min<int64_t>({want, cap, 256}));
}

Plan make_plan(int64_t B, int64_t Hq, int64_t Lq, int64_t D, int64_t L, const qkv_pack* k,
               int32_t q_dtype, const qkv_attn_opts* opts) {
    Plan pl{};
    const int64_t Hk = k->H;
    const int G = (int)(Hq / Hk);
    const int algo = opts ? opts->algo : QKV_ALGO_AUTO;
    const int bits = k->bits;
    pl.matrix = false;
    pl.prefill = false;
    pl.narrow = false;
    // the matrix kernels address a kv head's rows with 32-bit offsets
    const int64_t span = (k->L_cap - 1) * k->stride_l * row_bytes(k) + row_bytes(k);
    if (algo != QKV_ALGO_GENERIC && span < (int64_t(1) << 31) &&
        qkv::matrix_supported(q_dtype, k->mode, bits, k->group_size, (int)D, G, Lq)) {
        pl.matrix = true;
        pl.narrow = qkv::narrow_decode_supported(q_dtype, k->mode, bits, k->group_size, (int)D, G, Lq);
        pl.prefill = !pl.narrow &&
                     !qkv::decode_matrix_supported(q_dtype, k->mode, bits, k->group_size, (int)D, G, Lq);
    }
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
    } else if (pl.prefill) {
        // one workgroup per CU fits the largest tiles; split only short row counts
        const int64_t wgs = B * Hk * ((n_rows + pl.wg_rows - 1) / pl.wg_rows);
        S = auto_splits(wgs, L, 1024, 256);
    } else {
        // the generic kernel walks a split serially in 32-key blocks (one
        // memory round trip each), so even single-block splits pay off for
        // small caches (256 keys: 10.5 us with 8 splits, 12.9 us with 4)
        S = pl.matrix ? auto_splits(B * Hk * pl.n_rt, L, 256, 256)
                      : auto_splits(B * Hk * pl.n_rt, L, 32, 512);
    }
    int64_t chunk = (L + S - 1) / S;
    const int64_t gran = !pl.matrix ? 32
                         : pl.prefill ? 64
                         : pl.narrow  ? qkv::narrow_decode_key_quantum()
                                      : qkv::decode_matrix_key_quantum();
    chunk = (chunk + gran - 1) / gran * gran;
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
                     const qkv_attn_opts* opts, void* stream) {
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
    if (opts && (opts->num_splits < 0 || opts->algo < 0 || opts->algo > QKV_ALGO_MATRIX))
        return fail(QKV_EINVAL, "%s: bad options", name);
    const size_t qe = dtype_size(q_dtype);
    if (!aligned(q, qe) || !aligned(out, qe)) return fail(QKV_EINVAL, "%s: q/out misaligned", name);
    const size_t qbytes = (size_t)(B * Hq * Lq * D) * qe;
    Range ro{reinterpret_cast<uintptr_t>(out), reinterpret_cast<uintptr_t>(out) + qbytes};
    Range rq{reinterpret_cast<uintptr_t>(q), reinterpret_cast<uintptr_t>(q) + qbytes};
    if (overlap(ro, rq)) return fail(QKV_EINVAL, "%s: out overlaps q", name);
    const qkv_pack* packs[2] = {k, v};
    for (const qkv_pack* p : packs) {
        if (overlap(ro, codes_range(p)) || overlap(ro, scales_range(p, p->scales)) ||
            (p->biases && overlap(ro, scales_range(p, p->biases))))
            return fail(QKV_EINVAL, "%s: out overlaps a pack", name);
    }
    if (opts && opts->algo == QKV_ALGO_MATRIX &&
        !qkv::matrix_supported(q_dtype, k->mode, k->bits, k->group_size, (int)D, (int)G, Lq))
        return fail(QKV_EUNSUPPORTED, "%s: no matrix-core kernel for these arguments", name);

    Plan pl = make_plan(B, Hq, Lq, D, L, k, q_dtype, opts);
    if (B * k->H > 65535 || (!pl.prefill && pl.n_rt > 65535) || pl.S > 65535)
        return fail(QKV_EUNSUPPORTED, "%s: batch x kv heads or row tiles beyond the launch grid", name);
    if (pl.ws_bytes > 0) {
        if (!workspace || workspace_bytes < pl.ws_bytes)
            return fail(QKV_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", name,
                        pl.ws_bytes, workspace ? workspace_bytes : (size_t)0);
        if (!aligned(workspace, 256)) return fail(QKV_EINVAL, "%s: workspace not 256-byte aligned", name);
        Range rw{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + pl.ws_bytes};
        if (overlap(ro, rw)) return fail(QKV_EINVAL, "%s: out overlaps the workspace", name);
    }

    qkv::AttnLaunch a{};
    a.q = q;
    a.out = out;
    a.k = {k->codes, k->scales, k->biases, k->stride_b, k->stride_h, k->stride_l};
    a.v = {v->codes, v->scales, v->biases, v->stride_b, v->stride_h, v->stride_l};
    a.Hq = Hq;
    a.Hk = k->H;
    a.Lq = Lq;
    a.L = L;
    a.G = (int32_t)G;
    a.gs_log2 = ilog2(k->group_size);
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
    if (pl.ws_bytes > 0) {
        const int64_t tiles = B * k->H * pl.n_rt;
        a.tickets = static_cast<uint32_t*>(workspace);
        a.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + qkv::ticket_bytes(tiles));
        a.part_o = a.part_ml + (size_t)tiles * (size_t)pl.S * 16 * 2;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool timed = opts && opts->timing_events[0] && opts->timing_events[1];
    if (timed) {
        hipError_t te = hipEventRecord(static_cast<hipEvent_t>(opts->timing_events[0]), s);
        if (te != hipSuccess) return hip_status(te, name);
    }
    hipError_t e = pl.prefill  ? qkv::launch_prefill_matrix(k->mode, k->bits, (int)D, B, a, s)
                   : pl.narrow ? qkv::launch_attn_narrow(k->mode, k->bits, (int)D, B, a, s)
                   : pl.matrix ? qkv::launch_attn_matrix(k->mode, k->bits, (int)D, B, a, s)
                               : qkv::launch_attn_generic(q_dtype, k->mode, k->bits, (int)D, B, a, s);
    if (e == hipSuccess && timed) e = hipEventRecord(static_cast<hipEvent_t>(opts->timing_events[1]), s);
    // the narrow decode kernel merges its splits itself
    if (e == hipSuccess && pl.S > 1 && !pl.narrow) e = qkv::launch_merge(q_dtype, (int)D, B, a, s);
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
    qkv::QuantLaunch p{};
    p.job[0] = make_job(x, x_strides, dst);
    p.job[1] = p.job[0];
    p.H = dst->H;
    p.T = L;
    p.offset = 0;
    p.rows = dst->B * dst->H * L;
    hipError_t e = qkv::launch_quantize(x_dtype, dst->mode, dst->bits, dst->group_size, (int)dst->D, p,
                                        1, static_cast<hipStream_t>(stream));
    return hip_status(e, "qkv_quantize");
}

qkv_status qkv_update_append(const void* k_new, const void* v_new, int32_t dtype,
                             const int64_t new_strides[3], int64_t T, int64_t offset,
                             const qkv_pack* k_cache, const qkv_pack* v_cache, void* stream) {
    qkv_status st;
    if ((st = check_pack(k_cache, "qkv_update_append(k)")) != QKV_OK) return st;
    if ((st = check_pack(v_cache, "qkv_update_append(v)")) != QKV_OK) return st;
    if (!same_format(k_cache, v_cache))
        return fail(QKV_EINVAL, "qkv_update_append: K and V packs differ in format or shape");
    if ((st = check_source(k_new, dtype, new_strides, k_cache, "qkv_update_append(k_new)")) != QKV_OK) return st;
    if ((st = check_source(v_new, dtype, new_strides, v_cache, "qkv_update_append(v_new)")) != QKV_OK) return st;
    if (T < 1) return fail(QKV_EINVAL, "qkv_update_append: T must be >= 1");
    if (offset < 0 || offset + T > k_cache->L_cap || offset + T > v_cache->L_cap)
        return fail(QKV_EINVAL, "qkv_update_append: rows [%lld, %lld) exceed the capacity", (long long)offset,
                    (long long)(offset + T));
    if (overlap(codes_range(k_cache), codes_range(v_cache)))
        return fail(QKV_EINVAL, "qkv_update_append: K and V codes overlap");
    qkv::QuantLaunch p{};
    p.job[0] = make_job(k_new, new_strides, k_cache);
    p.job[1] = make_job(v_new, new_strides, v_cache);
    p.H = k_cache->H;
    p.T = T;
    p.offset = offset;
    p.rows = k_cache->B * k_cache->H * T;
    hipError_t e = qkv::launch_quantize(dtype, k_cache->mode, k_cache->bits, k_cache->group_size,
                                        (int)k_cache->D, p, 2, static_cast<hipStream_t>(stream));
    return hip_status(e, "qkv_update_append");
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
    plan->algo = pl.matrix ? QKV_ALGO_MATRIX : QKV_ALGO_GENERIC;
    plan->num_splits = pl.S;
    plan->row_tile = pl.prefill ? pl.wg_rows : pl.RT;
    plan->kernel = !pl.matrix  ? QKV_KERNEL_GENERIC
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

qkv_status qsdpa_prefill(const void* q, int32_t q_dtype, int64_t B, int64_t Hq, int64_t Lq,
                         int64_t D, const qkv_pack* k, const qkv_pack* v, int64_t L, float scale,
                         int32_t mask_kind, const void* mask, int32_t mask_dtype,
                         const int64_t mask_strides[4], void* out, void* workspace,
                         size_t workspace_bytes, const qkv_attn_opts* opts, void* stream) {
    return attention("qsdpa_prefill", q, q_dtype, B, Hq, Lq, D, k, v, L, scale, mask_kind, mask,
                     mask_dtype, mask_strides, out, workspace, workspace_bytes, opts, stream);
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

const char* qkv_last_error(void) { return g_last_error.c_str(); }

int32_t qkv_abi_version(void) { return QKV_ABI_VERSION; }

}  // extern "C"
