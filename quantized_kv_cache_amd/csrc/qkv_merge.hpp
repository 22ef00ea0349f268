// Merge of split-key softmax states.  Each split s of a row left (m, l) and an
// unnormalised o[D] with
//   o = sum_j 2^(z_j - m) v_j,  l = sum_j 2^(z_j - m)   (z in log2 units),
// and the row's result is  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// M = max_s m_s (the merge of partial softmax states on the MLX page
// "add fast::quantized_kv_update", sdpa_vector.h quant_sdpa_vector, applied
// across workgroups).  A row with no visible key (every m_s = -inf) gives 0.
//
// Workspace of a call: [tickets: kTicketBytes, one uint32 per (batch, kv
// head)] [ml: tiles x S x 16 x 2] [o: tiles x S x 16 x D] (fp32).  The
// merges take the row's maximum over its splits first and then add the
// states weighted by 2^(m_s - M).  Either the
// attention kernel writes the states and merge_splits_kernel, launched next on
// the same stream, reads them (kernel order is the only synchronisation), or
// the attention kernel merges them itself (merge_last below): every workgroup
// of a tile stores its state at device scope and takes a ticket, and the one
// that takes the last ticket combines the S states.
#pragma once

#include "qkv_device.hpp"
#include "qkv_internal.hpp"

namespace qkv {

constexpr int kMaxSplits = 256;

hipError_t launch_merge(int q_dtype, int D, int64_t B, const AttnLaunch& p, hipStream_t stream);

// The ticket header at the start of every split workspace: one uint32 per
// (batch, kv head) of the fused-merge decode, whose grid holds fewer than
// 2^16 of them.  Its size does not depend on the call, so the partial states
// of one call never lie where a later call on the same workspace keeps its
// tickets.
constexpr size_t kTicketWords = 65536;
constexpr size_t kTicketBytes = kTicketWords * 4;

// Zero-fills 'bytes' (a multiple of 16) at p on 'stream' with a kernel (no
// memset node, so the call can be captured in a graph).
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);

// Cache policy bits of a buffer access: sc1 = device scope.  A store with it
// is performed in memory shared by all XCDs (not only in the writer's L2)
// when its vmcnt completes; a load with it does not return a line another
// XCD's L2 may hold stale.
constexpr int kScopeDevice = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t flat_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

// Ticket of the fused merge, taken by one thread of each workgroup of a tile
// after the workgroup's state stores have completed (s_waitcnt vmcnt(0) in
// every thread, then a barrier).  atomic_dec with limit S - 1 counts a zero
// counter down S - 1, S - 2, ..., 1, 0: the workgroup that reads 1 took the
// last ticket, and the counter is 0 again for the next call.  Returns true
// for the last workgroup.
__device__ __forceinline__ bool take_last_ticket(uint32_t* ticket, int S) {
    return __builtin_amdgcn_atomic_dec32(ticket, (uint32_t)(S - 1), __ATOMIC_RELAXED, "agent") == 1u;
}

// s_waitcnt vmcnt(0): the thread's stores so far are complete.
__device__ __forceinline__ void wait_stores() {
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __asm__ __volatile__("" ::: "memory");
}

// The fused merge for single-query tiles (rows = the G <= GP query heads of a
// kv head), run by all NTHR threads of the last workgroup: thread -> (float4
// column c of the GP x D outputs, split group sg); it combines splits sg,
// sg + SGN, ...  When a thread has at most U splits (S <= U SGN) their m, l
// and o are all requested at once, so the merge costs one round trip to
// memory: each (m, l) pair is read once, by one thread, and shared through
// 'lds' (>= 6 NTHR + 256 floats), where every thread then finds the row's
// maximum M.  With more splits the m values are read first
// (U loads in flight at a time) and the states after M is known.  Either way
// the states are weighted by 2^(m_s - M) in split order, the split groups'
// sums are added through 'lds' in group order, and column c's 4 fp16 outputs
// are stored.  No split waits on another's rescaling, and any workgroup that
// runs it gets the same result.
template <int NTHR, int D, int GP>
__device__ __forceinline__ void merge_last(const AttnLaunch& p, int64_t b, int64_t kvh, int64_t bk,
                                           float* lds) {
    constexpr int F4 = D / 4;
    constexpr int NC = GP * F4;
    constexpr int SGN = NTHR / NC;
    constexpr int U = 8;
    static_assert(NTHR % NC == 0, "whole split groups");
    const int tid = threadIdx.x;
    const int c = tid % NC, sg = tid / NC;
    const int h = c / F4, f = c % F4;
    const int S = p.S, G = p.G;
    const auto rml = flat_rsrc(p.part_ml + bk * S * 32, (uint32_t)S * 32 * 4);
    const auto ro = flat_rsrc(p.part_o + bk * S * 16 * D, (uint32_t)S * 16 * D * 4);
    // states of splits s0 + u SGN, u < U (absent ones: m = -inf, l = 0, o = 0)
    auto load_states = [&](int s0, float* m, float* ls, float4* x) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t s = (uint32_t)(s0 + u * SGN);
            if (h < G && s < (uint32_t)S) {
                const auto a = __builtin_amdgcn_raw_buffer_load_b64(rml, (int)((s * 32 + 2 * h) * 4), 0,
                                                                    kScopeDevice);
                const auto y = __builtin_amdgcn_raw_buffer_load_b128(
                    ro, (int)(((s * 16 + h) * D + 4 * f) * 4), 0, kScopeDevice);
                m[u] = __uint_as_float(a[0]);
                ls[u] = __uint_as_float(a[1]);
                x[u] = float4{__uint_as_float(y[0]), __uint_as_float(y[1]), __uint_as_float(y[2]),
                              __uint_as_float(y[3])};
            } else {
                m[u] = -INFINITY;
                ls[u] = 0.0f;
                x[u] = float4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    auto accumulate = [&](float M, const float* m, const float* ls, const float4* x, float& l, float4& o) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = m[u] == -INFINITY ? 0.0f : fast_exp2(m[u] - M);
            l += w * ls[u];
            o.x += w * x[u].x;
            o.y += w * x[u].y;
            o.z += w * x[u].z;
            o.w += w * x[u].w;
        }
    };
    auto row_max = [&](float mx) {
        lds[tid] = mx;
        __syncthreads();
        float M = lds[c];
#pragma unroll
        for (int g = 1; g < SGN; ++g) M = fmaxf(M, lds[g * NC + c]);
        return M;
    };
    float l = 0.0f;
    float4 o = {0.f, 0.f, 0.f, 0.f};
    if (S <= U * SGN) {
        // (m, l) of every (split, head) with one 8-byte load each (thread
        // s G + h), shared through LDS; the o of this thread's splits
        float* mlds = lds + 6 * NTHR;                 // [S][GP][2]
        float2 mlv = {0.0f, 0.0f};
        if (tid < S * G) {
            const int s = tid / G, hh = tid - (tid / G) * G;
            const auto a = __builtin_amdgcn_raw_buffer_load_b64(rml, (int)((s * 32 + 2 * hh) * 4), 0, kScopeDevice);
            mlv = float2{__uint_as_float(a[0]), __uint_as_float(a[1])};
        }
        float4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t s = (uint32_t)(sg + u * SGN);
            if (h < G && s < (uint32_t)S) {
                const auto y = __builtin_amdgcn_raw_buffer_load_b128(
                    ro, (int)(((s * 16 + h) * D + 4 * f) * 4), 0, kScopeDevice);
                x[u] = float4{__uint_as_float(y[0]), __uint_as_float(y[1]), __uint_as_float(y[2]),
                              __uint_as_float(y[3])};
            } else {
                x[u] = float4{0.f, 0.f, 0.f, 0.f};
            }
        }
        if (tid < S * G) {
            const int s = tid / G, hh = tid - (tid / G) * G;
            *(float2*)&mlds[(s * GP + hh) * 2] = mlv;
        }
        __syncthreads();
        float m[U], ls[U];
        float M = -INFINITY;
        if (h < G) {
            for (int s = 0; s < S; ++s) M = fmaxf(M, mlds[(s * GP + h) * 2]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = sg + u * SGN;
            const bool ok = h < G && s < S;
            m[u] = ok ? mlds[(s * GP + h) * 2] : -INFINITY;
            ls[u] = ok ? mlds[(s * GP + h) * 2 + 1] : 0.0f;
        }
        if (M != -INFINITY) accumulate(M, m, ls, x, l, o);
    } else {
        float mx = -INFINITY;
        if (h < G) {
            for (int s0 = sg; s0 < S; s0 += U * SGN) {
                float m[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t s = (uint32_t)(s0 + u * SGN);
                    m[u] = s < (uint32_t)S ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                                  rml, (int)((s * 32 + 2 * h) * 4), 0, kScopeDevice))
                                           : -INFINITY;
                }
#pragma unroll
                for (int u = 0; u < U; ++u) mx = fmaxf(mx, m[u]);
            }
        }
        const float M = row_max(mx);
        if (h < G && M != -INFINITY) {
            for (int s0 = sg; s0 < S; s0 += U * SGN) {
                float m[U], ls[U];
                float4 x[U];
                load_states(s0, m, ls, x);
                accumulate(M, m, ls, x, l, o);
            }
        }
    }
    __syncthreads();                              // every thread has read the maxima
    lds[tid] = l;
    *(float4*)&lds[2 * NTHR + 4 * tid] = o;
    __syncthreads();
    if (sg != 0 || h >= G) return;
#pragma unroll
    for (int g = 1; g < SGN; ++g) {
        const int t = g * NC + c;
        l += lds[t];
        const float4 y = *(const float4*)&lds[2 * NTHR + 4 * t];
        o.x += y.x;
        o.y += y.y;
        o.z += y.z;
        o.w += y.w;
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t* dst = (uint16_t*)p.out + (b * p.Hq + kvh * G + h) * D + 4 * f;
    const uint16_t hv[4] = {f32_to_f16(o.x * inv), f32_to_f16(o.y * inv), f32_to_f16(o.z * inv),
                            f32_to_f16(o.w * inv)};
    if ((reinterpret_cast<uintptr_t>(p.out) & 7) == 0) {
        *(uint2*)dst = uint2{(uint32_t)hv[0] | ((uint32_t)hv[1] << 16), (uint32_t)hv[2] | ((uint32_t)hv[3] << 16)};
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = hv[q];
    }
}

}  // namespace qkv
