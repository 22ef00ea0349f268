// Merge of split-key softmax states.  Each split s of a row left (m, l) and an
// unnormalised o[D] with
//   o = sum_j 2^(z_j - m) v_j,  l = sum_j 2^(z_j - m)   (z in log2 units),
// and the row's result is  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// M = max_s m_s (the merge of partial softmax states on the MLX page
// "add fast::quantized_kv_update", sdpa_vector.h quant_sdpa_vector, applied
// across workgroups).  A row with no visible key (every m_s = -inf) gives 0.
//
// Workspace of a call: [tickets: one uint32 per tile, padded to 256 bytes]
// [ml: tiles x S x 16 x 2] [o: tiles x S x 16 x D] (fp32).  Either the
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

// Bytes of the ticket area at the start of a workspace.
inline size_t ticket_bytes(int64_t tiles) { return (size_t)((tiles * 4 + 255) / 256 * 256); }

struct SplitState {
    float m, l;
    float4 o;
};

// Online combination of two partial softmax states (log2 units).
__device__ __forceinline__ void combine_state(SplitState& a, float m, float l, float4 o) {
    if (m == -INFINITY) return;
    const float mm = fmaxf(a.m, m);
    const float fa = (a.m == -INFINITY) ? 0.0f : fast_exp2(a.m - mm);
    const float fb = fast_exp2(m - mm);
    a.l = a.l * fa + l * fb;
    a.o.x = a.o.x * fa + o.x * fb;
    a.o.y = a.o.y * fa + o.y * fb;
    a.o.z = a.o.z * fa + o.z * fb;
    a.o.w = a.o.w * fa + o.w * fb;
    a.m = mm;
}

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
// sg + SGN, ... (loads issued 8 at a time), the SGN group states combine
// through 'lds' (>= 6 NTHR floats) in group order, and column c's 4 fp16
// outputs are stored.  Same result for any workgroup that runs it.
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
    SplitState st{-INFINITY, 0.0f, {0.f, 0.f, 0.f, 0.f}};
    if (h < G) {
        for (int s0 = sg; s0 < S; s0 += U * SGN) {
            float m[U], l[U];
            float4 o[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t s = (uint32_t)(s0 + u * SGN);
                const auto a = __builtin_amdgcn_raw_buffer_load_b64(rml, (int)((s * 32 + 2 * h) * 4), 0,
                                                                    kScopeDevice);
                const auto x = __builtin_amdgcn_raw_buffer_load_b128(
                    ro, (int)(((s * 16 + h) * D + 4 * f) * 4), 0, kScopeDevice);
                m[u] = __uint_as_float(a[0]);
                l[u] = __uint_as_float(a[1]);
                o[u] = float4{__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]),
                              __uint_as_float(x[3])};
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (s0 + u * SGN < S) combine_state(st, m[u], l[u], o[u]);
        }
    }
    lds[tid] = st.m;
    lds[NTHR + tid] = st.l;
    *(float4*)&lds[2 * NTHR + 4 * tid] = st.o;
    __syncthreads();
    if (sg != 0 || h >= G) return;
#pragma unroll
    for (int g = 1; g < SGN; ++g) {
        const int t = g * NC + c;
        combine_state(st, lds[t], lds[NTHR + t], *(const float4*)&lds[2 * NTHR + 4 * t]);
    }
    const float inv = st.l > 0.0f ? 1.0f / st.l : 0.0f;
    uint16_t* dst = (uint16_t*)p.out + (b * p.Hq + kvh * G + h) * D + 4 * f;
    const uint16_t hv[4] = {f32_to_f16(st.o.x * inv), f32_to_f16(st.o.y * inv), f32_to_f16(st.o.z * inv),
                            f32_to_f16(st.o.w * inv)};
    if ((reinterpret_cast<uintptr_t>(p.out) & 7) == 0) {
        *(uint2*)dst = uint2{(uint32_t)hv[0] | ((uint32_t)hv[1] << 16), (uint32_t)hv[2] | ((uint32_t)hv[3] << 16)};
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = hv[q];
    }
}

}  // namespace qkv
