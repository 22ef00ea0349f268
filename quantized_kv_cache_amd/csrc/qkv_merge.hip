// Split merge kernels.  Many splits: one workgroup per (row tile, row, 64-d
// chunk of the output row): grid x = tile, y = row, z = chunk.  Its 256 threads are 16
// float4 columns x 16 split groups, so a thread reads at most S/16 split
// states (all its loads issued before it waits: one memory round trip for
// S <= 128).  The row's maximum M over the splits' m (log2 units) comes
// first, then every state is weighted by 2^(m_s - M) and the weighted sums
// of the split groups are added through LDS, so no split waits on another's
// rescaling; the chunk is written in the query dtype.
#include <algorithm>

#include "qkv_merge.hpp"

namespace qkv {

namespace {

// Every argument the merge reads, fetched in one round trip at the start.
__device__ __forceinline__ void pin_args(const AttnLaunch& p) {
    pin_sgpr(p.n_rt); pin_sgpr(p.n_rows); pin_sgpr(p.Hk); pin_sgpr(p.G); pin_sgpr(p.S);
    pin_sgpr(p.part_ml); pin_sgpr(p.part_o); pin_sgpr(p.out); pin_sgpr(p.Hq); pin_sgpr(p.Lq);
}

// Output row r of 16-row tile 'tile' (tile = (b Hk + kvh) n_rt + rt): its
// GQA-packed row pr = 16 rt + r, query i = pr / G and head h = kvh G + pr % G.
// Tiles number below 2^24 (the grid's x size), so 32-bit division suffices.
struct Row {
    int pr;
    int64_t b, kvh, i, h;
};
__device__ __forceinline__ Row locate(const AttnLaunch& p, uint32_t tile, int r) {
    const uint32_t nrt = (uint32_t)p.n_rt, hk = (uint32_t)p.Hk, g = (uint32_t)p.G;
    const uint32_t bk = tile / nrt, rt = tile - bk * nrt;
    const uint32_t pr = rt * 16u + (uint32_t)r;
    const uint32_t b = bk / hk, kvh = bk - b * hk;
    const uint32_t i = pr / g;
    return Row{(int)pr, (int64_t)b, (int64_t)kvh, (int64_t)i, (int64_t)(kvh * g + (pr - i * g))};
}

constexpr int MC = 16;          // float4 columns per workgroup (64 d)
constexpr int SG = 256 / MC;    // split groups
constexpr int U = 8;            // loads in flight per batch

template <int QT, int D>
__global__ __launch_bounds__(256) void merge_splits_kernel(AttnLaunch p) {
    constexpr int F4 = D / 4;
    __shared__ float red_m[256];
    __shared__ float red_l[256];
    __shared__ float4 red_o[256];

    pin_args(p);
    const int64_t tile = blockIdx.x;
    const int r = blockIdx.y;
    const Row rw = locate(p, (uint32_t)tile, r);
    if (rw.pr >= p.n_rows) return;                // whole workgroup leaves together
    const int64_t b = rw.b, kvh = rw.kvh, i = rw.i, h = rw.h;
    const int f = blockIdx.z * MC + threadIdx.x % MC;   // float4 column of the row
    const int sg = threadIdx.x / MC;
    const int S = p.S;
    const bool f_ok = f < F4;                     // D = 96: the last chunk is 32 d wide

    // The row's maximum first, then the sums weighted by 2^(m_s - M): no
    // rescaling chain between splits.  With at most U SG splits every state
    // of the thread is loaded in one round trip before the maximum is
    // reduced; more splits take a pass for the maxima and one for the sums.
    // Both forms add in the same order, so they give the same bits.
    const float2* ml = (const float2*)p.part_ml + (tile * S * 16 + r);
    const float4* po = (const float4*)p.part_o + ((tile * S * 16 + r) * F4 + f);
    float l = 0.0f;
    float4 o = {0.f, 0.f, 0.f, 0.f};
    if (S <= U * SG) {
        float2 a[U];
        float4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = sg + u * SG;
            a[u] = s < S ? ml[(int64_t)s * 16] : float2{-INFINITY, 0.0f};
            x[u] = (s < S && f_ok) ? po[(int64_t)s * 16 * F4] : float4{0.f, 0.f, 0.f, 0.f};
        }
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) mx = fmaxf(mx, a[u].x);
        red_m[threadIdx.x] = mx;
        __syncthreads();
        float M = red_m[threadIdx.x % MC];
#pragma unroll
        for (int g = 1; g < SG; ++g) M = fmaxf(M, red_m[g * MC + threadIdx.x % MC]);
        if (M != -INFINITY && f_ok) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float w = a[u].x == -INFINITY ? 0.0f : fast_exp2(a[u].x - M);
                l += w * a[u].y;
                o.x += w * x[u].x;
                o.y += w * x[u].y;
                o.z += w * x[u].z;
                o.w += w * x[u].w;
            }
        }
    } else {
        float mx = -INFINITY;
        for (int s0 = sg; s0 < S; s0 += U * SG) {
            float a[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int s = s0 + u * SG;
                a[u] = s < S ? ml[(int64_t)s * 16].x : -INFINITY;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) mx = fmaxf(mx, a[u]);
        }
        red_m[threadIdx.x] = mx;
        __syncthreads();
        float M = red_m[threadIdx.x % MC];
#pragma unroll
        for (int g = 1; g < SG; ++g) M = fmaxf(M, red_m[g * MC + threadIdx.x % MC]);
        if (M != -INFINITY && f_ok) {
            for (int s0 = sg; s0 < S; s0 += U * SG) {
                float2 a[U];
                float4 x[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int s = s0 + u * SG;
                    if (s < S) {
                        a[u] = ml[(int64_t)s * 16];
                        x[u] = po[(int64_t)s * 16 * F4];
                    } else {
                        a[u] = float2{-INFINITY, 0.0f};
                        x[u] = float4{0.f, 0.f, 0.f, 0.f};
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float w = a[u].x == -INFINITY ? 0.0f : fast_exp2(a[u].x - M);
                    l += w * a[u].y;
                    o.x += w * x[u].x;
                    o.y += w * x[u].y;
                    o.z += w * x[u].z;
                    o.w += w * x[u].w;
                }
            }
        }
    }
    red_l[threadIdx.x] = l;
    red_o[threadIdx.x] = o;
    __syncthreads();
    if (sg != 0 || !f_ok) return;
#pragma unroll
    for (int g = 1; g < SG; ++g) {
        const int t = g * MC + threadIdx.x;
        l += red_l[t];
        const float4 y = red_o[t];
        o.x += y.x;
        o.y += y.y;
        o.z += y.z;
        o.w += y.w;
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const int64_t ob = ((b * p.Hq + h) * p.Lq + i) * D + 4 * f;
    store_from_f32<QT>(p.out, ob, o.x * inv);
    store_from_f32<QT>(p.out, ob + 1, o.y * inv);
    store_from_f32<QT>(p.out, ob + 2, o.z * inv);
    store_from_f32<QT>(p.out, ob + 3, o.w * inv);
}

// Few splits (S <= kSmallS, the prefill case): one thread per float4 column
// of a row combines all S states itself; a workgroup covers 256 / (D / 4)
// rows, so every load is a full-row, coalesced access.
constexpr int kSmallS = 8;

template <int QT, int D>
__global__ __launch_bounds__(256) void merge_splits_small(AttnLaunch p) {
    constexpr int F4 = D / 4;
    constexpr int RPW = 256 / F4;                 // rows per workgroup
    pin_args(p);
    const int64_t tile = blockIdx.x;
    if (threadIdx.x >= RPW * F4) return;          // D = 96: 240 of the 256 threads
    const int r = blockIdx.y * RPW + threadIdx.x / F4;
    if (r >= 16) return;
    const Row rw = locate(p, (uint32_t)tile, r);
    if (rw.pr >= p.n_rows) return;
    const int64_t b = rw.b, kvh = rw.kvh, i = rw.i, h = rw.h;
    const int f = threadIdx.x % F4;
    const int S = p.S;
    const float2* ml = (const float2*)p.part_ml + (tile * S * 16 + r);
    const float4* po = (const float4*)p.part_o + ((tile * S * 16 + r) * F4 + f);
    float2 a[kSmallS];
    float4 o[kSmallS];
#pragma unroll
    for (int s = 0; s < kSmallS; ++s) {
        if (s < S) {
            a[s] = ml[(int64_t)s * 16];
            o[s] = po[(int64_t)s * 16 * F4];
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kSmallS; ++s)
        if (s < S) M = fmaxf(M, a[s].x);
    float l = 0.0f;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSmallS; ++s) {
        if (s < S && a[s].x != -INFINITY) {
            const float w = fast_exp2(a[s].x - M);
            l += w * a[s].y;
            acc.x += w * o[s].x;
            acc.y += w * o[s].y;
            acc.z += w * o[s].z;
            acc.w += w * o[s].w;
        }
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const int64_t ob = ((b * p.Hq + h) * p.Lq + i) * D + 4 * f;
    store_from_f32<QT>(p.out, ob, acc.x * inv);
    store_from_f32<QT>(p.out, ob + 1, acc.y * inv);
    store_from_f32<QT>(p.out, ob + 2, acc.z * inv);
    store_from_f32<QT>(p.out, ob + 3, acc.w * inv);
}

template <int QT, int D>
hipError_t launch_small(int64_t B, const AttnLaunch& p, hipStream_t s) {
    constexpr int RPW = 256 / (D / 4);
    const unsigned rows = (unsigned)(p.n_rows < 16 ? p.n_rows : 16);
    dim3 grid((unsigned)(B * p.Hk * p.n_rt), (rows + RPW - 1) / RPW, 1);
    hipLaunchKernelGGL((merge_splits_small<QT, D>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int QT>
hipError_t launch_q(int D, int64_t B, const AttnLaunch& p, hipStream_t s) {
    if (p.S <= kSmallS) {
        switch (D) {
            case 64: return launch_small<QT, 64>(B, p, s);
            case 96: return launch_small<QT, 96>(B, p, s);
            case 128: return launch_small<QT, 128>(B, p, s);
            case 256: return launch_small<QT, 256>(B, p, s);
            default: return hipErrorNotSupported;
        }
    }
    // rows of a tile that exist: all 16 unless the (single) tile is short
    const unsigned rows = (unsigned)(p.n_rows < 16 ? p.n_rows : 16);
    dim3 grid((unsigned)(B * p.Hk * p.n_rt), rows, (unsigned)((D + 4 * MC - 1) / (4 * MC)));
    switch (D) {
        case 64: hipLaunchKernelGGL((merge_splits_kernel<QT, 64>), grid, dim3(256), 0, s, p); break;
        case 96: hipLaunchKernelGGL((merge_splits_kernel<QT, 96>), grid, dim3(256), 0, s, p); break;
        case 128: hipLaunchKernelGGL((merge_splits_kernel<QT, 128>), grid, dim3(256), 0, s, p); break;
        case 256: hipLaunchKernelGGL((merge_splits_kernel<QT, 256>), grid, dim3(256), 0, s, p); break;
        default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(int q_dtype, int D, int64_t B, const AttnLaunch& p, hipStream_t stream) {
    switch (q_dtype) {
        case DT_F32: return launch_q<DT_F32>(D, B, p, stream);
        case DT_F16: return launch_q<DT_F16>(D, B, p, stream);
        case DT_BF16: return launch_q<DT_BF16>(D, B, p, stream);
    }
    return hipErrorNotSupported;
}

// Zero fill of a workspace's ticket header (16-byte stores, grid-stride).
__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        p[i] = uint4{0u, 0u, 0u, 0u};
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    const size_t blocks = std::min<size_t>((n16 + 255) / 256, 1024);
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint4*)p, n16);
    return hipGetLastError();
}

}  // namespace qkv
