// Internal interface between the C-ABI host layer (qkv_api.cpp) and the HIP
// kernels.  Plain pointers and sizes only; every argument has already been
// validated by the host layer when a launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkv {

enum DType { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
enum Mode { MODE_AFFINE = 0, MODE_Q8_0 = 1, MODE_DENSE = 2, MODE_QSYM = 3 };

// Formats of the matrix-core and fast quantize kernels: affine 4/8-bit and
// Q8_0 with D a multiple of 64.  Every other format (affine 2/3/5/6-bit, the
// symmetric 4/5-bit blocks, head size 96) takes the general paths, which
// read codes as a bit stream; the narrow decode also takes the symmetric
// 4-bit blocks (narrow_decode_supported).
constexpr bool fast_format(int mode, int bits, int D) {
    return (mode == MODE_Q8_0 || (mode == MODE_AFFINE && (bits == 4 || bits == 8))) && D % 64 == 0;
}
enum MaskKind { MASK_NONE = 0, MASK_CAUSAL = 1, MASK_ADDITIVE = 2 };

// One tensor's worth of rows to quantize: source rows [B,H,T,D] with element
// strides, destination pack rows offset+t.
struct QuantJob {
    const void* x;
    int64_t xs0, xs1, xs2;          // element strides of b, h, t
    void* codes;
    void* scales;
    void* biases;                   // nullptr for Q8_0
    int64_t sb, sh, sl;             // pack strides in rows
};

struct QuantLaunch {
    QuantJob job[2];                // K (and V for append)
    int64_t H, T, offset;
    int64_t BH;                     // B*H
    int64_t rows;                   // B*H*T
};

// Read-only view of a pack for attention.
struct PackView {
    const void* codes;
    const void* scales;
    const void* biases;
    int64_t sb, sh, sl;             // strides in rows
};

struct AttnLaunch {
    const void* q;
    void* out;
    PackView k, v;
    int64_t Hq, Hk, Lq, L;
    int32_t G;                      // Hq / Hk
    int32_t gs_log2;                // log2(group_size) (5 for Q8_0)
    float scale;
    int32_t mask_kind;
    const void* mask;
    int32_t mask_dtype;
    int64_t ms0, ms1, ms2, ms3;     // mask element strides
    int32_t S;                      // splits of the key range
    int64_t chunk;                  // keys per split
    int32_t n_rows;                 // G * Lq rows per (b, kv head)
    int32_t n_rt;                   // row tiles per (b, kv head)
    int32_t RT;                     // rows per tile
    int32_t wg_rows;                // rows per workgroup of the prefill kernel (64 or 128)
    float* part_ml;                 // [B*Hk*n_rt][S][16][2] (m, l) of each split
    float* part_o;                  // [B*Hk*n_rt][S][16][D] unnormalised o of each split
    uint32_t* tickets;              // [B*Hk*n_rt] fused-merge tickets (zero between calls)
    // decode with append (narrow decode): the new fp16 K/V token of each
    // (batch, kv head) at element offset b ns0 + h ns1 is quantized into pack
    // row L - 1 before the tile holding it is loaded
    int32_t append;
    const void* k_new;
    const void* v_new;
    int64_t ns0, ns1;
    // unfused composition (launch_attn_unfused)
    float* un_scores;               // [B*Hq][L] scores, then probabilities
    float* un_stats;                // [B*Hq][L/4096 chunks] (m, l) of the softmax
    float* un_partial;              // [un_chunks][B*Hq][D] P V sums per key chunk
    int32_t un_chunks;              // key chunks of the P V product
    int64_t un_chunk;               // keys per chunk
};

// Rows [0, L) of every (b, h) of a quantized pack (src) -> a dense fp16 pack
// (dst codes, same B, H, D), one launch.
struct DequantLaunch {
    const void* codes;
    const void* scales;
    const void* biases;
    int64_t sb, sh, sl;             // src strides in rows
    void* out;
    int64_t db, dh, dl;             // dst strides in rows
    int64_t H, L, rows;             // rows = B * H * L
    int32_t gs;                     // group size (32 for Q8_0)
};
hipError_t launch_dequantize(int mode, int bits, int group_size, int D, const DequantLaunch& p,
                             hipStream_t stream);

// Launchers (return hipGetLastError() of the launch).
hipError_t launch_quantize(int x_dtype, int mode, int bits, int group_size, int D,
                           const QuantLaunch& p, int njobs, hipStream_t stream);

hipError_t launch_attn_generic(int q_dtype, int mode, int bits, int D, int64_t B,
                               const AttnLaunch& p, hipStream_t stream);

// Matrix-core kernels for fp16 queries and fp16 scales.  matrix_supported
// tells whether one of them covers the arguments; decode_matrix_supported
// picks the single-query kernel (launch_attn_matrix) over the tiled prefill
// kernel (launch_prefill_matrix).  Both launchers return hipErrorNotSupported
// when no instantiation covers the arguments.
bool matrix_supported(int q_dtype, int mode, int bits, int group_size, int D, int G,
                      int64_t Lq);
bool decode_matrix_supported(int q_dtype, int mode, int bits, int group_size, int D, int G,
                             int64_t Lq);
hipError_t launch_attn_matrix(int mode, int bits, int D, int64_t B, const AttnLaunch& p,
                              hipStream_t stream);
hipError_t launch_prefill_matrix(int mode, int bits, int D, int64_t B, const AttnLaunch& p,
                                 hipStream_t stream);
// Rows per workgroup of the prefill kernel: 128 (each dequantized K/V tile
// serves twice the rows) once a (batch, kv head) has at least
// kPrefillWideMinRows GQA-packed rows, else 64.
constexpr int kPrefillRows = 64;
constexpr int kPrefillRowsWide = 128;
constexpr int kPrefillWideMinRows = 256;
// Keys of one tile per wave of the single-query kernels: splits are rounded
// to a multiple of it.
int decode_matrix_key_quantum();
// Single-query kernel for GQA factors up to 4 (4x4x4 matrix tiles, one key
// per lane); used ahead of launch_attn_matrix where it applies.
bool narrow_decode_supported(int q_dtype, int mode, int bits, int group_size, int D, int G,
                             int64_t Lq);
int narrow_decode_key_quantum();

// Single-query decode (fp16 queries, G <= 4) for the formats without a
// matrix-core kernel: the bit-stream codes, the symmetric blocks and head
// size 96 (launch_attn_stream; its split states use the 16-row layout of
// the merge kernels).
bool stream_decode_supported(int q_dtype, int mode, int bits, int group_size, int scale_dtype, int D,
                             int G, int64_t Lq);
int stream_decode_key_quantum();
hipError_t launch_attn_stream(int mode, int bits, int D, int64_t B, const AttnLaunch& p,
                              hipStream_t stream);
hipError_t launch_attn_narrow(int mode, int bits, int D, int64_t B, const AttnLaunch& p,
                              hipStream_t stream);

// The unfused composition for one query per head (scores, softmax, P V over
// key chunks, sum of the chunks): fp32/fp16/bf16 queries, affine 4/8-bit or
// Q8_0 caches, D in {64, 128, 256}, G <= 16.  unfused_chunk_keys gives the
// keys per P V chunk (a power of two in [64, 1024], G rounded up to a power
// of two times it at most 4096).
int unfused_chunk_keys(int64_t B, int64_t Hk, int64_t L, int G);
int64_t unfused_stats_floats(int64_t B, int64_t Hq, int64_t L);
hipError_t launch_attn_unfused(int q_dtype, int mode, int bits, int D, int64_t B, const AttnLaunch& p,
                               hipStream_t stream);

// The device address of this GPU's static split workspace
// (QKV_STATIC_SCRATCH_BYTES, its ticket header zeroed on 'stream' at the first
// use on the device).  The stream must belong to the current device
// (hipErrorInvalidDevice otherwise).
hipError_t static_scratch(hipStream_t stream, void** addr);

}  // namespace qkv
