/*
 * qkv.h -- C ABI of libqkv.so: scaled-dot-product attention over a
 * group-quantized KV cache on AMD Instinct MI355X (gfx950).
 *
 * Operations (names follow MLX's quantized_kv_update /
 * quantized_scaled_dot_product_attention and llama.cpp's Q8_0 KV cache):
 *   qkv_quantize       quantize K or V rows into a pack
 *   qkv_update_append  quantize new K and V tokens into a cache at an offset
 *   qsdpa_decode       softmax(scale q K^T + mask) V for one query per head
 *   qsdpa_prefill      the same for Lq >= 1 queries, optional causal mask
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *    never allocates, frees or synchronises; 'stream' is a hipStream_t passed
 *    as void* (NULL = the default stream) and every call is stream-ordered.
 *  - Validation is synchronous and complete before anything is enqueued: on
 *    any status other than QKV_OK no output, cache or workspace byte is
 *    touched, and qkv_last_error() holds a message (thread-local).  A kernel
 *    fault surfaces at the caller's next synchronisation, as with any HIP
 *    launch.  No C++ exception crosses this boundary.
 *  - Tensors are row-major.  A "row" is one token of one head: D values.
 *  - Floating dtypes: QKV_F32, QKV_F16 (IEEE binary16), QKV_BF16.
 *
 * Cache format ("pack")
 * ---------------------
 *  QKV_AFFINE (MLX page "add fast::quantized_kv_update", kernels/quantized.h
 *  affine quantize and sdpa_vector.h load_keys/load_values): per group of
 *  group_size consecutive values of a row, a scale s and a bias b stored in
 *  scale_dtype and unsigned codes c in [0, 2^bits - 1]; the value is
 *  s * c + b.  Codes are packed LSB-first into little-endian uint32 words:
 *  element j of a row is bits [j*bits, (j+1)*bits) of word j / (32/bits).
 *  Quantization: s = max((max - min) / (2^bits - 1), T(1e-7)) rounded to T,
 *  b = min rounded to T, c = clamp(round_half_even((x - b) / s), 0, 2^bits-1)
 *  computed in IEEE fp32 from the stored s and b.
 *
 *  QKV_Q8_0 (llama.cpp page "Metal: Optimize q8_0 KV - #25556"): blocks of 32
 *  consecutive values of a row share one fp16 scale d = fp16(amax / 127);
 *  codes are signed int8 c = clamp(round_half_even(x / d), -127, 127) (0 when
 *  d == 0); the value is d * c.  Codes are stored one byte per value in a
 *  codes plane, scales in a separate plane (biases == NULL).
 *
 *  Layout of a pack with B batches, H heads, capacity L_cap, head size D:
 *    codes  : row r at byte offset r * row_bytes, row_bytes = D*bits/8
 *    scales : row r at element offset r * (D / group_size)
 *    biases : same as scales (affine only)
 *  where r = b*stride_b + h*stride_h + l*stride_l (strides in ROWS; the
 *  dense layout [B,H,L_cap] is {H*L_cap, L_cap, 1}).
 *  Requirements: codes 16-byte aligned; scales/biases aligned to one row
 *  of scales (min(16, (D / group_size) * element size) bytes); D in
 *  {64, 128, 256}; bits in {4, 8} with group_size in
 *  {32, 64, 128} dividing D (affine), bits 8 and group_size 32 (Q8_0);
 *  affine scale_dtype equal to the dtype of the values it was made from.
 */
#ifndef QKV_H
#define QKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKV_ABI_VERSION 2

typedef enum {
    QKV_OK = 0,
    QKV_EINVAL = 1,        /* bad argument: null/misaligned pointer, shape, range, overlap */
    QKV_EUNSUPPORTED = 2,  /* valid but not instantiated (D, bits, group, dtype, G) */
    QKV_EWORKSPACE = 3,    /* workspace smaller than qsdpa_workspace_bytes() */
    QKV_EHIP = 4           /* the HIP launch itself failed */
} qkv_status;

typedef enum { QKV_F32 = 0, QKV_F16 = 1, QKV_BF16 = 2 } qkv_dtype;
typedef enum { QKV_AFFINE = 0, QKV_Q8_0 = 1 } qkv_mode;
typedef enum { QKV_MASK_NONE = 0, QKV_MASK_CAUSAL = 1, QKV_MASK_ADDITIVE = 2 } qkv_mask_kind;

/* Kernel selection for the attention calls.  AUTO picks the fastest kernel
 * instantiated for the arguments; GENERIC is the plain vector kernel (every
 * supported combination); MATRIX uses the gfx950 matrix cores (fp16 queries). */
typedef enum { QKV_ALGO_AUTO = 0, QKV_ALGO_GENERIC = 1, QKV_ALGO_MATRIX = 2 } qkv_algo;

typedef struct {
    int32_t mode;          /* qkv_mode */
    int32_t bits;          /* AFFINE: 4 | 8.  Q8_0: 8 */
    int32_t group_size;    /* AFFINE: 32 | 64 | 128.  Q8_0: 32 */
    int32_t scale_dtype;   /* qkv_dtype of scales/biases.  Q8_0: QKV_F16 */
    int64_t B, H, L_cap, D;
    void* codes;
    void* scales;
    void* biases;          /* AFFINE only; NULL for Q8_0 */
    int64_t stride_b, stride_h, stride_l;   /* in rows */
} qkv_pack;

/* Options of the attention calls; a NULL pointer means all defaults.
 * timing_events: an optional pair of hipEvent_t handles (created by the
 * caller, with timing enabled).  When both are non-NULL the call records [0]
 * on its stream right before the attention kernel and [1] right after it,
 * before the split merge kernel, so that the caller can time the attention
 * kernel alone with hipEventElapsedTime.  NULL (the default) records nothing. */
typedef struct {
    int32_t num_splits;    /* key-range partitions per (batch, kv head, row tile); 0 = automatic */
    int32_t algo;          /* qkv_algo */
    void* timing_events[2];
} qkv_attn_opts;

/* Quantize x[B,H,L,D] (element strides x_strides = {b, h, l}; D contiguous,
 * strides multiples of 8, x 16-byte aligned) into rows [0, L) of dst, whose
 * B, H, D must match.  x_dtype must equal dst->scale_dtype for AFFINE.
 * Errors: EINVAL (null pointers, L > L_cap, misalignment, shape mismatch),
 * EUNSUPPORTED (format outside the instantiated set). */
qkv_status qkv_quantize(const void* x, int32_t x_dtype, const int64_t x_strides[3], int64_t L,
                        const qkv_pack* dst, void* stream);

/* Append: for every b < B, h < H, t < T, quantize k_new[b,h,t,:] into row
 * offset+t of k_cache and v_new[b,h,t,:] into row offset+t of v_cache (the
 * same bits as quantizing that row alone; other rows are untouched).  One
 * launch covers K and V.  new_strides = element strides {b, h, t} shared by
 * k_new and v_new.  (MLX page "add fast::quantized_kv_update": fast::kv_update
 * and the kv_update kernel quantize the new keys and values into the cache
 * at 'offset'.)  Errors: EINVAL when offset < 0, T < 1, offset + T > L_cap,
 * K/V packs disagree in B, H, D or format, or on the rules of qkv_quantize. */
qkv_status qkv_update_append(const void* k_new, const void* v_new, int32_t dtype,
                             const int64_t new_strides[3], int64_t T, int64_t offset,
                             const qkv_pack* k_cache, const qkv_pack* v_cache, void* stream);

/* Bytes of workspace the attention calls need for these sizes (0 when no
 * key partitioning is used): a ticket area (4 bytes per batch x kv head x
 * row tile, rounded up to 256 bytes), then per row tile and split the partial
 * softmax state (m, l) and an unnormalised output row.  The ticket area must
 * hold zeros when the workspace is first used (zero-fill the workspace once
 * after allocating it); every call leaves it zero.  The partial states need no
 * initialisation: a call writes them and either merges them in the same
 * kernel (the last workgroup of each batch x kv head, counted by its ticket)
 * or with the split merge kernel it launches next on the same stream.  Calls
 * that may overlap (different streams) need separate workspaces.  It must be
 * 256-byte aligned. */
size_t qsdpa_workspace_bytes(int64_t B, int64_t Hq, int64_t Lq, int64_t D, int64_t L,
                             const qkv_pack* k, int32_t q_dtype, const qkv_attn_opts* opts);

/* Kernels a plan can name (qkv_attn_plan.kernel). */
typedef enum {
    QKV_KERNEL_GENERIC = 0,        /* any dtype / format, CUDA-core arithmetic */
    QKV_KERNEL_DECODE = 1,         /* single query, fp16, GQA factor <= 16, 16x16x32 MFMA */
    QKV_KERNEL_DECODE_NARROW = 2,  /* single query, fp16, GQA factor <= 4, 4x4x4 MFMA */
    QKV_KERNEL_PREFILL = 3         /* 64-row tiles, fp16, K/V dequantized into LDS */
} qkv_kernel;

/* The launch plan an attention call with these arguments would use:
 * the algorithm class (QKV_ALGO_GENERIC or QKV_ALGO_MATRIX) and the kernel
 * (qkv_kernel), the key splits, the (GQA-packed) query rows per workgroup
 * and the workspace size.  Errors: EINVAL for null pointers or shapes that
 * the attention calls would reject as such. */
typedef struct {
    int32_t algo;
    int32_t num_splits;
    int32_t row_tile;
    int32_t kernel;
    int64_t keys_per_split;
    size_t workspace_bytes;
} qkv_attn_plan;

qkv_status qsdpa_plan(int64_t B, int64_t Hq, int64_t Lq, int64_t D, int64_t L, const qkv_pack* k,
                      int32_t q_dtype, const qkv_attn_opts* opts, qkv_attn_plan* plan);

/* Decode: q, out [B,Hq,1,D] contiguous in q_dtype; attends keys [0, L) of
 * the packs (L <= L_cap); query head h uses kv head h / (Hq/Hk).
 *   out = softmax(scale * q K^T + mask) V   (softmax over the L keys)
 * with K, V the dequantized packs and the scale applied in fp32 (MLX page
 * "add fast::quantized_kv_update": fast.cpp
 * quantized_scaled_dot_product_attention and sdpa_vector.h
 * quant_sdpa_vector).  mask: NULL or additive, element (b,h,0,j) at
 * b*ms[0]+h*ms[1]+j*ms[3] of mask_dtype (stride 0 = broadcast); unlike the
 * page's fused single-query path, the mask is applied.  A row whose keys are
 * all masked to -inf produces zeros.  out must not overlap q, the packs or
 * the workspace.  Errors: EINVAL (shapes, Hq % Hk != 0, L < 1 or > L_cap,
 * packs mismatch, overlap), EUNSUPPORTED, EWORKSPACE. */
qkv_status qsdpa_decode(const void* q, int32_t q_dtype, int64_t B, int64_t Hq, int64_t D,
                        const qkv_pack* k, const qkv_pack* v, int64_t L, float scale,
                        const void* mask, int32_t mask_dtype, const int64_t mask_strides[4],
                        void* out, void* workspace, size_t workspace_bytes,
                        const qkv_attn_opts* opts, void* stream);

/* Prefill: q, out [B,Hq,Lq,D] contiguous; keys [0, L).  QKV_MASK_CAUSAL hides
 * key j from query i when j > L - Lq + i (the queries are the last Lq
 * positions); QKV_MASK_ADDITIVE adds mask element (b,h,i,j) at
 * b*ms[0]+h*ms[1]+i*ms[2]+j*ms[3].  Lq = 1 gives the same result as
 * qsdpa_decode.  Errors as qsdpa_decode, plus EINVAL when causal and L < Lq. */
qkv_status qsdpa_prefill(const void* q, int32_t q_dtype, int64_t B, int64_t Hq, int64_t Lq,
                         int64_t D, const qkv_pack* k, const qkv_pack* v, int64_t L, float scale,
                         int32_t mask_kind, const void* mask, int32_t mask_dtype,
                         const int64_t mask_strides[4], void* out, void* workspace,
                         size_t workspace_bytes, const qkv_attn_opts* opts, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* qkv_last_error(void);

/* QKV_ABI_VERSION of the loaded library. */
int32_t qkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QKV_H */
