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
 *  Affine codes of 2, 3, 5 and 6 bits follow the pack factors and bytes per
 *  pack of the MLX CUDA page "Fixed mma and working dequant"
 *  (quantized_utils.cuh: 3 and 5 bits pack 8 values into 3 and 5 bytes, 6
 *  bits 4 values into 3 bytes): the codes of a row form one
 *  least-significant-bit-first stream, element j at bits [j*bits,
 *  (j+1)*bits), which for 2, 4 and 8 bits is the word layout above.
 *
 *  QKV_QSYM: symmetric blocks of 32 values at 4 or 5 bits, the rule of Q8_0
 *  with the code range of the width -- the reading taken for the Q4_0 and
 *  Q5_0 caches that the llama.cpp page names: d = fp16(amax / qmax) with
 *  qmax = 2^(bits-1) - 1, c = clamp(round_half_even(x / d), -qmax, qmax) (0
 *  when d == 0), the value d * c; codes are bits-wide two's complement in the
 *  row's bit stream, scales fp16 (group_size 32, biases NULL).  The affine
 *  4-bit and 5-bit formats with group_size 32 and fp16 scales play the role
 *  of Q4_1 and Q5_1 (a scale and a minimum per block of 32).
 *
 *  QKV_DENSE: the unquantized cache the pages compare against (the dense
 *  fp16 K/V of the MLX benchmark's sdpa baseline, sdpa_vector_bench.py; the
 *  F16 KV cache and the F16 scratch copies of the llama.cpp page): codes hold
 *  fp16 values, one per element (bits 16, group_size D, scale_dtype QKV_F16,
 *  scales and biases NULL).  Attention over dense packs takes fp16 queries.
 *
 *  Layout of a pack with B batches, H heads, capacity L_cap, head size D:
 *    codes  : row r at byte offset r * row_bytes, row_bytes = D*bits/8
 *    scales : row r at element offset r * (D / group_size)
 *    biases : same as scales (affine only)
 *  where r = b*stride_b + h*stride_h + l*stride_l (strides in ROWS; the
 *  dense layout [B,H,L_cap] is {H*L_cap, L_cap, 1}).
 *  Requirements: codes 16-byte aligned; scales/biases aligned to one row
 *  of scales (min(16, (D / group_size) * element size) bytes, a power of
 *  two); D in {64, 96, 128, 256} (96: affine, Q8_0 and QSYM); bits in
 *  {2, 3, 4, 5, 6, 8} with group_size in {32, 64, 128} dividing D (affine),
 *  bits 8 and group_size 32 (Q8_0), bits 4 or 5 and group_size 32 (QSYM);
 *  affine scale_dtype equal to the dtype of the values it was made from.
 *  The matrix-core kernels take affine 4/8-bit and Q8_0 packs with D in
 *  {64, 128, 256}; every other format runs on the generic kernel.
 */
#ifndef QKV_H
#define QKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKV_ABI_VERSION 6

typedef enum {
    QKV_OK = 0,
    QKV_EINVAL = 1,        /* bad argument: null/misaligned pointer, shape, range, overlap */
    QKV_EUNSUPPORTED = 2,  /* valid but not instantiated (D, bits, group, dtype, G) */
    QKV_EWORKSPACE = 3,    /* workspace smaller than qsdpa_workspace_bytes() */
    QKV_EHIP = 4           /* the HIP launch itself failed */
} qkv_status;

typedef enum { QKV_F32 = 0, QKV_F16 = 1, QKV_BF16 = 2 } qkv_dtype;
typedef enum { QKV_AFFINE = 0, QKV_Q8_0 = 1, QKV_DENSE = 2, QKV_QSYM = 3 } qkv_mode;
typedef enum { QKV_MASK_NONE = 0, QKV_MASK_CAUSAL = 1, QKV_MASK_ADDITIVE = 2 } qkv_mask_kind;

/* Kernel selection for the attention calls.  AUTO picks the fastest kernel
 * instantiated for the arguments; GENERIC is the plain vector kernel (every
 * supported combination); MATRIX uses the gfx950 matrix cores (fp16 queries).
 * UNFUSED (decode only, GQA factor <= 16) runs the composition that the MLX
 * page "add fast::quantized_kv_update" gives as the fallback of
 * quantized_scaled_dot_product_attention (mlx/fast.cpp) and times against the
 * fused kernel in sdpa_vector_bench.py (quant_attention): a quantized
 * matrix-vector product q K^T into an fp32 score buffer, a softmax over each
 * row, and a quantized vector-matrix product P V split over key chunks
 * (qvm_split_k on the MLX 1.0.0 Metal host page), then the sum of the
 * chunks, as four kernels; its workspace holds the scores and the chunk sums.
 * DEQUANT_F16 (fp16 queries, affine caches with fp16 scales or Q8_0) is the
 * strategy of the llama.cpp page "Metal: Optimize q8_0 KV - #25556" (merged
 * #27390, kernel_flash_attn_ext_dequant_to_f16): K and V rows [0, L) are
 * first dequantized into dense fp16 copies in the workspace (qkv_dequantize),
 * then the dense matrix-core attention runs on them. */
typedef enum { QKV_ALGO_AUTO = 0, QKV_ALGO_GENERIC = 1, QKV_ALGO_MATRIX = 2,
               QKV_ALGO_UNFUSED = 3, QKV_ALGO_DEQUANT_F16 = 4 } qkv_algo;

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
 * The operation is the group-wise affine quantize of the MLX page "add
 * fast::quantized_kv_update" (kernels/quantized.h affine_quantize: per group,
 * scale (max - min) / (2^bits - 1) floored at T(1e-7), bias = min, codes
 * packed as sdpa_vector.h load_keys reads them) and of the MLX CUDA page
 * "Fixed mma and working dequant" (quantized.cu affine_quantize), or the Q8_0
 * block of the llama.cpp page "Metal: Optimize q8_0 KV - #25556" (32 signed
 * int8 codes with one fp16 scale); the exact arithmetic is stated under
 * "Cache format" above.  L = 0 enqueues nothing.  dst rows >= L are not
 * touched.  The values must be finite: a NaN or an infinity in a group gives
 * unspecified codes and scale for that group (the other groups are exact).
 * Errors: EINVAL (null pointers, L > L_cap, misalignment, shape mismatch),
 * EUNSUPPORTED (format outside the instantiated set, or a source row stride
 * x_strides[2] * element size or a pack row stride of 2^27 bytes or more). */
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

/* Dequantize rows [0, L) of every (b, h) of a quantized pack into a dense
 * fp16 pack of the same B, H, D (L <= both capacities): element j of a row
 * becomes fp16(fp32(s) * c + fp32(b)) (affine, the product and the sum each
 * rounded in fp32, then rounded to fp16) or fp16(fp32(d) * c) (Q8_0) -- the
 * dequantization of the MLX page "add fast::quantized_kv_update"
 * (kernels/quantized.h: scale * code + bias) stored as the fp16 copy of the
 * llama.cpp page "Metal: Optimize q8_0 KV - #25556" (merged #27390,
 * kernel_flash_attn_ext_dequant_to_f16).  src must be AFFINE with fp16
 * scales, or Q8_0.  Errors: EINVAL (pack checks, dst not DENSE, shape
 * mismatch, L outside [0, capacity], src and dst overlapping), EUNSUPPORTED. */
qkv_status qkv_dequantize(const qkv_pack* src, int64_t L, const qkv_pack* dst, void* stream);

/* Bytes of workspace the attention calls need for these sizes (0 when no
 * key partitioning is used): a ticket header of QKV_TICKET_BYTES (one 32-bit
 * counter per batch x kv head, at the same place for every call), then per
 * row tile and split the partial softmax state (m, l) and an unnormalised
 * output row.  The ticket header must hold zeros when the workspace is first
 * used (zero-fill it after allocating, or call qsdpa_workspace_reset); every
 * call that completes leaves it zero.  The partial states need no
 * initialisation: a call writes them and either merges them in the same
 * kernel (the last workgroup of each batch x kv head, counted by its ticket)
 * or with the split merge kernel it launches next on the same stream.  Calls
 * that may overlap (different streams) need separate workspaces.  The
 * workspace must be 256-byte aligned and must not overlap q, out, the packs
 * or the mask. */
size_t qsdpa_workspace_bytes(int64_t B, int64_t Hq, int64_t Lq, int64_t D, int64_t L,
                             const qkv_pack* k, int32_t q_dtype, const qkv_attn_opts* opts);

#define QKV_TICKET_BYTES ((size_t)262144)

/* Zero-fills the ticket header of a workspace (its first QKV_TICKET_BYTES)
 * on 'stream' with a kernel, which a HIP graph may capture: for a workspace
 * just allocated, or one whose last call did not complete (a ticket left
 * non-zero would make later calls merge at the wrong moment).  Errors:
 * EINVAL for a null or misaligned workspace or workspace_bytes below
 * QKV_TICKET_BYTES; EHIP if the launch fails. */
qkv_status qsdpa_workspace_reset(void* workspace, size_t workspace_bytes, void* stream);

/* Kernels a plan can name (qkv_attn_plan.kernel). */
typedef enum {
    QKV_KERNEL_GENERIC = 0,        /* any dtype / format, CUDA-core arithmetic */
    QKV_KERNEL_DECODE = 1,         /* single query, fp16, GQA factor <= 16, 16x16x32 MFMA */
    QKV_KERNEL_DECODE_NARROW = 2,  /* single query, fp16, GQA factor <= 4, 4x4x4 MFMA */
    QKV_KERNEL_PREFILL = 3,        /* 64-row tiles, fp16, K/V dequantized into LDS */
    QKV_KERNEL_UNFUSED = 4,        /* scores, softmax, P V, chunk sum: four kernels */
    QKV_KERNEL_DECODE_STREAM = 5   /* single query, fp16, GQA factor <= 4, the formats without a
                                      matrix-core kernel (bit-stream codes, symmetric blocks,
                                      D = 96), VALU arithmetic; chosen under QKV_ALGO_AUTO */
} qkv_kernel;

/* The launch plan an attention call with these arguments would use:
 * the algorithm class (QKV_ALGO_GENERIC for the VALU kernels -- the generic
 * kernel and the bit-stream decode --, QKV_ALGO_MATRIX, QKV_ALGO_UNFUSED or
 * QKV_ALGO_DEQUANT_F16) and the kernel (qkv_kernel), the key splits (for the
 * unfused composition: the key chunks of its P V product), the (GQA-packed)
 * query rows per workgroup and the workspace size.  Errors: EINVAL for null pointers or shapes that
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
 * packs mismatch, overlap of out or the workspace with an input),
 * EUNSUPPORTED, EWORKSPACE. */
qkv_status qsdpa_decode(const void* q, int32_t q_dtype, int64_t B, int64_t Hq, int64_t D,
                        const qkv_pack* k, const qkv_pack* v, int64_t L, float scale,
                        const void* mask, int32_t mask_dtype, const int64_t mask_strides[4],
                        void* out, void* workspace, size_t workspace_bytes,
                        const qkv_attn_opts* opts, void* stream);

/* Decode with append: qkv_update_append of one new token per (batch, kv
 * head) at row 'offset' (k_new, v_new [B,Hk,1,D] in q_dtype, element strides
 * new_strides = {b, h, t}), then qsdpa_decode over keys [0, offset + 1) --
 * one step of a decoding loop over a quantized cache: the MLX page "add
 * fast::quantized_kv_update" appends the step's keys and values with
 * fast::quantized_kv_update (kv_update) and then attends the updated cache
 * with quantized_scaled_dot_product_attention.  The cache rows written are
 * the bits qkv_update_append writes, and out is what qsdpa_decode returns on
 * the updated packs with the same options.  On the matrix-core decodes (fp16
 * queries, GQA factor <= 16, affine 4/8-bit or Q8_0 codes, no mask) it is
 * one launch: the wave that loads the tile holding row 'offset' quantizes the
 * two new rows first; otherwise the append kernel runs before the decode.
 * Arguments and errors as qkv_update_append (T = 1, dtype = q_dtype) and
 * qsdpa_decode (L = offset + 1), and EINVAL when k_new or v_new overlaps
 * out, the packs or the workspace; size the workspace with qsdpa_plan or
 * qsdpa_workspace_bytes for L = offset + 1.  timing_events in opts bracket
 * the attention kernel (the fused one, or the decode after the append). */
qkv_status qsdpa_decode_append(const void* q, int32_t q_dtype, int64_t B, int64_t Hq, int64_t D,
                               const void* k_new, const void* v_new, const int64_t new_strides[3],
                               int64_t offset, const qkv_pack* k_cache, const qkv_pack* v_cache,
                               float scale, const void* mask, int32_t mask_dtype,
                               const int64_t mask_strides[4], void* out, void* workspace,
                               size_t workspace_bytes, const qkv_attn_opts* opts, void* stream);

/* qsdpa_decode for callers that cannot allocate (code under HIP graph
 * capture, serving loops that forbid hipMalloc): the same computation and
 * kernels, with the split workspace in a device array inside the library
 * instead of a caller's buffer.  The array holds QKV_STATIC_SCRATCH_BYTES;
 * each GPU has its own copy, resolved and its ticket header zeroed (with a
 * kernel on 'stream') at the first call on that device, and kept until the
 * process ends.  Nothing is allocated or freed by this call.  Every call on a
 * GPU shares that GPU's array and leaves its contents (tickets zero, split
 * states of the last call): calls that may overlap on one GPU (different
 * streams, or host threads) race and must not be issued.  'stream' must
 * belong to the current device.  Arguments and errors as qsdpa_decode, plus
 * EWORKSPACE when the call's plan needs more than QKV_STATIC_SCRATCH_BYTES
 * (then pass fewer splits in opts, or use qsdpa_decode with a workspace),
 * and EHIP when the device array cannot be resolved. */
#define QKV_STATIC_SCRATCH_BYTES ((size_t)(QKV_TICKET_BYTES + 16u * 1024u * 1024u))

qkv_status qsdpa_decode_static(const void* q, int32_t q_dtype, int64_t B, int64_t Hq, int64_t D,
                               const qkv_pack* k, const qkv_pack* v, int64_t L, float scale,
                               const void* mask, int32_t mask_dtype,
                               const int64_t mask_strides[4], void* out,
                               const qkv_attn_opts* opts, void* stream);

/* Prefill: q, out [B,Hq,Lq,D] contiguous; keys [0, L).
 *   out[b,h,i] = softmax_j(scale * q[b,h,i] . K[b,h/(Hq/Hk),j] + m_ij) V
 * for every query row i < Lq: the composition that the MLX page "add
 * fast::quantized_kv_update" gives for more than one query per head
 * (mlx/fast.cpp quantized_scaled_dot_product_attention, fallback:
 * quantized_matmul(q, K^T), plus the additive mask, softmax over the keys,
 * quantized_matmul with V, query heads grouped onto kv heads by a reshape),
 * with the scale applied in fp32 as in its fused kernel; and the prompt
 * processing over a Q8_0 cache of the llama.cpp page "Metal: Optimize q8_0
 * KV - #25556" (512-query prompt batches at 10K and 20K cache depth, the new
 * tokens being the last positions of the cache).  m_ij: QKV_MASK_NONE 0;
 * QKV_MASK_CAUSAL -inf when j > L - Lq + i (the queries are the last Lq
 * positions, bottom-right aligned); QKV_MASK_ADDITIVE mask element (b,h,i,j)
 * at b*ms[0]+h*ms[1]+i*ms[2]+j*ms[3] of mask_dtype.  A row with no visible
 * key produces zeros.  Lq = 1 gives the same result as qsdpa_decode.  out
 * must not overlap q, the packs or the workspace.  Errors as qsdpa_decode,
 * plus EINVAL when causal and L < Lq. */
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
