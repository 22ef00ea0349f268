// Merge of split-key softmax states.  Each split s of a row left (m, l) and an
// unnormalised o[D] with
//   o = sum_j 2^(z_j - m) v_j,  l = sum_j 2^(z_j - m)   (z in log2 units),
// and the row's result is  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// M = max_s m_s (the merge of partial softmax states on the MLX page
// "add fast::quantized_kv_update", sdpa_vector.h quant_sdpa_vector, applied
// across workgroups).  A row with no visible key (every m_s = -inf) gives 0.
//
// Workspace of a call: [ml: tiles x S x 16 x 2] [o: tiles x S x 16 x D]
// (fp32).  The attention kernels write it; merge_splits_kernel, launched next
// on the same stream, reads it (kernel order is the only synchronisation).
#pragma once

#include "qkv_device.hpp"
#include "qkv_internal.hpp"

namespace qkv {

constexpr int kMaxSplits = 256;

hipError_t launch_merge(int q_dtype, int D, int64_t B, const AttnLaunch& p, hipStream_t stream);

}  // namespace qkv
