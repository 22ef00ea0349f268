// Matrix-core (MFMA) attention kernels for fp16 queries on gfx950.
#include "qkv_device.hpp"
#include "qkv_internal.hpp"

namespace qkv {

bool matrix_supported(int, int, int, int, int, int, int64_t) { return false; }

hipError_t launch_attn_matrix(int, int, int, int64_t, const AttnLaunch&, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace qkv
