// Instantiation of the MFMA attention forward kernel with dropout on the
// probabilities, head dimension 64.
#include "attn_fwd_mfma.hpp"

namespace mi_attn {

hipError_t launch_mfma_drop_d64(const FwdParams& p, int in_dtype, int out_dtype,
                                hipStream_t stream) {
    return launch_d<64, true>(p, in_dtype, out_dtype, stream);
}

}  // namespace mi_attn
