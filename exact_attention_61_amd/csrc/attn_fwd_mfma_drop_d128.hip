// Instantiation of the MFMA attention forward kernel with dropout on the
// probabilities, head dimension 128.
#include "attn_fwd_mfma.hpp"

namespace mi_attn {

hipError_t launch_mfma_drop_d128(const FwdParams& p, int in_dtype, int out_dtype,
                                 hipStream_t stream) {
    return launch_d<128, true>(p, in_dtype, out_dtype, stream);
}

}  // namespace mi_attn
