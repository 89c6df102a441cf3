// Instantiation of the MFMA attention forward kernel for head dimension 64.
#include "attn_fwd_mfma.hpp"

namespace mi_attn {

hipError_t launch_mfma_d64(const FwdParams& p, int in_dtype, int out_dtype,
                          hipStream_t stream) {
    return launch_d<64>(p, in_dtype, out_dtype, stream);
}

int causal_split_pairs_d64(const FwdParams& p) { return causal_split_pairs<64>(p); }

int64_t split_floats_per_tile_d64() { return split_floats_per_tile<64>(); }

}  // namespace mi_attn
