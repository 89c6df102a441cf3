// Instantiation of the MFMA attention forward kernel for head dimension 128.
#include "attn_fwd_mfma.hpp"

namespace mi_attn {

hipError_t launch_mfma_d128(const FwdParams& p, const SplitOrder& so,
                          int in_dtype, int out_dtype, hipStream_t stream) {
    return launch_d<128>(p, so, in_dtype, out_dtype, stream);
}

int split_tiles_d128(const FwdParams& p, int cus) { return split_tiles<128>(p, cus); }

void split_order_d128(const FwdParams& p, int hs, SplitOrder& so) {
    split_order<128>(p, hs, so);
}

int64_t split_floats_per_tile_d128() { return split_floats_per_tile<128>(); }

}  // namespace mi_attn
