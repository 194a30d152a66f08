// Split-kernel instantiations for head sizes with 16 code words per row
// (head_size 64, or padded from smaller ones).
#include "decode_kernel.h"

namespace q8kv {

hipError_t launch_split_hs16(const DecodeArgs& a, const SplitConsts& c, uint32_t nbm1, dim3 grid, hipStream_t st,
                             bool vis, bool tiled, bool exact) {
    return exact ? launch_split_g<16, true>(a, c, nbm1, grid, st, vis, tiled)
                 : launch_split_g<16, false>(a, c, nbm1, grid, st, vis, tiled);
}

}  // namespace q8kv
