// Split-kernel instantiations for head sizes with 64 code words per row
// (head_size 256, or padded from smaller ones).
#include "decode_kernel.h"

namespace q8kv {

const void* split_kernel_hs64(bool vis, bool tiled, bool exact, uint32_t group, uint32_t seg_rows) {
    return exact ? split_kernel_g<64, true>(vis, tiled, group, seg_rows)
                 : split_kernel_g<64, false>(vis, tiled, group, seg_rows);
}

}  // namespace q8kv
