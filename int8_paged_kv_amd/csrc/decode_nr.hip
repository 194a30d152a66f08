// Split-kernel instantiations of the decode step with the per-head RMSNorm +
// partial rotary step on q and the new K row (head_size 128).
#include "decode_kernel.h"

namespace q8kv {

const void* split_kernel_nr_hs32(uint32_t group, uint32_t seg_rows) {
    if (group == 4) return split_kernel_nr<1>(seg_rows);
    if (group == 8) return split_kernel_nr<2>(seg_rows);
    return nullptr;
}

}  // namespace q8kv
