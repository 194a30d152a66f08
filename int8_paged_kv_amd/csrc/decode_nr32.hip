// Split-kernel instantiations of the decode step with the per-head RMSNorm +
// partial rotary step on q and the new K row, head_size 128.
#include "decode_kernel.h"

namespace q8kv {

const void* split_kernel_nr_hs32(uint32_t group, uint32_t seg_rows) { return split_kernel_nr<32>(group, seg_rows); }

}  // namespace q8kv
