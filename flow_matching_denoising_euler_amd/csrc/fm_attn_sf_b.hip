// Explicit instantiations of the register-resident attention launcher
// (head_dim, query blocks per workgroup, head-dim split): (256, 2, 1), (256, 1, 1).
#include "fm_attn_sf.h"

namespace fm {

template hipError_t attn_sf<256, 2, 1>(AttnArgs, hipStream_t);
template hipError_t attn_sf<256, 1, 1>(AttnArgs, hipStream_t);

}  // namespace fm
