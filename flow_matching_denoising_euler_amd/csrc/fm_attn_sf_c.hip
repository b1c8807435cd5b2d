// Explicit instantiations of the register-resident attention launcher
// (head_dim, query blocks per workgroup, head-dim split): (256, 1, 4).
#include "fm_attn_sf.h"

namespace fm {

template hipError_t attn_sf<256, 1, 4>(AttnArgs, hipStream_t);

}  // namespace fm
