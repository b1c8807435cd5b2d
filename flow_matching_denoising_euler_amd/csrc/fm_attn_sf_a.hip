// Explicit instantiations of the register-resident attention launcher
// (head_dim, query blocks per workgroup, head-dim split): (32, 2, 1), (32, 1, 1), (64, 2, 1), (64, 1, 1), (128, 2, 1), (128, 1, 1).
#include "fm_attn_sf.h"

namespace fm {

template hipError_t attn_sf<32, 2, 1>(AttnArgs, hipStream_t);
template hipError_t attn_sf<32, 1, 1>(AttnArgs, hipStream_t);
template hipError_t attn_sf<64, 2, 1>(AttnArgs, hipStream_t);
template hipError_t attn_sf<64, 1, 1>(AttnArgs, hipStream_t);
template hipError_t attn_sf<128, 2, 1>(AttnArgs, hipStream_t);
template hipError_t attn_sf<128, 1, 1>(AttnArgs, hipStream_t);

}  // namespace fm
