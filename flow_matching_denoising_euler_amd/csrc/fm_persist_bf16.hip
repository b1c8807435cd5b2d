// The persistent batch-1 loop kernel with bf16 weights (see fm_persist.h).
#include "fm_persist.h"

namespace fm {

hipError_t launch_persist_bf16(int R, int DS, const PersistArgs& p, int grid, hipStream_t st) {
  return PersistLaunch<ELT_BF16>::launch(R, DS, p, grid, st);
}
hipError_t persist_occupancy_bf16(int R, int DS, int* blocks_per_cu) {
  return PersistLaunch<ELT_BF16>::occupancy(R, DS, blocks_per_cu);
}

}  // namespace fm
