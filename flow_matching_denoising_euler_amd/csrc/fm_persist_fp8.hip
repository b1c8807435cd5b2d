// The persistent batch-1 loop kernel with fp8 E4M3 weights (widened exactly to bf16 in registers) (see fm_persist.h).
#include "fm_persist.h"

namespace fm {

hipError_t launch_persist_fp8(int R, int DS, const PersistArgs& p, int grid, hipStream_t st) {
  return PersistLaunch<ELT_FP8>::launch(R, DS, p, grid, st);
}
hipError_t persist_occupancy_fp8(int R, int DS, int* blocks_per_cu) {
  return PersistLaunch<ELT_FP8>::occupancy(R, DS, blocks_per_cu);
}

}  // namespace fm
