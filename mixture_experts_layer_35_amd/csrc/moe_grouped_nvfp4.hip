// Grouped-path expert kernels (gate+up, down) for routed NVFP4 weights.
// One translation unit per routed format keeps the builds parallel.
#include "moe_grouped.h"

namespace moe {

template <>
hipError_t launch_experts<FMT_NVFP4>(const GroupedArgs& a, int fs, hipStream_t st, hipEvent_t* ev) {
  return launch_experts_fs<FMT_NVFP4>(a, fs, st, ev);
}

}  // namespace moe
