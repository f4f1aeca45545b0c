// Instantiations of the persistent tile worker for weight-only INT8 weights, sampled token selection, BF16 KV cache: one translation unit
// per combination, so that the build compiles them in parallel.
#define TILES_WORKER_UNIT
#include "kernel.hip"

namespace tiles {

const void* worker_unit_6(int head_dim, int group) {
  return worker_for<true, true, false>(head_dim, group);
}

}  // namespace tiles
