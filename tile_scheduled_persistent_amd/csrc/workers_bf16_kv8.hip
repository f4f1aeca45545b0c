// Instantiations of the persistent tile worker for BF16 weights, greedy token selection, INT8 KV cache: one translation unit
// per combination, so that the build compiles them in parallel.
#define TILES_WORKER_UNIT
#include "kernel.hip"

namespace tiles {

const void* worker_unit_1(int head_dim, int group) {
  return worker_for<false, false, true>(head_dim, group);
}

}  // namespace tiles
