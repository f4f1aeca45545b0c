// Instantiations of the persistent tile worker for weight-only INT8 weights, sampled token selection: one translation unit per weight
// format and token selection, so that the build compiles them in parallel.
#define TILES_WORKER_UNIT
#include "kernel.hip"

namespace tiles {

const void* worker_int8_sampled(int head_dim, int group) { return worker_for<true, true>(head_dim, group); }

}  // namespace tiles
