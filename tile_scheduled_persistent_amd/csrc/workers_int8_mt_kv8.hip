// Instantiations of the persistent tile worker for multi-token verify steps with weight-only INT8
// weights and the INT8 KV cache (greedy): one translation unit, compiled in parallel with the others.
#define TILES_WORKER_UNIT
#include "kernel.hip"

namespace tiles {

const void* worker_mt_unit_3(int head_dim, int group, int mt) { return worker_mt_for<true, true>(head_dim, group, mt); }

}  // namespace tiles
