// Instantiations of the persistent tile worker for multi-token verify steps with weight-only INT8
// weights (greedy, BF16 KV cache): one translation unit, compiled in parallel with the others.
#define TILES_WORKER_UNIT
#include "kernel.hip"

namespace tiles {

const void* worker_mt_unit_1(int head_dim, int group, int mt) { return worker_mt_for<true, false>(head_dim, group, mt); }

}  // namespace tiles
