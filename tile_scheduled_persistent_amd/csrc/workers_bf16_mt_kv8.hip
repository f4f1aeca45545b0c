// Instantiations of the persistent tile worker for multi-token verify steps with BF16 weights and the
// INT8 KV cache (greedy): one translation unit, compiled in parallel with the others.
#define TILES_WORKER_UNIT
#include "kernel.hip"

namespace tiles {

const void* worker_mt_unit_2(int head_dim, int group, int mt) { return worker_mt_for<false, true>(head_dim, group, mt); }

}  // namespace tiles
