// Instantiations of the persistent tile worker for multi-token verify steps with BF16 weights (greedy,
// BF16 KV cache): one translation unit, compiled in parallel with the others.
#define TILES_WORKER_UNIT
#include "kernel.hip"

namespace tiles {

const void* worker_mt_unit_0(int head_dim, int group, int mt) { return worker_mt_for<false, false>(head_dim, group, mt); }

}  // namespace tiles
