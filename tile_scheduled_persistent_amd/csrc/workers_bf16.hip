// Instantiations of the persistent tile worker for BF16 weights, greedy token selection, BF16 KV cache: one translation unit
// per combination, so that the build compiles them in parallel.
#define TILES_WORKER_UNIT
#include "kernel.hip"

namespace tiles {

const void* worker_unit_0(int head_dim, int group) {
  return worker_for<false, false, false>(head_dim, group);
}

// the test instantiation whose waits check their watchdog every polling round
const void* worker_watchdog(int head_dim) {
  if (head_dim == 64) return reinterpret_cast<const void*>(&tiles_worker<64, 1, true, false, false, false>);
  if (head_dim == 128) return reinterpret_cast<const void*>(&tiles_worker<128, 1, true, false, false, false>);
  return nullptr;
}

}  // namespace tiles
