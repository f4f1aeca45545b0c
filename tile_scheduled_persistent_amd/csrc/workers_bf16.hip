// Instantiations of the persistent tile worker for BF16 weights, greedy token selection (and the short-watchdog test worker): one translation unit per weight
// format and token selection, so that the build compiles them in parallel.
#define TILES_WORKER_UNIT
#include "kernel.hip"

namespace tiles {

const void* worker_bf16_greedy(int head_dim, int group) { return worker_for<false, false>(head_dim, group); }

// the test instantiation whose waits check their watchdog every polling round
const void* worker_watchdog(int head_dim) {
  if (head_dim == 64) return reinterpret_cast<const void*>(&tiles_worker<64, 1, true, false, false>);
  if (head_dim == 128) return reinterpret_cast<const void*>(&tiles_worker<128, 1, true, false, false>);
  return nullptr;
}

}  // namespace tiles
