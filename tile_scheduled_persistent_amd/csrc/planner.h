// Host planner: tile graph, static schedule, validation and weight-packing layout.
// Pure C++ (no HIP): it runs without a GPU and is exercised by tiles_plan_dry_run.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/tiles.h"
#include "plan_types.h"

namespace tiles {

// Which source tensor a packing copy reads.
enum SrcTensor : int32_t {
  SRC_EMBED, SRC_FINAL_NORM, SRC_LM_HEAD,
  SRC_ATTN_NORM, SRC_WQ, SRC_WK, SRC_WV, SRC_Q_NORM, SRC_K_NORM, SRC_WO, SRC_MLP_NORM, SRC_WGATE, SRC_WUP, SRC_WDOWN,
};

// Copy `nrows` rows of `cols` BF16 values starting at row `src_row` of a source tensor
// into the packed buffer at `dst_off`, rows `dst_pitch` bytes apart (padding stays zero).
struct CopySeg {
  int32_t tensor;
  int32_t layer;
  int64_t src_row;
  int64_t nrows;
  int64_t cols;
  int64_t dst_off;
  int64_t dst_pitch;
  // Quantized copy (weight-only INT8): the rows are written as INT8 codes (cols bytes each) and row i's
  // FP32 scale goes to scale_off + i * scale_pitch; -1 for a plain BF16 copy.
  int64_t scale_off = -1;
  int64_t scale_pitch = 0;
};

// Buffers named by the hazard check.
// Tagged output buffer of wave k: BUF_WAVE + k.
enum BufId : int32_t { BUF_EMBED, BUF_LMPART, BUF_KV, BUF_LOGITS, BUF_WAVE = 16 };

struct Interval {
  int32_t buf;
  int64_t lo, hi;  // [lo, hi)
};

struct Shape {
  int32_t n_layers, H, n_heads, n_kv, hd, F, V;
  int32_t G;                  // query heads per KV head
  int32_t qkv_rows;           // (n_heads + 2 n_kv) * hd
  int32_t Hpad, Qpad, Fpad;   // padded GEMV widths (multiples of CHUNK_COLS)
  bool qk_norm, tied;
  int32_t max_positions;
};

struct HostPlan {
  Shape s;
  int32_t W = 0;               // workers
  int32_t q8 = 0;              // 1: weight-only INT8 linear layers (codes + per-row FP32 scales)
  int32_t wb = 2;              // bytes per packed weight: 2 (BF16) or 1 (INT8)
  int32_t S = 1;               // KV splits
  int32_t combine_in_o = 1;    // 1 prologue, 0 own wave
  int32_t T = 1;               // query heads per attention tile (divides G)
  int32_t mt = 1;              // positions per step: 1 (decode), 2 .. 4 (verify plans)
  int32_t top_k = 0;           // sampled decoding: 1 .. MAX_TOP_K; 0 greedy
  int32_t kv8 = 0;             // 1: INT8 KV cache (codes, per-position scales, smoothed keys)
  int32_t kv8_span = 0;        // INT8 KV: positions per LDS scale area (the longest split, rounded up to 64)
  float temperature = 1.0f, top_p = 1.0f;
  std::vector<WaveDesc> waves;
  std::vector<TileDesc> tiles; // [n_waves][W]
  std::vector<LayerSmall> small;
  int64_t final_norm_off = 0, embed_off = 0, embed_stride = 0;
  int64_t packed_bytes = 0;
  int64_t weight_bytes_per_step = 0;  // algorithmic (unpadded) weight bytes per token
  std::vector<CopySeg> copies;
  std::vector<int64_t> wave_bytes, wave_max_bytes;  // padded bytes streamed per wave (all / max worker)
  std::vector<int32_t> wave_busy;
  double max_over_mean = 1.0;
  int32_t lds_vec_floats = 0, lds_part_floats = 0, lds_xres_floats = 0, lds_bytes = 0;
  int32_t lds_stage_floats = 0, stage_batches = 0;  // staging of the next GEMV range's chunks
  int64_t ll_words = 0;        // tagged-data buffers of all waves (uint32 words)
  uint64_t checksum = 0;
};

// Bytes of a GEMV tile in the packed buffer: its rows, then (INT8) their scales padded to a chunk.
inline int64_t tile_packed_bytes(const HostPlan& p, const TileDesc& t) {
  const int64_t rows = (int64_t)t.nrows * (t.kind == KIND_GU ? 2 : 1);
  const int64_t scales = p.q8 ? (rows * 4 + CHUNK_BYTES - 1) / CHUNK_BYTES * CHUNK_BYTES : 0;
  return rows * t.kpad * p.wb + scales;
}

// Symmetric per-row INT8 codes of BF16 rows (weight-only INT8): s = max |w| / 127 and
// q = round-half-even(w / s) clamped to [-127, 127], each operation in IEEE FP32; s = 0, q = 0 for
// a row of zeros.  src: `rows` rows of `cols` BF16 values, `src_pitch` values apart.
void quantize_rows_int8(const uint16_t* src, int64_t src_pitch, int64_t rows, int64_t cols, int8_t* q,
                        int64_t q_pitch, float* scales, int64_t scale_pitch_floats);

// Build and validate a plan.  Returns TILES_OK or a TILES_E_* code with `err` set.
int build_plan(const tiles_config_t& cfg, int32_t n_workers, HostPlan& plan, std::string& err);

// Re-run every structural check on an existing plan (used at create and by tests).
int validate_plan(const HostPlan& plan, std::string& err);

// 64-bit FNV-1a over the schedule and its geometry.
uint64_t plan_checksum(const HostPlan& plan);

// Per-worker hash of the schedule words each worker loads into LDS (its TileDesc of every wave,
// every WaveDesc, every LayerSmall; see table_mix): W entries, re-checked by the kernel.
std::vector<uint64_t> worker_table_hashes(const HostPlan& plan);

// Planted mistakes for tests of validate_plan (host only): each makes one rule fail.
enum DebugMutation : int32_t {
  DBG_NONE = 0,
  DBG_ROW_OVERLAP = 1,        // a gate/up tile takes one row more: rows covered twice
  DBG_ROW_GAP = 2,            // a gate/up tile gives up a row: a row covered by nobody
  DBG_ATTN_DUPLICATE = 3,     // an attention tile copied to an idle worker
  DBG_ATTN_MISSING = 4,       // an attention tile removed
  DBG_SPLIT_OUT_OF_RANGE = 5, // an attention tile's split index = S
  DBG_TAGGED_OVERLAP = 6,     // wave 1's tagged buffer placed on wave 0's
  DBG_TAGGED_OUT_OF_BOUNDS = 7,
  DBG_UNBALANCED = 8,         // a down tile takes two rows of its neighbour (coverage and packing stay exact)
  DBG_WAVE_ORDER = 9,         // waves 1 and 2 swapped
  DBG_LM_NOT_LAST = 10,       // the step does not end with the LM head (no per-step all-to-all)
  DBG_PACKED_OVERLAP = 11,    // two QKV tiles read the same packed bytes
  DBG_PACKED_SWAPPED = 12,    // two LM-head tiles exchange their packed rows
  DBG_COPY_DROPPED = 13,      // one packing copy removed
  DBG_GAIN_MISPLACED = 14,    // layer 1's MLP gain offset points at layer 0's
  DBG_STAGING = 15,           // more staging batches than the LDS layout allows
};
int debug_mutate_plan(HostPlan& plan, int32_t mutation, std::string& err);

// Words of wave `kind`'s tagged output buffer (0 for the LM head, whose partials live apart).
inline int64_t wave_out_words(const Shape& s, int32_t S, int32_t kind) {
  switch (kind) {
    case KIND_QKV: return s.qkv_rows;
    case KIND_ATTN: return (int64_t)s.n_heads * S * (s.hd + 4);  // records (m, l, acc[hd], 2 pad)
    case KIND_COMBINE: return (int64_t)s.n_heads * s.hd;
    case KIND_O: return s.H;
    case KIND_GU: return s.F;
    case KIND_DOWN: return s.H;
    default: return 0;
  }
}

// The split [lo, hi) of KV positions that split `s` of `S` covers when `L` positions are attended.
inline void split_range(int64_t L, int32_t S, int32_t s, int64_t& lo, int64_t& hi) {
  int64_t c = (L + S - 1) / S;
  lo = (int64_t)s * c;
  hi = lo + c < L ? lo + c : L;
  if (lo > L) lo = L;
}

}  // namespace tiles
