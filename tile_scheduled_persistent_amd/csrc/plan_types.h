// Plain-old-data structures shared by the host planner and the persistent kernel.
//
// A plan is a per-step schedule: `n_waves` waves, each holding one tile slot per
// worker (workgroup).  The same schedule repeats for every decoded token; only the
// token, the position and the attended length change between steps.
#pragma once
#include <stdint.h>

namespace tiles {

// Kinds of wave (and of the tiles they hold).  Values are part of the C ABI
// (tiles_wave_info_t.kind).
enum : int32_t {
  KIND_NONE = 0,
  KIND_QKV = 1,      // RMSNorm prologue + rows of [Wq; Wk; Wv]
  KIND_ATTN = 2,     // q/k norm + RoPE + KV write + split-KV attention for one (KV head, split)
  KIND_COMBINE = 3,  // merge the splits of one query head
  KIND_O = 4,        // (combine prologue) + rows of Wo + residual add
  KIND_GU = 5,       // RMSNorm prologue + paired rows of W_gate / W_up + SwiGLU
  KIND_DOWN = 6,     // rows of W_down + residual add
  KIND_LM = 7,       // final RMSNorm prologue + vocabulary rows + partial argmax
};

// Geometry of the GEMV inner loop: one "chunk" is 64 lanes x 16 bytes = 512 BF16
// columns of one row.  Every GEMV row is padded to a multiple of CHUNK_COLS.
constexpr int CHUNK_COLS = 512;
constexpr int CHUNK_BYTES = 1024;
// Weight-only INT8 plans pack every linear layer as signed 8-bit codes, 1024 columns per chunk, each
// tile's rows followed by their FP32 scales (one per row, padded to a whole chunk).
constexpr int CHUNK_COLS_I8 = 1024;
enum : int32_t { WEIGHTS_BF16 = 0, WEIGHTS_INT8 = 1 };
constexpr int XCDS = 8;  // MI355X: 8 XCDs of 32 CUs, each with its own L2; workgroup i runs on XCD i % 8
constexpr int BLOCK_THREADS = 512;
constexpr int NWAVES = BLOCK_THREADS / 64;
// Wavefront 0 of every workgroup is the control wave (epilogues and global stores);
// wavefronts 1..NCOMP stream weights into registers and compute.  All eight gather inputs.
constexpr int NCOMP = NWAVES - 1;
constexpr int SMALL_FLOATS = 1024;                          // LDS scratch for reductions / broadcasts
struct SegDesc {  // per-wave GEMV geometry of one worker (LDS copy used by the weight prefetch)
  int64_t woff;
  int32_t chunks_per_row;
  int32_t rows;  // weight rows of the tile (0: no GEMV tile in this wave)
};
constexpr int MAX_GROUP = 4;  // query heads per KV head the kernel supports
constexpr int MAX_BLOCK_ROWS = 640;
constexpr int32_t LDS_LIMIT = 160 * 1024;  // LDS of one CU (gfx950)
// Register streaming of the compute wavefronts: two batches of STREAM_BATCH 16-byte loads per
// lane in flight (STREAM_DEPTH; the kernel's ring has two register sets), for weight chunks and
// K/V rows alike.
constexpr int STREAM_BATCH = 4;
constexpr int STREAM_DEPTH = 2 * STREAM_BATCH;
// Up to this many further batches of a compute wavefront's next GEMV range are staged in its LDS
// area by direct-to-LDS loads issued with the register prefetch (as many as the LDS holds).
constexpr int MAX_STAGE_BATCHES = 2;
// Verify plans: positions per step at most (each GEMV tile streams its weights once for all of them;
// the step's input vectors are held in LDS side by side).
constexpr int MAX_STEP_TOKENS = 4;
constexpr uint32_t DEFAULT_SPIN_LIMIT = 1u << 22;  // polling rounds before a wait gives up (watchdog)
constexpr int32_t MAX_POSITIONS = 1 << 23;
// Sampled decoding (top-k / top-p): each worker publishes its top_k largest logits, at most this many.
constexpr int32_t MAX_TOP_K = 32;
// KV cache formats: BF16 rows, or INT8 codes with one FP32 scale per (layer, KV head, position) and
// keys smoothed by a per-(layer, KV head, channel) factor.
enum : int32_t { KVFMT_BF16 = 0, KVFMT_INT8 = 1 };
// INT8 KV: an attention tile stages its split's per-position K and V scales in LDS, in an area of the
// plan's kv8_span positions each (the longest split rounded up to 64); at most this many positions
// per split (the planner raises the split count, or rejects the plan).
constexpr int32_t MAX_SPLIT_POSITIONS_KV8 = 4096;

struct TileDesc {   // 32 bytes
  int32_t kind;
  int32_t row0;     // GEMV: first output row (GU: first j). ATTN: KV head. COMBINE: query head.
  int32_t nrows;    // GEMV: output rows (GU: number of j; the tile holds 2*nrows rows, gate/up interleaved). ATTN: split.
  int32_t kpad;     // GEMV: packed columns per row (a multiple of the plan's columns per chunk)
  int64_t woff;     // GEMV: byte offset of the tile's first packed row
  int32_t aux0;     // reserved
  int32_t aux1;     // reserved
};

struct WaveDesc {   // 16 bytes
  int32_t kind;
  int32_t layer;    // -1 for the LM head
  int32_t max_rows; // largest GEMV row count of any tile in the wave (sizes the LDS partial area)
  int32_t ll_off;   // first word of the wave's tagged output buffer (-1: the LM head, see lmpart)
};

// Offsets (bytes) of the per-layer norm gains inside the packed buffer.
struct LayerSmall {
  int64_t attn_norm, mlp_norm, q_norm, k_norm;
};

// Sync area layout (uint32 words, one 64-byte line each).
constexpr int SYNC_STATUS_WORD = 0;      // fault word: 0 ok, STATUS_WATCHDOG or STATUS_TABLES
constexpr uint32_t STATUS_WATCHDOG = 1;  // a wait's watchdog expired
constexpr uint32_t STATUS_TABLES = 2;    // a worker's device-resident schedule failed its check
constexpr int SYNC_ABORT_WORD = 16;      // set by any worker that gives up waiting
constexpr int SYNC_WORDS = 32;
// Size of the file-scope scratch array of the allocation-free decode entry point (per GPU): the
// tagged-data buffers, LM-head partials and status words of one launch must fit in it.
constexpr int64_t NOALLOC_SCRATCH_BYTES = 8ll << 20;

// In-kernel trace record per (step, wave, worker), 100 MHz wall clock:
//   0 wave start, 1 inputs staged (after barrier P), 2 compute done (after barrier B),
//   3 outputs published, 7 after barrier A  -- all taken by the control wave;
//   5 own gather done (before P), 6 after barrier A, 4 own share of the tile done (before B)
//   -- taken by the first compute wave (4 stays 0 when it had no share).
constexpr int TRACE_WORDS = 12;

// Hash of the schedule bytes worker `w` loads: its TileDesc of every wave, every WaveDesc and
// every LayerSmall, as 32-bit words; word i of the sequence contributes mix(i << 32 | word) and the
// contributions are summed modulo 2^64 (so that lanes may add them up in any grouping).  The host
// computes it at plan creation; the kernel recomputes it from the copies it loaded before using them.
// (constexpr: callable from host and device code alike)
constexpr uint64_t table_mix(uint64_t x) {  // the splitmix64 finaliser
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ull;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebull;
  x ^= x >> 31;
  return x;
}

// Tagged-data buffers are filled with this word before every launch: a quiet NaN whose
// parity bit (bit 0) is 0, so that step 0 (parity 1) never mistakes it for a value.
constexpr uint32_t TAG_FILL = 0x7fc00000u;

// One weight-packing copy executed on the device: `rows` rows of `row_bytes` bytes from
// `src` (rows `src_pitch` apart) to packed + dst_off (rows `dst_pitch` apart).
struct PackSeg {
  const uint8_t* src;
  int64_t src_pitch;
  int64_t dst_off;
  int64_t dst_pitch;
  int64_t rows;
  int64_t row_bytes;
};

struct KernelArgs {
  const TileDesc* tiles;     // [n_waves][W]
  const WaveDesc* waves;     // [n_waves]
  const LayerSmall* small;   // [n_layers]
  const uint8_t* packed;     // packed weights
  const float* rope;         // [max_positions][head_dim/2][2] (cos, sin)
  int64_t final_norm_off;    // bytes into packed
  int64_t embed_off;         // bytes into packed: embedding row 0
  int64_t embed_stride;      // bytes between embedding rows
  // tagged-data buffers (see the kernel): one per wave, and the LM-head partials
  uint32_t* ll;              // FP32 values, parity in bit 0; wave k's output at ll + waves[k].ll_off
  uint32_t* lmpart;          // [W][max(1, top_k)][2] (logit bits, index | parity << 31): the worker's
                             // maximum (greedy) or its top_k logits in decreasing order (sampled)
  uint32_t* sync;            // SYNC_WORDS status / abort words
  const uint64_t* table_check;  // [W + 1]: per-worker hash of the schedule it loads, then the build id
  uint16_t* kv_k;            // BF16 cache, or (INT8 KV) INT8 codes [layer][kv head][capacity][head_dim]
  uint16_t* kv_v;
  float* kv_ks;              // INT8 KV: K and V scales [layer][kv head][capacity], smoothing factors
  float* kv_vs;              //   [layer][kv head][head_dim]
  const float* kv_sigma;
  int64_t kv_cap;
  int32_t* out_tokens;
  float* out_logits;         // may be null
  const float* uniforms;     // [n_steps] FP32 in [0, 1): the draw of each sampled step (null: greedy)
  float* dbg_hidden;         // [n_steps][n_layers][H] or null
  uint64_t* trace;           // [n_steps][n_waves][W][TRACE_WORDS] or null
  int32_t token0, pos0, n_steps, n_waves;
  int32_t W, n_layers, H, Hpad, n_heads, n_kv, head_dim, F, Fpad, V, qkv_rows, Qpad, S;
  int32_t combine_in_o;      // 1: the o_proj prologue merges the splits
  float eps;
  float qscale;              // log2(e) / sqrt(head_dim): scores in the base-2 domain
  uint32_t spin_limit;       // watchdog of every wait (polls)
  int32_t lds_vec_floats;    // LDS layout
  int32_t lds_part_floats;
  int32_t lds_xres_floats;
  int32_t lds_stage_floats;  // NCOMP staging areas of stage_batches batches
  int32_t stage_batches;
  int32_t top_k;             // 0: greedy; 1 .. MAX_TOP_K: sampled (top-k, temperature, top-p)
  float temperature;
  float top_p;
  const int32_t* forced;     // [n_steps * mt - 1] or null: position i > 0 of the launch consumes forced[i - 1]
                             // (verify steps); the argmax is still recorded in out_tokens
  int32_t mt;                // positions per step: 1 (decode), or 2 .. MAX_STEP_TOKENS (verify plans: every
                             // step runs mt consecutive teacher-forced positions through each tile)
  int64_t ll_tok;            // words between the tagged buffers of consecutive positions of a step
  int32_t kv8_span;          // INT8 KV: positions of each of the LDS scale areas (K, then V) of a split
};

}  // namespace tiles
