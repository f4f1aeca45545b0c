/*
 * tiles.h -- C ABI of the tile-scheduled persistent decoder for AMD MI355X (gfx950).
 *
 * One batch-1 greedy BF16 decode step of a Llama/Qwen3-style decoder runs as a
 * static graph of tiles: a host planner cuts every operator into output-row
 * tiles, assigns each tile to a fixed workgroup (one per compute unit), groups
 * the tiles into dependency-ordered waves, validates the schedule and packs the
 * weights tile-contiguously; one cooperative persistent kernel then executes
 * that schedule for up to 64 tokens per launch, with greedy selection inside the
 * kernel.  The pages separate waves with grid barriers; this kernel carries each
 * dependency in the data instead (every published value holds the step's parity
 * in its lowest mantissa bit and consumers poll the values themselves).
 *
 * Sources: "Tiles: Scheduling LLM Decoding as a Graph of Tiles" (intro: tiles
 * as the unit of scheduled work, a fixed worker per tile, byte balancing,
 * waves separated by grid barriers, validation before launch, bit-identical
 * runs; "What the code contains": an offline plan builder that sizes the grid
 * from the kernel's occupancy, validates the graph and packs the weights, and
 * a runtime that checks the plan before using it and runs many tokens per
 * cooperative launch with greedy selection on the GPU).  The fused
 * operations follow "History and roadmap" (TileInfer.jl), "M8 so far" table:
 * q/k norm + RoPE + KV write, residual add + RMSNorm, SwiGLU in the GEMV;
 * split-KV decode attention follows its "Milestones" table, M5.
 *
 * Conventions for every entry point:
 *   - Return value: TILES_OK (0) or a negative TILES_E_* code; the text of the
 *     last error of the calling thread is available from tiles_last_error().
 *   - Pointers marked "device" are HIP device memory on the current device;
 *     pointers marked "host" are ordinary host memory.
 *   - No entry point takes ownership of caller memory.
 *   - BF16 tensors are raw IEEE bfloat16 bit patterns (uint16), row-major.
 */
#ifndef TILES_H
#define TILES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define TILES_OK 0
#define TILES_E_ARG (-1)     /* null pointer, out-of-range token / n_steps, KV capacity exceeded */
#define TILES_E_CONFIG (-2)  /* model shape the planner cannot tile (e.g. heads not dividing) */
#define TILES_E_PLAN (-3)    /* schedule validation failed or the plan was modified after creation */
#define TILES_E_DEVICE (-4)  /* not gfx950, CU count differs from the plan, no cooperative launch, occupancy < 1 */
#define TILES_E_HIP (-5)     /* a HIP runtime call failed; its message is in tiles_last_error() */
#define TILES_E_KERNEL (-6)  /* the kernel reported a fault (the watchdog of a wait expired) */

/* ---- plan flags (tiles_config_t.flags) --------------------------------- */
#define TILES_DEBUG_HIDDEN 0x1u /* record the residual stream after every layer of every step */
#define TILES_TRACE 0x2u        /* record per-worker, per-wave timestamps (100 MHz wall clock) */
#define TILES_POISON 0x4u       /* before every launch, NaN-fill the KV rows the launch will write
                                   (positions length .. length+n_steps-1 of every layer and KV head),
                                   so that a read before the kernel's own write shows up as NaN */

/* ---- model + plan options ---------------------------------------------- */
typedef struct tiles_config {
  int32_t n_layers;       /* decoder layers */
  int32_t hidden;         /* H */
  int32_t n_heads;        /* query heads */
  int32_t n_kv_heads;     /* key/value heads; must divide n_heads (grouped-query attention) */
  int32_t head_dim;       /* 64 or 128 */
  int32_t ffn;            /* SwiGLU intermediate size F */
  int32_t vocab;          /* V */
  float rope_theta;       /* RoPE base */
  float rms_eps;          /* RMSNorm epsilon (also used for the q/k norms) */
  int32_t qk_norm;        /* 1: per-head RMSNorm of q and k before RoPE (Qwen3) */
  int32_t tie_embeddings; /* 1: the LM head is the embedding matrix */
  int32_t max_positions;  /* largest KV length (cached + decoded) the plan supports, 1 .. 2^23 */
  uint32_t flags;         /* TILES_DEBUG_HIDDEN | TILES_TRACE | TILES_POISON */
  int32_t kv_splits;      /* split-KV count per KV head; 0 lets the planner choose */
  int32_t combine_mode;   /* 0 planner choice, 1 combine splits in the o_proj prologue, 2 own wave */
  int32_t attn_heads;     /* query heads per attention tile (divides n_heads / n_kv_heads); 0 planner choice */
  int32_t n_workers;      /* 0 = one workgroup per compute unit (required on the GPU) */
  void *stream;           /* hipStream_t used by create (copies) and by every decode; NULL = null stream */
  int32_t o_placement;    /* workers of the o_proj tiles: 0 planner choice (all), 1 all workers, 2 those
                             without an attention tile, when there are any and the splits merge in the
                             o_proj prologue */
  int32_t weight_format;  /* TILES_WEIGHTS_BF16, or TILES_WEIGHTS_INT8: every linear layer (Wq, Wk, Wv, Wo,
                             W_gate, W_up, W_down and the LM head) packed as symmetric per-row INT8
                             codes with one FP32 scale per row, quantized from the BF16 weights at plan
                             creation (see tiles_quantize_rows_int8) and dequantized in registers; the
                             norm gains and the embedding lookup stay BF16 */
  /* Sampled decoding ("History and roadmap" (TileInfer.jl), "M8 so far" table: top-k/top-p sampling
   * on the device, inside the graph).  top_k = 0: greedy (tiles_decode).  1 <= top_k <= 32 (and
   * <= vocab): the plan samples (tiles_decode_sampled): rank the logits in decreasing order (equal
   * logits by increasing id), keep the first top_k, weigh them by exp((z - z_max) / temperature),
   * keep the shortest prefix whose cumulative weight reaches top_p of the kept total (at least one
   * token), and draw the first token of the prefix whose cumulative weight exceeds u * (prefix
   * total), u being the step's uniform; every sum and comparison in FP32, sums in ranking order.
   * Needs temperature > 0 (finite) and 0 < top_p <= 1; both ignored when top_k = 0. */
  int32_t top_k;
  float temperature;
  float top_p;
  /* KV cache format ("History and roadmap" (TileInfer.jl), "M8 so far" table: INT8 KV cache with
   * smoothed keys): TILES_KV_BF16, or TILES_KV_INT8: every cached K and V row as symmetric INT8 codes
   * with one FP32 scale per (layer, KV head, position), keys divided by a per-(layer, KV head,
   * channel) smoothing factor before quantization; attention reads the codes and computes with the
   * dequantized rows (queries stay FP32).  An attention tile stages its split's scales in LDS: at
   * most 4096 positions per split (the planner raises its split count to fit; a kv_splits that
   * leaves longer splits fails with TILES_E_CONFIG).  See tiles_kv_t and tiles_kv_convert_int8. */
  int32_t kv_format;
  /* Positions per step of a verify plan ("History and roadmap" (TileInfer.jl), "M8 so far" table:
   * verify steps of up to 16 tokens; "Tried and not kept" table: verify GEMMs at 2-64 tokens).  0 or 1:
   * one position per step (decode plans; tiles_verify then runs its m positions as m steps).  2, 3
   * or 4: a verify plan, usable with tiles_verify only: every step takes tokens_per_step consecutive
   * teacher-forced positions through each tile, so that each GEMV tile streams its weights once for
   * all of them (its LDS holds one input vector per position) and each attention tile serves all of
   * them with one pass over the cached rows, the step's own rows entering the positions at or after
   * them (INT8 KV: each quantized as in a one-position step).  Needs greedy selection (top_k = 0) and
   * query heads per attention tile x tokens_per_step <= 4 (the planner's choice of attn_heads and
   * kv_splits keeps to that).  The LDS must hold tokens_per_step input vectors of max(hidden, ffn)
   * floats (padded), plus the split merge of every position where the o_proj prologue merges the
   * splits (combine_mode 1; the planner's choice takes it only where it fits); plan creation fails
   * with TILES_E_CONFIG otherwise. */
  int32_t tokens_per_step;
} tiles_config_t;

#define TILES_KV_BF16 0
#define TILES_KV_INT8 1

#define TILES_WEIGHTS_BF16 0
#define TILES_WEIGHTS_INT8 1

/* Per-layer weights, BF16, row-major [out, in]:
 *   attn_norm, mlp_norm [H]; q_norm, k_norm [head_dim] (only read when qk_norm);
 *   wq [n_heads*head_dim, H]; wk, wv [n_kv_heads*head_dim, H]; wo [H, n_heads*head_dim];
 *   w_gate, w_up [F, H]; w_down [H, F]. */
typedef struct tiles_layer_weights {
  const void *attn_norm, *wq, *wk, *wv, *q_norm, *k_norm, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
} tiles_layer_weights_t;

typedef struct tiles_weights {
  const void *embed;                   /* [V, H] */
  const void *final_norm;              /* [H] */
  const void *lm_head;                 /* [V, H]; NULL when tie_embeddings */
  const tiles_layer_weights_t *layers; /* host array of n_layers entries */
  int32_t on_device;                   /* 1: the tensors are device memory, 0: host memory */
} tiles_weights_t;

typedef struct tiles_plan tiles_plan_t;

/* KV cache, caller-owned device memory.  BF16 plans: k, v are BF16 [n_layers][n_kv_heads][capacity]
 * [head_dim].  INT8 KV plans (kv_format = TILES_KV_INT8): k holds the int8 codes of K and V interleaved,
 * [n_layers][n_kv_heads][capacity][2 * head_dim] with, for every group of 8 dimensions, the 8 K codes
 * followed by the 8 V codes (one 16-byte load then reads both for a position); v is unused (may be
 * NULL); k_scale and v_scale are float [n_layers][n_kv_heads][capacity] (a row is codes * scale,
 * keys then times k_smooth); k_smooth is float [n_layers][n_kv_heads][head_dim] (> 0; see
 * tiles_kv_convert_int8).
 * Keys are stored after q/k norm and RoPE.  A decode reads positions [0, length + i) at step i
 * (position length + i itself from the values it has just computed) and writes position
 * length + i (INT8: its codes and scales, quantized from FP32); the contents of every other row --
 * the unused tail, NaN included -- never affect any result. */
typedef struct tiles_kv {
  void *k;
  void *v;
  int64_t capacity; /* positions allocated */
  int64_t length;   /* positions already cached; tiles_decode adds n_steps on success */
  float *k_scale;   /* INT8 KV only (else ignored) */
  float *v_scale;
  float *k_smooth;
} tiles_kv_t;

/* Convert the first `length` positions of a BF16 cache (k_bf16, v_bf16: device BF16 [n_layers]
 * [n_kv_heads][capacity][head_dim]) into the INT8 cache `dst` of an INT8 KV plan ("History and
 * roadmap" (TileInfer.jl), "M8 so far" table: INT8 KV cache with smoothed keys): k_smooth[l][h][c]
 * = the largest |K| of channel c over those positions (1 for a channel that is zero there), then
 * every row r quantized symmetrically, keys divided by k_smooth first: s = max|r| / 127, code =
 * round-half-even(r / s) clamped to [-127, 127] (s = 0 and codes 0 for a zero row), FP32 divisions.
 * dst: device buffers as tiles_kv_t describes (dst->v unused), capacity equal to `capacity`; dst->length is set to
 * `length`.  Positions from `length` on are left as they are.  Runs on the plan's stream
 * (asynchronous); allocates nothing.  TILES_E_ARG for a BF16 plan, null pointers, or a length
 * beyond the capacity. */
int tiles_kv_convert_int8(tiles_plan_t *plan, const void *k_bf16, const void *v_bf16, int64_t capacity,
                          int64_t length, tiles_kv_t *dst);


/* Summary of a plan (see tiles_plan_info). */
typedef struct tiles_plan_info {
  int32_t n_workers;          /* workgroups = grid size */
  int32_t block_threads;      /* threads per workgroup */
  int32_t lds_bytes;          /* dynamic LDS per workgroup */
  int32_t waves_per_step;     /* waves (dependency levels) per decoded token */
  int32_t n_tiles;            /* tiles per step (all waves) */
  int32_t kv_splits;          /* S */
  int32_t combine_mode;       /* 1 prologue, 2 own wave */
  int32_t occupancy;          /* workgroups per CU the kernel can hold (0 in a dry run) */
  int64_t packed_bytes;       /* device bytes of the packed weights */
  int64_t weight_bytes_per_step; /* weight bytes one token streams (algorithmic) */
  double max_over_mean;       /* worst per-wave worker byte imbalance (max / mean over the busy workers of a GEMV wave) */
  uint64_t checksum;          /* schedule checksum (re-checked at every decode) */
  uint64_t build_id;          /* worker-kernel build id the plan was made for */
  int32_t attn_heads;         /* query heads per attention tile */
  int32_t o_workers;          /* workers holding o_proj tiles (all, or those without an attention tile) */
  int32_t weight_format;      /* TILES_WEIGHTS_BF16 or TILES_WEIGHTS_INT8 */
  int32_t top_k;              /* 0: greedy plan; else the plan samples (tiles_decode_sampled) */
  int32_t kv_format;          /* TILES_KV_BF16 or TILES_KV_INT8 */
  int32_t tokens_per_step;    /* positions per step: 1, or 2 .. 4 for a verify plan */
  int32_t stage_batches;      /* LDS staging batches per compute wavefront (0 .. 2; a verify plan may have none) */
} tiles_plan_info_t;

/* One wave of the per-step schedule (see tiles_plan_wave). */
typedef struct tiles_wave_info {
  int32_t kind;        /* 1 QKV, 2 attention, 3 split combine, 4 o_proj, 5 gate/up, 6 down, 7 LM head */
  int32_t layer;       /* -1 for the LM head */
  int32_t busy_workers;
  int32_t pad;
  int64_t weight_bytes;   /* weight bytes streamed by the wave, all workers */
  int64_t max_worker_bytes;
} tiles_wave_info_t;

/* Build, validate and upload a plan.  cfg and w are read only during the call;
 * the source weights may be freed afterwards (the plan keeps a packed copy).
 * Returns NULL on error (see tiles_last_error()).  Allocates device memory:
 * packed weights (= model bytes), RoPE table [max_positions][head_dim/2] x2 FP32,
 * the tagged-data buffers (one per wave), status words, and the debug/trace
 * buffers when flagged. */
tiles_plan_t *tiles_plan_create(const tiles_config_t *cfg, const tiles_weights_t *w);

/* Greedy-decode n_steps tokens (1..64) in one cooperative launch on the plan's stream.
 * Step i consumes `token` (i = 0) or out_tokens[i-1], at position kv->length + i, writes
 * that position's K and V, and stores its argmax (lowest index on ties) in out_tokens[i].
 *   kv          : host struct; kv->k / kv->v device BF16 cache; kv->length is advanced by
 *                 n_steps when the launch has been enqueued successfully.
 *   token       : 0 <= token < vocab.
 *   out_tokens  : device int32 [n_steps].
 *   out_logits  : device float [n_steps][vocab], or NULL to skip writing logits.
 * Asynchronous: results are valid after the stream synchronizes.  Errors detected on the
 * host (arguments, capacity, plan checksum, device identity) return before launching.
 * Allocates nothing. */
int tiles_decode(tiles_plan_t *plan, tiles_kv_t *kv, int32_t token, int32_t n_steps, int32_t *out_tokens,
                 float *out_logits);

/* Sampled decoding ("History and roadmap" (TileInfer.jl), "M8 so far" table: top-k/top-p sampling on
 * the device, inside the graph): as tiles_decode, but step i stores in out_tokens[i] the token drawn
 * from its logits with the plan's top_k / temperature / top_p (see tiles_config_t) and the uniform
 * uniforms[i], in the same cooperative launch (every worker draws the same token from every
 * worker's top_k candidates; no host round trip).
 *   uniforms : device float [n_steps], each in [0, 1) (values outside are clamped into it; NaN
 *              counts as 0).  The caller owns it; it is read during the launch.
 * Errors as tiles_decode, plus TILES_E_ARG for a greedy plan (top_k = 0) or null uniforms;
 * tiles_decode and tiles_decode_noalloc return TILES_E_ARG for a sampling plan.  Allocates nothing. */
int tiles_decode_sampled(tiles_plan_t *plan, tiles_kv_t *kv, int32_t token, int32_t n_steps, const float *uniforms,
                         int32_t *out_tokens, float *out_logits);

/* Greedy verify step ("History and roadmap" (TileInfer.jl), "M8 so far" table: verify steps of up
 * to 16 tokens on the split-KV decode kernels; "Milestones" M7: exact verification for greedy
 * decoding): m positions in one cooperative launch, position i (at kv->length + i) consuming the given
 * token tokens[i] -- the last accepted token, then m - 1 drafts -- and storing its argmax in
 * out_argmax[i] (lowest index on ties).  Draft tokens[i + 1] is accepted while out_argmax[i] equals it;
 * with n accepted, the verified output is tokens[1 .. n] followed by out_argmax[n], and the caller
 * sets the cache length to (length before the call) + n + 1 (rows written past it are overwritten
 * by later steps).  With a decode plan the m positions run as m steps of the decode launch (each
 * streams the weights once); a verify plan (tokens_per_step = T > 1) runs them as m / T steps of T
 * positions each, every tile taking the T positions of a step at once (one weight stream per step).
 *   tokens     : host int32 [m], each 0 <= t < vocab; read during the call.
 *   m          : 1 .. 64, a multiple of the plan's tokens_per_step.
 *   out_argmax : device int32 [m].   out_logits : device float [m][vocab], or NULL.
 * kv as tiles_decode (kv->length is advanced by m).  Errors as tiles_decode, plus TILES_E_ARG for a
 * sampling plan, null tokens, a token out of range or m not a multiple of tokens_per_step.  The
 * decode entry points return TILES_E_ARG for a verify plan.  Copies tokens[1 ..] into a buffer the plan
 * owns, on the plan's stream; allocates nothing. */
int tiles_verify(tiles_plan_t *plan, tiles_kv_t *kv, const int32_t *tokens, int32_t m, int32_t *out_argmax,
                 float *out_logits);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): tiles_decode with the same arguments, semantics and results,
 * except that the launch's tagged-data buffers, LM-head partials and status words live in a
 * file-scope device array of this library, 8 MiB per GPU, held from the first call on a GPU until
 * the process ends, instead of the plan's own buffers.  Calls no allocating routine (the plan must
 * exist already).  Errors as tiles_decode, plus TILES_E_ARG when the plan's scratch (its tagged
 * buffers: about (qkv rows + n_heads * splits * (head_dim + 4) + 2 * hidden + ffn) words per layer)
 * exceeds 8 MiB.  Every call on one GPU shares that array and each launch first clears what it
 * uses: calls that overlap on one GPU (in different streams, or from different threads) race and
 * give undefined results; sequential calls, also of different plans, are fine. */
int tiles_decode_noalloc(tiles_plan_t *plan, tiles_kv_t *kv, int32_t token, int32_t n_steps, int32_t *out_tokens,
                         float *out_logits);

/* Release every resource of the plan (synchronizes its stream first).  NULL-safe. */
void tiles_plan_destroy(tiles_plan_t *plan);

/* Message of the last error raised on the calling thread ("" if none). */
const char *tiles_last_error(void);

/* Fill *info for a plan. */
int tiles_plan_info(const tiles_plan_t *plan, tiles_plan_info_t *info);

/* Describe wave `wave` (0 <= wave < waves_per_step) of a plan. */
int tiles_plan_wave(const tiles_plan_t *plan, int32_t wave, tiles_wave_info_t *out);

/* Host-only planning: build and validate the schedule for `n_workers` workers without
 * touching any GPU (no device memory, no kernel).  Fills *info (occupancy = 0). */
int tiles_plan_dry_run(const tiles_config_t *cfg, int32_t n_workers, tiles_plan_info_t *info);

/* Test hook (host only, no GPU): build the schedule for `n_workers` workers as tiles_plan_dry_run does,
 * plant mistake number `mutation` in it (0 none; 1 rows covered twice, 2 a row covered by nobody,
 * 3 an attention tile duplicated, 4 one missing, 5 a split index out of range, 6 two waves' tagged
 * buffers overlapping, 7 one out of bounds, 8 a worker streaming two rows more than the balance
 * allows, 9 waves out of dependency order, 10 a step not ending with the LM head, 11 two tiles
 * reading the same packed bytes, 12 two tiles' packed rows exchanged, 13 a packing copy dropped,
 * 14 a norm gain misplaced, 15 more staging than the LDS layout holds) and run the plan validator
 * on the result.  Returns what the validator returns (TILES_E_PLAN with its message for every planted
 * mistake), or TILES_E_ARG for an unknown mutation or one the plan has no site for. */
int tiles_plan_debug_validate(const tiles_config_t *cfg, int32_t n_workers, int32_t mutation);

/* Change the stream used by subsequent decodes (hipStream_t, NULL = null stream). */
int tiles_plan_set_stream(tiles_plan_t *plan, void *stream);

/* Synchronize the plan's stream and report a device-side fault of the last launch, and clear it:
 * TILES_OK, TILES_E_KERNEL (a wait's watchdog expired) or TILES_E_PLAN (a worker found that the
 * schedule it loaded from device memory, or the build id stored with it, differs from what the plan
 * recorded at creation; that launch did nothing). */
int tiles_plan_status(tiles_plan_t *plan);

/* Copy debug buffers to host memory after synchronizing the plan's stream.
 *   hidden : host float [n_steps_of_last_decode][n_layers][H] or NULL (needs TILES_DEBUG_HIDDEN);
 *   trace  : host uint64 [n_steps / tokens_per_step][waves_per_step][n_workers][12] or NULL (needs
 *            TILES_TRACE; one record per kernel step, which a verify plan runs per tokens_per_step positions),
 *            100 MHz wall-clock ticks per (step, wave, worker): 0 wave start, 1 inputs staged,
 *            2 compute done, 3 outputs published, 7 after the LDS prologue (control wavefront);
 *            5 own gather done, 6 after the LDS prologue, 9 streaming loop entered, 8 first
 *            batch consumed, 4 own share of the tile done (first compute wavefront, GEMV and
 *            attention tiles; 4, 8 and 9 are 0 when it had no share, all five are 0 for other
 *            tiles); 11 the last compute wavefront's share done (GEMV and attention tiles),
 *            10 the control wavefront ready for barrier B after its KV-row write (attention
 *            tiles, else 0).
 *   *n_steps_out receives the position count of the last decode or verify call. */
int tiles_read_debug(tiles_plan_t *plan, float *hidden, uint64_t *trace, int32_t *n_steps_out);

/* Test hook: corrupt one byte of the host copy of the schedule so that the next
 * decode must fail its checksum (TILES_E_PLAN).  Does not touch the device. */
int tiles_plan_debug_corrupt(tiles_plan_t *plan);

/* Test hook: flip one bit of the device-resident copy of the schedule (a tile's weight offset) and
 * leave the host copy alone.  The next decode's launch detects it before the corrupted entry is used
 * (the worker holding it re-hashes the schedule it loaded and leaves; the others leave at their next
 * wait) and tiles_plan_status then reports TILES_E_PLAN.  The plan stays corrupted. */
int tiles_plan_debug_corrupt_device(tiles_plan_t *plan);

/* Test hook: the watchdog of every wait in later decodes of this plan -- after `rounds`
 * unanswered polling rounds a wait gives up, the launch ends early (every worker leaves after
 * its next input barrier) and tiles_plan_status reports TILES_E_KERNEL.  0 restores the default
 * (2^22 rounds, seconds).  A small value makes ordinary waits give up, which exercises that path
 * without any fault; under 32 rounds the plan launches a test instantiation of the worker that
 * checks its watchdog every round (BF16 weights and KV, greedy, one query head per attention tile
 * and one position per step only: TILES_E_CONFIG otherwise).  Host only (plus an occupancy query of
 * that instantiation). */
int tiles_plan_debug_spin_limit(tiles_plan_t *plan, uint32_t rounds);

/* The weight-only INT8 quantizer plan creation applies to every linear layer ("History and roadmap"
 * (TileInfer.jl), "M8 so far" table: weight-only INT8 linear layers; per-row scales, as group-wise
 * scales were not tried there): for each of `rows` rows of `cols` BF16 values (host memory, row-major),
 * s = max |w| / 127 and q = round-half-even(w / s) clamped to [-127, 127], each operation in IEEE FP32;
 * a row of zeros gets s = 0 and q = 0.  q: host int8 [rows][cols]; scales: host float [rows].  Host
 * only (no GPU).  Errors: TILES_E_ARG for a null pointer or a negative size. */
int tiles_quantize_rows_int8(const uint16_t *bf16, int64_t rows, int64_t cols, int8_t *q, float *scales);

/* Measurement helper, not part of the decode path: the stream-read ceiling against which the
 * decode kernel's HBM rate is compared ("History and roadmap" page, "Where it stands": decode
 * speed is stated as a fraction of what memory bandwidth allows).  Reads `bytes` of device
 * memory at `buf` with the decode kernel's load form -- 16-byte non-temporal loads, one 1 KB
 * chunk per wavefront instruction, 8 chunks in flight per wavefront -- in `n_groups`
 * workgroups of 512 threads, each wavefront one contiguous share, and XORs every word read
 * into the device word *sink (so the loads cannot be dropped; the caller zeroes it first if
 * it wants the checksum).  Asynchronous on `stream` (hipStream_t, NULL = null stream); the
 * caller times it.  buf and sink are caller-owned device memory.  Errors: TILES_E_ARG for a
 * null pointer, n_groups outside [1, 65536], or bytes not a positive multiple of
 * n_groups * 8 * 8192 (or above 4 GB per wavefront); TILES_E_HIP for a launch error. */
int tiles_stream_read(const void *buf, int64_t bytes, int32_t n_groups, uint32_t *sink, void *stream);

/* Measurement helper, not part of the decode path: the latency floor of one dependency edge
 * (Tiles page, introduction: what the synchronisation between waves costs decides whether a
 * static schedule pays).  Workgroups 0 and `peer` of a (peer + 1)-workgroup launch, one lane
 * each, pass a counter 1, 2, ..., iters back and forth through words[0] and words[16] with the
 * decode kernel's publish (agent-scope store) and poll (device-coherent load) forms.  Workgroups
 * are dealt to the 8 XCDs in turn, so a peer that is a multiple of 8 shares workgroup 0's XCD.
 * out[0] receives the wall-clock ticks (100 MHz) workgroup 0 spent on the whole exchange
 * (iters round trips); out[1] / out[2] become nonzero if the peer / workgroup 0 gave up a wait
 * after `spin_limit` polls (the exchange then ends early, no wait is unbounded).  words (at
 * least 17 words, zeroed by the caller before every call) and out (3 words) are caller-owned
 * device memory.  Asynchronous on `stream` (hipStream_t, NULL = null stream).  Errors:
 * TILES_E_ARG for a null pointer, peer outside [1, 255], iters outside [1, 2^20] or a zero
 * spin_limit; TILES_E_HIP for a launch error. */
int tiles_edge_latency(uint32_t *words, int32_t peer, int32_t iters, uint32_t spin_limit, uint64_t *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* TILES_H */
