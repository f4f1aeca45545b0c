// Host planner: cuts every operator of a decoder step into output-row tiles, assigns the
// tiles of each wave to fixed workers, picks the split-KV count, lays out the packed
// weights and validates the result.
//
// The planning rules follow "Tiles: Scheduling LLM Decoding as a Graph of Tiles" (intro):
// a tile is a small range of output rows plus the work that produces it; small operations
// fold into neighbouring tiles; each tile has a fixed worker, one worker per compute unit;
// the planner balances the bytes each worker streams and groups tiles into waves (the pages
// separate them with grid barriers; here each wave's tagged outputs carry the dependency);
// the schedule is validated before launch.  The fusions are those of the
// "M8 so far" table of the TileInfer.jl roadmap (residual add + RMSNorm, SwiGLU in the GEMV,
// q/k norm + RoPE + KV write), and attention is split over KV positions as in its "Milestones"
// table (M5, split-KV decode kernel); the roadmap's "Tried and not kept" table found a
// separate combine faster than one fused into the split kernel, which is the reason the
// split merge lives in the o_proj prologue or a wave of its own, never in the split tiles.
#include "planner.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <sstream>
#include <tuple>
#include <unordered_map>

namespace tiles {

namespace {

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

uint32_t float_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

// rows [lo, hi) of `R` rows for worker w of W: balanced to within one row.
void row_split(int64_t R, int32_t W, int32_t w, int64_t& lo, int64_t& hi) {
  lo = R * w / W;
  hi = R * (w + 1) / W;
}

struct TileIO {  // read and write sets of one tile, for the hazard check
  std::vector<Interval> reads, writes;
};

int fail(std::string& err, int code, const std::string& msg) {
  err = msg;
  return code;
}

// Split count: about `target` bytes of K+V per split tile at the largest attended
// length, at least 1, at most as many tiles as workers.
// Split partials of all heads up to this size are merged in the o_proj prologue (combine mode 0).
constexpr int64_t COMBINE_IN_O_BYTES = 68 * 1024;

int32_t choose_splits(const Shape& s, int32_t W) {
  // Preferably a split's K/V rows fit the compute wavefronts' register prefetch (STREAM_DEPTH
  // 16-byte loads per lane, NCOMP wavefronts), so that its attention runs in one pass, as long
  // as the partials still merge in the o_proj prologue; else about 96 KB of K/V per split.
  const int64_t kv_head_bytes = (int64_t)s.max_positions * s.hd * 2 /*K,V*/ * 2 /*bf16*/;
  const int64_t one_pass = (int64_t)NCOMP * STREAM_DEPTH * 64 * 16;
  const int64_t split_record_bytes = (int64_t)s.n_heads * (s.hd + 4) * 4;
  int64_t S = (kv_head_bytes + one_pass - 1) / one_pass;
  if (S * split_record_bytes > COMBINE_IN_O_BYTES) {
    const int64_t target = 96 * 1024;
    S = (kv_head_bytes + target / 2) / target;
    // A merge wave of its own costs a dependency edge per layer: when at least two thirds of
    // those splits still merge in the prologue, take that count instead (Qwen3-4B shape at 1K
    // positions: 4 splits merged in o_proj measured faster than 6 with a merge wave).
    const int64_t fit = COMBINE_IN_O_BYTES / split_record_bytes;
    if (S * split_record_bytes > COMBINE_IN_O_BYTES && fit >= 1 && 3 * fit >= 2 * S) S = fit;
  }
  S = std::max<int64_t>(1, std::min<int64_t>(S, W / s.n_kv));
  return (int32_t)S;
}

}  // namespace

void quantize_rows_int8(const uint16_t* src, int64_t src_pitch, int64_t rows, int64_t cols, int8_t* q,
                        int64_t q_pitch, float* scales, int64_t scale_pitch_floats) {
  auto widen = [](uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
  };
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* w = src + r * src_pitch;
    float amax = 0.0f;
    for (int64_t j = 0; j < cols; ++j) amax = std::max(amax, std::fabs(widen(w[j])));
    const float sc = amax / 127.0f;  // IEEE FP32 division
    int8_t* qr = q + r * q_pitch;
    for (int64_t j = 0; j < cols; ++j) {
      float v = sc > 0.0f ? std::nearbyint(widen(w[j]) / sc) : 0.0f;  // round half to even (default mode)
      v = std::min(127.0f, std::max(-127.0f, v));
      qr[j] = (int8_t)v;
    }
    scales[r * scale_pitch_floats] = sc;
  }
}

uint64_t plan_checksum(const HostPlan& p) {
  // 64-bit words mixed with a multiply-xorshift step (FNV-style); fast enough to run before every launch.
  uint64_t h = 1469598103934665603ull;
  auto word = [&](uint64_t v) {
    h ^= v;
    h *= 1099511628211ull;
    h ^= h >> 29;
  };
  auto mix = [&](const void* data, size_t n) {
    const unsigned char* b = static_cast<const unsigned char*>(data);
    size_t i = 0;
    for (; i + 8 <= n; i += 8) {
      uint64_t v;
      std::memcpy(&v, b + i, 8);
      word(v);
    }
    uint64_t tail = 0;
    if (i < n) std::memcpy(&tail, b + i, n - i);
    word(tail ^ ((uint64_t)n << 56));
  };
  const Shape& s = p.s;
  const int64_t dims[] = {s.n_layers, s.H, s.n_heads, s.n_kv, s.hd, s.F, s.V, s.G, s.qkv_rows, s.Hpad, s.Qpad, s.Fpad,
                          s.qk_norm ? 1 : 0, s.tied ? 1 : 0, s.max_positions, p.W, p.S, p.combine_in_o, p.T, p.q8, p.wb,
                          p.final_norm_off, p.embed_off, p.embed_stride, p.packed_bytes, p.lds_vec_floats,
                          p.lds_part_floats, p.lds_xres_floats, p.lds_bytes, p.ll_words, p.lds_stage_floats,
                          p.stage_batches, p.top_k, (int64_t)float_bits(p.temperature), (int64_t)float_bits(p.top_p),
                          p.kv8, p.mt, p.kv8_span};
  mix(dims, sizeof(dims));
  if (!p.waves.empty()) mix(p.waves.data(), p.waves.size() * sizeof(WaveDesc));
  if (!p.tiles.empty()) mix(p.tiles.data(), p.tiles.size() * sizeof(TileDesc));
  if (!p.small.empty()) mix(p.small.data(), p.small.size() * sizeof(LayerSmall));
  return h;
}

std::vector<uint64_t> worker_table_hashes(const HostPlan& p) {
  std::vector<uint64_t> out(p.W, 0);
  const size_t nw = p.waves.size();
  std::vector<uint32_t> common((nw * sizeof(WaveDesc) + p.small.size() * sizeof(LayerSmall)) / 4);
  if (nw) std::memcpy(common.data(), p.waves.data(), nw * sizeof(WaveDesc));
  if (!p.small.empty()) std::memcpy(common.data() + nw * sizeof(WaveDesc) / 4, p.small.data(), p.small.size() * sizeof(LayerSmall));
  constexpr size_t TW = sizeof(TileDesc) / 4;
  for (int32_t w = 0; w < p.W; ++w) {
    uint64_t h = 0, i = 0;
    for (size_t k = 0; k < nw; ++k) {
      uint32_t t[TW];
      std::memcpy(t, &p.tiles[k * p.W + w], sizeof(TileDesc));
      for (size_t j = 0; j < TW; ++j, ++i) h += table_mix((i << 32) | t[j]);
    }
    for (uint32_t x : common) h += table_mix((i++ << 32) | x);
    out[w] = h;
  }
  return out;
}

// Multi-token plans: GEMV row blocks of at least this many rows (their partials are held per position).
constexpr int32_t MIN_MT_BLOCK_ROWS = 64;

// LDS floats of an attention tile's work areas: q[mt * T][hd], kc[mt][hd], vc[mt][hd], the compute
// waves' states [NCOMP][mt * T][hd + 4] and the merged partial [mt * T][hd + 4]; multi-token steps add
// one RoPE row (hd floats) per position (one-position steps keep theirs in the small area).
static int64_t attn_lds_floats(const HostPlan& p) {
  const int64_t rows = (int64_t)p.mt * p.T, hd = p.s.hd;
  return rows * hd + 2 * p.mt * hd + (NCOMP + 1) * rows * (hd + 4) + (p.mt > 1 ? p.mt * hd : 0);
}

// Floats of one position's GEMV input area (the largest input, or an attention tile's raw q/k/v).
static int64_t vec_floats(const Shape& s) {
  return round_up(std::max<int64_t>({s.Hpad, s.Qpad, s.Fpad, (int64_t)(s.G + 2) * s.hd}), 64);
}

// Multi-token plans whose o_proj prologue merges the splits keep the merged heads of the mt positions
// at the start of the input area (Qpad apart) and every position's split partials after them, on
// into the partial area: those two areas together must hold mt * (Qpad + n_heads * S * (hd + 4)).
static int64_t mt_merge_floats(const HostPlan& p) {
  return (int64_t)p.mt * (p.s.Qpad + (int64_t)p.s.n_heads * p.S * (p.s.hd + 4));
}

// Whether that layout fits the LDS beside the residual rows, the small area, the schedule tables
// (one wave per kind and layer, plus the LM head), the smallest GEMV row blocks and one staging batch.
static bool mt_merge_in_o_fits(const HostPlan& p) {
  if (p.mt == 1) return true;
  const Shape& s = p.s;
  const int64_t vs = vec_floats(s);
  const int64_t vec_part = std::max<int64_t>(p.mt * vs + (int64_t)MIN_MT_BLOCK_ROWS * NCOMP * p.mt, mt_merge_floats(p));
  const int64_t xres = p.mt * round_up(s.Hpad, 64) + (p.q8 ? MAX_BLOCK_ROWS : 0);
  const int64_t n_waves = (int64_t)s.n_layers * 5 + 1;
  const int64_t tables = round_up(n_waves * (int64_t)(sizeof(SegDesc) + sizeof(TileDesc) + sizeof(WaveDesc)) +
                                      (int64_t)s.n_layers * (int64_t)sizeof(LayerSmall), 256);
  return (vec_part + xres + SMALL_FLOATS) * 4 + tables + (int64_t)NCOMP * STREAM_BATCH * CHUNK_BYTES <= LDS_LIMIT;
}

int build_plan(const tiles_config_t& cfg, int32_t n_workers, HostPlan& p, std::string& err) {
  p = HostPlan();
  Shape& s = p.s;
  s.n_layers = cfg.n_layers;
  s.H = cfg.hidden;
  s.n_heads = cfg.n_heads;
  s.n_kv = cfg.n_kv_heads;
  s.hd = cfg.head_dim;
  s.F = cfg.ffn;
  s.V = cfg.vocab;
  s.qk_norm = cfg.qk_norm != 0;
  s.tied = cfg.tie_embeddings != 0;
  s.max_positions = cfg.max_positions;
  if (s.n_layers < 1 || s.H < 1 || s.n_heads < 1 || s.n_kv < 1 || s.F < 1 || s.V < 1)
    return fail(err, TILES_E_CONFIG, "non-positive model dimension");
  if (s.hd != 64 && s.hd != 128) return fail(err, TILES_E_CONFIG, "head_dim must be 64 or 128");
  if (s.n_heads % s.n_kv != 0) return fail(err, TILES_E_CONFIG, "n_kv_heads must divide n_heads");
  s.G = s.n_heads / s.n_kv;
  if (s.G > MAX_GROUP) return fail(err, TILES_E_CONFIG, "more than 4 query heads per KV head");
  if (s.max_positions < 1) return fail(err, TILES_E_CONFIG, "max_positions must be >= 1");
  // positions and byte offsets within one KV head's cache rows are 32-bit in the kernel
  if (s.max_positions > MAX_POSITIONS) return fail(err, TILES_E_CONFIG, "max_positions above 2^23");
  if (!(cfg.rms_eps > 0.0f) || !(cfg.rope_theta > 1.0f)) return fail(err, TILES_E_CONFIG, "bad rms_eps or rope_theta");
  if (n_workers < 1) return fail(err, TILES_E_CONFIG, "n_workers must be >= 1");
  if (n_workers < s.n_heads || n_workers < s.n_kv) return fail(err, TILES_E_CONFIG, "fewer workers than attention heads");
  if (s.n_heads * s.hd > 65536 || s.H > 65536 || s.F > 65536) return fail(err, TILES_E_CONFIG, "dimension too large");
  if (s.H % 4 != 0 || s.F % 4 != 0) return fail(err, TILES_E_CONFIG, "hidden and ffn must be multiples of 4");
  p.W = n_workers;
  const int32_t W = n_workers;
  s.qkv_rows = (s.n_heads + 2 * s.n_kv) * s.hd;
  // weight format: BF16, or weight-only INT8 (every linear layer as per-row INT8 codes + FP32 scales)
  if (cfg.weight_format != WEIGHTS_BF16 && cfg.weight_format != WEIGHTS_INT8)
    return fail(err, TILES_E_CONFIG, "weight_format must be 0 (BF16) or 1 (INT8)");
  p.q8 = cfg.weight_format == WEIGHTS_INT8;
  p.wb = p.q8 ? 1 : 2;
  if (cfg.top_k < 0 || cfg.top_k > MAX_TOP_K || cfg.top_k > cfg.vocab)
    return fail(err, TILES_E_CONFIG, "top_k must be 0 (greedy) or in [1, min(32, vocab)]");
  if (cfg.top_k > 0 && !(cfg.temperature > 0.0f && cfg.temperature < 1e30f && cfg.top_p > 0.0f && cfg.top_p <= 1.0f))
    return fail(err, TILES_E_CONFIG, "sampling needs 0 < temperature (finite) and 0 < top_p <= 1");
  if (cfg.top_k > 0 && n_workers > 256)
    return fail(err, TILES_E_CONFIG, "sampled decoding supports at most 256 workers (the token draw merges 4 lists per lane)");
  if (cfg.kv_format != KVFMT_BF16 && cfg.kv_format != KVFMT_INT8)
    return fail(err, TILES_E_CONFIG, "kv_format must be 0 (BF16) or 1 (INT8)");
  p.kv8 = cfg.kv_format == KVFMT_INT8;
  // verify plans: every step runs tokens_per_step consecutive teacher-forced positions through each
  // tile (one weight stream for all of them)
  if (cfg.tokens_per_step < 0 || cfg.tokens_per_step > MAX_STEP_TOKENS)
    return fail(err, TILES_E_CONFIG, "tokens_per_step must be 0 .. 4");
  p.mt = cfg.tokens_per_step > 1 ? cfg.tokens_per_step : 1;
  if (p.mt > 1 && cfg.top_k > 0) return fail(err, TILES_E_CONFIG, "multi-token steps are greedy verify steps");
  p.top_k = cfg.top_k;
  p.temperature = cfg.top_k > 0 ? cfg.temperature : 1.0f;
  p.top_p = cfg.top_k > 0 ? cfg.top_p : 1.0f;
  const int32_t ccols = CHUNK_BYTES / p.wb;  // columns per packed chunk
  s.Hpad = (int32_t)round_up(s.H, ccols);
  s.Qpad = (int32_t)round_up((int64_t)s.n_heads * s.hd, ccols);
  s.Fpad = (int32_t)round_up(s.F, ccols);
  const int64_t wb = p.wb;

  // split-KV and combine placement
  p.S = cfg.kv_splits > 0 ? cfg.kv_splits : choose_splits(s, W);
  // INT8 KV: a split's per-position scales are staged in LDS, at most MAX_SPLIT_POSITIONS_KV8 of them
  if (p.kv8 && cfg.kv_splits <= 0)
    p.S = std::max<int32_t>(p.S, (int32_t)((s.max_positions + MAX_SPLIT_POSITIONS_KV8 - 1) / MAX_SPLIT_POSITIONS_KV8));
  if (p.kv8 && (s.max_positions + p.S - 1) / p.S > MAX_SPLIT_POSITIONS_KV8)
    return fail(err, TILES_E_CONFIG, "INT8 KV: more than 4096 positions per split (raise kv_splits)");
  // query heads per attention tile: the group's heads spread over as many tiles as the workers
  // allow (each re-reads the split's K/V rows; attention is bound by arithmetic per head)
  if (cfg.attn_heads > 0) {
    p.T = cfg.attn_heads;
    if (s.G % p.T != 0) return fail(err, TILES_E_CONFIG, "attn_heads must divide n_heads / n_kv_heads");
  } else {
    // the first divisor whose tiles fit the workers, else the largest (then rejected below); multi-token
    // steps: at most MAX_GROUP query rows per tile, heads x positions
    p.T = 0;
    for (int32_t t = 1; t <= s.G; ++t)
      if (s.G % t == 0 && t * p.mt <= MAX_GROUP) {
        p.T = t;
        if ((int64_t)s.n_kv * (s.G / t) * std::max(p.S, 1) <= W) break;
      }
  }
  if (p.T * p.mt > MAX_GROUP)
    return fail(err, TILES_E_CONFIG, "attn_heads x tokens_per_step exceeds 4 query rows per attention tile");
  // a verify plan whose bound on heads per tile leaves more attention tiles than workers takes fewer
  // splits (the planner's own count only; the Qwen3-4B shape at 32K positions: 16 instead of 32)
  if (p.mt > 1 && cfg.kv_splits <= 0 && (int64_t)p.S * s.n_kv * (s.G / p.T) > W)
    p.S = std::max<int32_t>(1, W / (s.n_kv * (s.G / p.T)));
  if (p.kv8 && (s.max_positions + p.S - 1) / p.S > MAX_SPLIT_POSITIONS_KV8)
    return fail(err, TILES_E_CONFIG, "INT8 KV: more than 4096 positions per split (raise kv_splits, or fewer positions)");
  // INT8 KV: the LDS scale areas hold the longest split (a split of a launch's step never holds more
  // positions than one at the cache's capacity)
  if (p.kv8) p.kv8_span = (int32_t)round_up((s.max_positions + p.S - 1) / p.S, 64);
  if (p.S < 1 || (int64_t)p.S * s.n_kv * (s.G / p.T) > W)
    return fail(err, TILES_E_CONFIG, "kv_splits * n_kv_heads * (query heads per KV head / attn_heads) exceeds workers");
  const int64_t part_bytes = (int64_t)s.n_heads * p.S * (s.hd + 4) * 4;
  if (cfg.o_placement < 0 || cfg.o_placement > 2) return fail(err, TILES_E_CONFIG, "o_placement must be 0, 1 or 2");
  if (cfg.combine_mode == 1) p.combine_in_o = 1;
  else if (cfg.combine_mode == 2) p.combine_in_o = 0;
  else if (cfg.combine_mode == 0) p.combine_in_o = part_bytes <= COMBINE_IN_O_BYTES && mt_merge_in_o_fits(p) ? 1 : 0;
  else return fail(err, TILES_E_CONFIG, "combine_mode must be 0, 1 or 2");

  // ---- packed layout: norm gains first, then the GEMV waves in execution order ----
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    int64_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  p.small.resize(s.n_layers);
  for (int l = 0; l < s.n_layers; ++l) {
    LayerSmall& ls = p.small[l];
    ls.attn_norm = take((int64_t)s.H * 2);
    p.copies.push_back({SRC_ATTN_NORM, l, 0, 1, s.H, ls.attn_norm, (int64_t)s.H * 2});
    ls.mlp_norm = take((int64_t)s.H * 2);
    p.copies.push_back({SRC_MLP_NORM, l, 0, 1, s.H, ls.mlp_norm, (int64_t)s.H * 2});
    if (s.qk_norm) {
      ls.q_norm = take((int64_t)s.hd * 2);
      p.copies.push_back({SRC_Q_NORM, l, 0, 1, s.hd, ls.q_norm, (int64_t)s.hd * 2});
      ls.k_norm = take((int64_t)s.hd * 2);
      p.copies.push_back({SRC_K_NORM, l, 0, 1, s.hd, ls.k_norm, (int64_t)s.hd * 2});
    } else {
      ls.q_norm = ls.k_norm = -1;
    }
  }
  p.final_norm_off = take((int64_t)s.H * 2);
  p.copies.push_back({SRC_FINAL_NORM, -1, 0, 1, s.H, p.final_norm_off, (int64_t)s.H * 2});
  off = round_up(off, CHUNK_BYTES);

  int64_t wbytes = 0;  // algorithmic weight bytes per step
  for (int l = 0; l < s.n_layers; ++l) wbytes += (int64_t)s.H * 2 * 2 + (s.qk_norm ? (int64_t)s.hd * 2 * 2 : 0);
  wbytes += (int64_t)s.H * 2;  // final norm

  auto new_wave = [&](int32_t kind, int32_t layer) {
    p.waves.push_back({kind, layer, 0, -1});
    p.tiles.resize(p.waves.size() * (size_t)W);
    for (int w = 0; w < W; ++w) {
      TileDesc& t = p.tiles[(p.waves.size() - 1) * W + w];
      std::memset(&t, 0, sizeof(t));
      t.kind = KIND_NONE;
    }
    return (int32_t)p.waves.size() - 1;
  };
  auto tile_at = [&](int32_t wave, int32_t w) -> TileDesc& { return p.tiles[(size_t)wave * W + w]; };

  // A GEMV wave over R output rows of width K (padded to kpad).  `seg` emits the
  // copy segments for worker rows [lo, hi) given the destination offset.
  // `on` (optional) restricts the wave to these workers, in increasing order.
  auto gemv_wave = [&](int32_t kind, int32_t layer, int64_t R, int32_t K, int32_t kpad, int32_t rows_per_out,
                       auto&& seg, const std::vector<int32_t>* on = nullptr) {
    int32_t wv = new_wave(kind, layer);
    int32_t max_rows = 0;
    const int32_t n_on = on ? (int32_t)on->size() : W;
    for (int i = 0; i < n_on; ++i) {
      const int w = on ? (*on)[i] : i;
      int64_t lo, hi;
      row_split(R, n_on, i, lo, hi);
      if (hi <= lo) continue;
      TileDesc& t = tile_at(wv, w);
      t.kind = kind;
      t.row0 = (int32_t)lo;
      t.nrows = (int32_t)(hi - lo);
      t.kpad = kpad;
      t.woff = off;
      seg(lo, hi, off);
      const int64_t rows = (hi - lo) * rows_per_out;
      max_rows = std::max<int32_t>(max_rows, (int32_t)rows);
      off += tile_packed_bytes(p, t);
    }
    p.waves[wv].max_rows = max_rows;
    // algorithmic bytes: the weights (and, INT8, one FP32 scale per row)
    wbytes += R * rows_per_out * ((int64_t)K * wb + (p.q8 ? 4 : 0));
    return wv;
  };

  // With one KV head per XCD (8 KV heads, and that head's attention tiles fit the XCD's workers),
  // each KV head's QKV rows (its query heads, k and v) and its attention tiles go to workers of
  // one XCD (index equal to the KV head mod XCDS): the QKV -> attention dependency then stays
  // inside that XCD (a published word reaches a poller there sooner than one on another XCD;
  // measured +0.1 to +0.3 %).  A QKV tile belongs to the KV head of its first row; tiles beyond
  // an XCD's share go to XCDs with free workers.
  const int64_t qr0 = (int64_t)s.n_heads * s.hd, kr0 = (int64_t)s.n_kv * s.hd;
  const bool kv_per_xcd = s.n_kv == XCDS && W % XCDS == 0 && (int64_t)(s.G / p.T) * p.S <= W / XCDS;
  std::vector<int32_t> qkv_on;
  if (kv_per_xcd) {
    const int32_t cap = W / XCDS;
    std::vector<int32_t> cnt(XCDS, 0), over;
    qkv_on.assign(W, -1);
    for (int i = 0; i < W; ++i) {
      int64_t lo, hi;
      row_split(s.qkv_rows, W, i, lo, hi);
      const int64_t r = lo < s.qkv_rows ? lo : s.qkv_rows - 1;
      const int32_t g = (int32_t)(r < qr0 ? r / s.hd / s.G : r < qr0 + kr0 ? (r - qr0) / s.hd : (r - qr0 - kr0) / s.hd);
      if (cnt[g] < cap) qkv_on[i] = g + XCDS * cnt[g]++;
      else over.push_back(i);
    }
    for (int i : over)
      for (int g = 0; g < XCDS; ++g)
        if (cnt[g] < cap) {
          qkv_on[i] = g + XCDS * cnt[g]++;
          break;
        }
  }
  for (int l = 0; l < s.n_layers; ++l) {
    // QKV: rows of [Wq; Wk; Wv]
    const int64_t qr = (int64_t)s.n_heads * s.hd, kr = (int64_t)s.n_kv * s.hd;
    gemv_wave(KIND_QKV, l, s.qkv_rows, s.H, s.Hpad, 1, [&](int64_t lo, int64_t hi, int64_t dst) {
      const int64_t bounds[4] = {0, qr, qr + kr, qr + 2 * kr};
      const int32_t src[3] = {SRC_WQ, SRC_WK, SRC_WV};
      const int64_t scl = dst + (hi - lo) * s.Hpad * wb;
      for (int m = 0; m < 3; ++m) {
        int64_t a = std::max(lo, bounds[m]), b = std::min(hi, bounds[m + 1]);
        if (b > a)
          p.copies.push_back({src[m], l, a - bounds[m], b - a, s.H, dst + (a - lo) * s.Hpad * wb, (int64_t)s.Hpad * wb,
                              p.q8 ? scl + (a - lo) * 4 : -1, p.q8 ? 4 : 0});
      }
    }, kv_per_xcd ? &qkv_on : nullptr);
    // attention: one tile per (KV head, group of T query heads, split).  The tiles that read the
    // same K/V rows (one KV head and split, every query-head group) go to workers on one XCD:
    // workgroups are dealt to the XCDs in turn, so workers with equal index mod XCDS share an L2,
    // which then serves all but the first read of those rows (measured +0.2 to +0.6 %).  With one
    // KV head per XCD, all of a KV head's tiles go to its XCD (see the QKV placement above).
    int32_t attn_wv = -1;
    {
      int32_t wv = attn_wv = new_wave(KIND_ATTN, l);
      const int32_t nhs = s.G / p.T;
      const int32_t units = s.n_kv * p.S;  // distinct K/V ranges
      const bool xcd_groups = (int64_t)(units + XCDS - 1) / XCDS * XCDS * nhs <= W;
      for (int g = 0; g < s.n_kv; ++g)
        for (int hs = 0; hs < nhs; ++hs)
          for (int sp = 0; sp < p.S; ++sp) {
            const int32_t u = g * p.S + sp;
            const int32_t w = kv_per_xcd ? g + XCDS * (hs * p.S + sp)
                              : xcd_groups ? (u / XCDS) * XCDS * nhs + hs * XCDS + u % XCDS : (g * nhs + hs) * p.S + sp;
            TileDesc& t = tile_at(wv, w);
            t.kind = KIND_ATTN;
            t.row0 = g;
            t.nrows = sp;
            t.aux0 = g * s.G + hs * p.T;  // first query head
          }
    }
    if (!p.combine_in_o) {
      int32_t wv = new_wave(KIND_COMBINE, l);
      for (int h = 0; h < s.n_heads; ++h) {
        TileDesc& t = tile_at(wv, h);
        t.kind = KIND_COMBINE;
        t.row0 = h;
      }
    }
    // o_proj on all workers (planner choice), or on the workers without an attention tile
    // (o_placement 2, splits merged in the o_proj prologue): those can prefetch their whole o_proj
    // share while the attention tiles run, and the attention workers go straight on to gate/up.
    // Measured on the 1B Llama shape the second costs 1.7 %: the o_proj workers reach gate/up with
    // less of it prefetched.
    std::vector<int32_t> o_workers;
    if (p.combine_in_o && cfg.o_placement == 2)
      for (int w = 0; w < W; ++w)
        if (tile_at(attn_wv, w).kind == KIND_NONE) o_workers.push_back(w);
    gemv_wave(KIND_O, l, s.H, s.n_heads * s.hd, s.Qpad, 1, [&](int64_t lo, int64_t hi, int64_t dst) {
      p.copies.push_back({SRC_WO, l, lo, hi - lo, (int64_t)s.n_heads * s.hd, dst, (int64_t)s.Qpad * wb,
                          p.q8 ? dst + (hi - lo) * s.Qpad * wb : -1, p.q8 ? 4 : 0});
    }, o_workers.empty() ? nullptr : &o_workers);
    // gate and up rows interleaved (gate j, up j, gate j+1, ...) so any even row block holds whole pairs
    gemv_wave(KIND_GU, l, s.F, s.H, s.Hpad, 2, [&](int64_t lo, int64_t hi, int64_t dst) {
      const int64_t scl = dst + 2 * (hi - lo) * s.Hpad * wb;  // scales interleaved like the rows
      p.copies.push_back({SRC_WGATE, l, lo, hi - lo, s.H, dst, (int64_t)s.Hpad * wb * 2, p.q8 ? scl : -1, p.q8 ? 8 : 0});
      p.copies.push_back({SRC_WUP, l, lo, hi - lo, s.H, dst + (int64_t)s.Hpad * wb, (int64_t)s.Hpad * wb * 2,
                          p.q8 ? scl + 4 : -1, p.q8 ? 8 : 0});
    });
    gemv_wave(KIND_DOWN, l, s.H, s.F, s.Fpad, 1, [&](int64_t lo, int64_t hi, int64_t dst) {
      p.copies.push_back({SRC_WDOWN, l, lo, hi - lo, s.F, dst, (int64_t)s.Fpad * wb,
                          p.q8 ? dst + (hi - lo) * s.Fpad * wb : -1, p.q8 ? 4 : 0});
    });
  }
  const int64_t lm_base = off;
  gemv_wave(KIND_LM, -1, s.V, s.H, s.Hpad, 1, [&](int64_t lo, int64_t hi, int64_t dst) {
    p.copies.push_back({s.tied ? SRC_EMBED : SRC_LM_HEAD, -1, lo, hi - lo, s.H, dst, (int64_t)s.Hpad * wb,
                        p.q8 ? dst + (hi - lo) * s.Hpad * wb : -1, p.q8 ? 4 : 0});
  });
  wbytes += (int64_t)s.H * 2;  // one (BF16) embedding row per token
  if (s.tied && !p.q8) {
    p.embed_off = lm_base;  // LM-head rows are the embedding rows, in order
    p.embed_stride = (int64_t)s.Hpad * 2;
  } else {
    // the lookup reads BF16 rows of their own (untied, or an INT8 head)
    const int64_t stride = round_up((int64_t)s.H * 2, 256);
    p.embed_off = off;
    p.embed_stride = stride;
    p.copies.push_back({SRC_EMBED, -1, 0, s.V, s.H, off, stride});
    off += (int64_t)s.V * stride;
  }
  p.packed_bytes = round_up(off, 4096);
  p.weight_bytes_per_step = wbytes;

  // ---- tagged output buffers, one per wave (64-word aligned) ----
  {
    int64_t w_off = 0;
    for (WaveDesc& wd : p.waves) {
      const int64_t n = wave_out_words(s, p.S, wd.kind);
      if (n == 0) {
        wd.ll_off = -1;
        continue;
      }
      wd.ll_off = (int32_t)w_off;
      w_off = round_up(w_off + n, 64);
    }
    p.ll_words = w_off;
  }

  // ---- per-wave bytes and balance ----
  const int nw = (int)p.waves.size();
  p.wave_bytes.assign(nw, 0);
  p.wave_max_bytes.assign(nw, 0);
  p.wave_busy.assign(nw, 0);
  double worst = 1.0;
  for (int wv = 0; wv < nw; ++wv) {
    int64_t tot = 0, mx = 0, row_bytes = 0;
    int busy = 0;
    for (int w = 0; w < W; ++w) {
      const TileDesc& t = p.tiles[(size_t)wv * W + w];
      if (t.kind == KIND_NONE) continue;
      ++busy;
      int64_t b = 0;
      if (t.kind != KIND_ATTN && t.kind != KIND_COMBINE) {
        const int64_t rows = (int64_t)t.nrows * (t.kind == KIND_GU ? 2 : 1);
        b = rows * t.kpad * p.wb;
        row_bytes = (int64_t)t.kpad * p.wb * (t.kind == KIND_GU ? 2 : 1);
      }
      tot += b;
      mx = std::max(mx, b);
    }
    p.wave_bytes[wv] = tot;
    p.wave_max_bytes[wv] = mx;
    p.wave_busy[wv] = busy;
    if (tot > 0) {
      // over the wave's busy workers: a wave placed on a subset on purpose (o_proj) is balanced there
      const double mean = (double)tot / busy;
      worst = std::max(worst, (double)mx / mean);
      (void)row_bytes;
    }
  }
  p.max_over_mean = worst;

  // ---- LDS sizing ----
  // vec: GEMV input vector, or the raw q/k/v of an attention tile
  int32_t vec = (int32_t)vec_floats(s);
  // GEMV tiles run in row blocks of at most MAX_BLOCK_ROWS rows (partials [rows][NCOMP] in LDS).
  // Multi-token steps (mt positions): mt input vectors, mt residual rows and mt partials per row, in
  // blocks of as many rows as the LDS holds beside the other areas and one staging batch (at least
  // MIN_MT_BLOCK_ROWS); attention tiles hold mt x T query rows and mt K/V rows.
  const int32_t mt = p.mt;
  const int64_t tables_bytes = round_up((int64_t)p.waves.size() * (int64_t)(sizeof(SegDesc) + sizeof(TileDesc) +
                                                                             sizeof(WaveDesc)) +
                                            (int64_t)s.n_layers * (int64_t)sizeof(LayerSmall), 256);
  int32_t brows = MAX_BLOCK_ROWS;
  if (mt > 1) {
    const int64_t other_floats = (int64_t)mt * vec + mt * round_up(s.Hpad, 64) + (p.q8 ? MAX_BLOCK_ROWS : 0) +
                                 SMALL_FLOATS;
    // rows that fit beside `batches` staging batches; where not even MIN_MT_BLOCK_ROWS fit beside one,
    // the plan stages nothing (the planner then finds no room for a batch) and the blocks take it all
    auto room = [&](int64_t batches) {
      return (LDS_LIMIT - other_floats * 4 - tables_bytes - batches * NCOMP * STREAM_BATCH * CHUNK_BYTES) /
             (4 * (int64_t)NCOMP * mt);
    };
    const int64_t r = room(1) >= MIN_MT_BLOCK_ROWS ? room(1) : room(0);
    brows = (int32_t)(std::max<int64_t>(MIN_MT_BLOCK_ROWS, std::min<int64_t>(MAX_BLOCK_ROWS, r)) & ~1);
  }
  int32_t part = 0;
  for (const WaveDesc& wd : p.waves) part = std::max(part, std::min(wd.max_rows, brows) * NCOMP * mt);
  // attention tile: q[G][hd], k[hd], v[hd], the compute-wave states [NCOMP][G][hd + 4] and the merged partial
  const int32_t ps = s.hd + 4;
  part = std::max(part, (int32_t)attn_lds_floats(p) + 2 * p.kv8_span);
  part = std::max(part, mt * p.S * ps);  // one head's splits (combine tile)
  if (p.combine_in_o && mt == 1) part = std::max(part, s.n_heads * p.S * ps);  // all splits (o_proj prologue)
  if (p.combine_in_o && mt > 1) part = std::max(part, (int32_t)(mt_merge_floats(p) - (int64_t)mt * vec));
  p.lds_vec_floats = (int32_t)round_up(vec, 64);
  p.lds_part_floats = (int32_t)round_up(part, 64);
  // sampled decoding: the token gather holds every worker's top_k (value, index) pairs in vec + part
  // (whole 16-byte units: two candidates each)
  const int64_t cand_floats = ((int64_t)p.W * p.top_k + 1) / 2 * 4;
  if (p.top_k > 0 && p.lds_vec_floats + p.lds_part_floats < cand_floats)
    p.lds_part_floats = (int32_t)round_up(cand_floats - p.lds_vec_floats, 64);
  p.lds_xres_floats = mt * (int32_t)round_up(s.Hpad, 64) + (p.q8 ? MAX_BLOCK_ROWS : 0);  // (INT8: then a block's scales)
  // schedule tables: per wave a SegDesc, this worker's TileDesc and the WaveDesc; per layer a LayerSmall
  p.lds_bytes = (mt * p.lds_vec_floats + p.lds_part_floats + p.lds_xres_floats + SMALL_FLOATS) * 4 + (int32_t)tables_bytes;
  if (p.lds_bytes > LDS_LIMIT) return fail(err, TILES_E_CONFIG, "LDS demand exceeds 160 KB");
  // staging areas for the next GEMV range's chunks, as many batches per compute wave as fit
  const int32_t stage_batch_bytes = NCOMP * STREAM_BATCH * CHUNK_BYTES;
  // (the area sits at LDS address 0 and must end below 64 KB: the load's LDS address is 16 bits)
  p.stage_batches = std::min<int32_t>({MAX_STAGE_BATCHES, (LDS_LIMIT - p.lds_bytes) / stage_batch_bytes,
                                       65536 / stage_batch_bytes});
  p.lds_stage_floats = p.stage_batches * stage_batch_bytes / 4;
  p.lds_bytes += p.lds_stage_floats * 4;
  // more than half the LDS of a CU: at most one workgroup per compute unit
  p.lds_bytes = std::max(p.lds_bytes, 84 * 1024);
  // a one-position plan needs a staging batch (see validate_plan): where the planner's own choice of
  // the o_proj prologue merge leaves no room for one (Qwen3-4B shape, INT8 weights), merge in a wave
  // of its own instead
  if (p.mt == 1 && p.stage_batches < 1 && p.combine_in_o && cfg.combine_mode == 0) {
    tiles_config_t own = cfg;
    own.combine_mode = 2;
    return build_plan(own, n_workers, p, err);
  }

  int rc = validate_plan(p, err);
  if (rc != TILES_OK) return rc;
  p.checksum = plan_checksum(p);
  return TILES_OK;
}

namespace {

// Rows of the source tensor a packing copy reads, and their width (BF16 values).
bool source_geometry(const Shape& s, int32_t tensor, int64_t& rows, int64_t& cols) {
  const int64_t q = (int64_t)s.n_heads * s.hd, kv = (int64_t)s.n_kv * s.hd;
  switch (tensor) {
    case SRC_EMBED: case SRC_LM_HEAD: rows = s.V; cols = s.H; return true;
    case SRC_FINAL_NORM: case SRC_ATTN_NORM: case SRC_MLP_NORM: rows = 1; cols = s.H; return true;
    case SRC_Q_NORM: case SRC_K_NORM: rows = 1; cols = s.hd; return true;
    case SRC_WQ: rows = q; cols = s.H; return true;
    case SRC_WK: case SRC_WV: rows = kv; cols = s.H; return true;
    case SRC_WO: rows = s.H; cols = q; return true;
    case SRC_WGATE: case SRC_WUP: rows = s.F; cols = s.H; return true;
    case SRC_WDOWN: rows = s.H; cols = s.F; return true;
  }
  return false;
}

// The source row packed at output row r of a GEMV tile kind (GU rows interleave gate and up).
void expected_source(const Shape& s, int32_t kind, int32_t layer, bool tied, int64_t out_row, int64_t r,
                     int32_t& tensor, int32_t& src_layer, int64_t& src_row) {
  const int64_t q = (int64_t)s.n_heads * s.hd, kv = (int64_t)s.n_kv * s.hd;
  src_layer = layer;
  switch (kind) {
    case KIND_QKV:
      if (out_row < q) { tensor = SRC_WQ; src_row = out_row; }
      else if (out_row < q + kv) { tensor = SRC_WK; src_row = out_row - q; }
      else { tensor = SRC_WV; src_row = out_row - q - kv; }
      return;
    case KIND_O: tensor = SRC_WO; src_row = out_row; return;
    case KIND_GU: tensor = (r & 1) ? SRC_WUP : SRC_WGATE; src_row = out_row; return;
    case KIND_DOWN: tensor = SRC_WDOWN; src_row = out_row; return;
    default: tensor = tied ? SRC_EMBED : SRC_LM_HEAD; src_layer = -1; src_row = out_row; return;
  }
}

}  // namespace

int validate_plan(const HostPlan& p, std::string& err) {
  const Shape& s = p.s;
  const int32_t W = p.W;
  const int nw = (int)p.waves.size();
  std::ostringstream os;
  if (W < 1 || (size_t)nw * W != p.tiles.size()) return fail(err, TILES_E_PLAN, "tile table size mismatch");

  // wave order: per layer QKV, ATTN, [COMBINE], O, GU, DOWN; then LM.  A step therefore starts with
  // layer 0's QKV wave, in which every worker gathers all LM-head partials of the previous step (the
  // token), and ends with the LM-head wave, in which every worker publishes its partial: this
  // all-to-all once per step is what lets one parity bit tell a buffer's generations apart.
  {
    std::vector<int32_t> want;
    for (int l = 0; l < s.n_layers; ++l) {
      want.push_back(KIND_QKV);
      want.push_back(KIND_ATTN);
      if (!p.combine_in_o) want.push_back(KIND_COMBINE);
      want.push_back(KIND_O);
      want.push_back(KIND_GU);
      want.push_back(KIND_DOWN);
    }
    want.push_back(KIND_LM);
    if ((int)want.size() != nw) return fail(err, TILES_E_PLAN, "unexpected number of waves");
    int per = p.combine_in_o ? 5 : 6;
    for (int wv = 0; wv < nw; ++wv) {
      if (p.waves[wv].kind != want[wv]) return fail(err, TILES_E_PLAN, "waves out of dependency order");
      const int32_t layer = wv == nw - 1 ? -1 : wv / per;
      if (p.waves[wv].layer != layer) return fail(err, TILES_E_PLAN, "wave layer mismatch");
    }
  }

  // tagged buffers: every wave but the LM head owns a 4-word aligned buffer, disjoint from the others
  {
    std::vector<std::pair<int64_t, int64_t>> bufs;
    for (int wv = 0; wv < nw; ++wv) {
      const int64_t n = wave_out_words(s, p.S, p.waves[wv].kind);
      const int32_t off = p.waves[wv].ll_off;
      if (n == 0) {
        if (off != -1) return fail(err, TILES_E_PLAN, "LM-head wave with a tagged buffer");
        continue;
      }
      if (off < 0 || off % 4 != 0 || n % 4 != 0 || off + n > p.ll_words)
        return fail(err, TILES_E_PLAN, "tagged buffer misaligned or out of bounds");
      bufs.push_back({off, off + n});
    }
    std::sort(bufs.begin(), bufs.end());
    for (size_t i = 1; i < bufs.size(); ++i)
      if (bufs[i].first < bufs[i - 1].second) return fail(err, TILES_E_PLAN, "tagged buffers overlap");
  }

  // per wave: tile ranges and coverage, the read and write sets, dataflow and hazards
  std::vector<std::pair<int64_t, int64_t>> packed_ranges;
  for (int wv = 0; wv < nw; ++wv) {
    const int32_t kind = p.waves[wv].kind;
    const int32_t layer = p.waves[wv].layer;
    std::vector<TileIO> io(W);
    int64_t covered = 0;
    std::vector<std::pair<int64_t, int64_t>> spans;  // GEMV tiles' (row0, nrows), in any worker order
    std::vector<int> seen;
    const int32_t in_buf = wv > 0 ? BUF_WAVE + wv - 1 : BUF_EMBED;
    const int32_t out_buf = BUF_WAVE + wv;
    for (int w = 0; w < W; ++w) {
      const TileDesc& t = p.tiles[(size_t)wv * W + w];
      TileIO& x = io[w];
      // What every worker does in this wave, tile or not (the kernel's gathers and the LM partial):
      // layer 0's QKV wave reads all LM partials of the previous step (the token) and an embedding
      // row; every other QKV wave and every gate/up wave reads the residual stream x from the wave
      // before (the o_proj and down epilogues add their rows to it); in the LM wave every worker
      // publishes its (max, index) partial.
      if (kind == KIND_QKV) {
        if (layer == 0) {
          x.reads.push_back({BUF_LMPART, 0, W});
          x.reads.push_back({BUF_EMBED, 0, s.H});
        } else {
          x.reads.push_back({in_buf, 0, s.H});
        }
      } else if (kind == KIND_GU) {
        x.reads.push_back({in_buf, 0, s.H});
      } else if (kind == KIND_LM) {
        x.writes.push_back({BUF_LMPART, w, w + 1});
      }
      if (t.kind == KIND_NONE) continue;
      if (t.kind != kind) return fail(err, TILES_E_PLAN, "tile kind differs from its wave");
      switch (kind) {
        case KIND_QKV: case KIND_O: case KIND_GU: case KIND_DOWN: case KIND_LM: {
          int64_t R = kind == KIND_QKV ? s.qkv_rows : kind == KIND_GU ? s.F : kind == KIND_LM ? s.V : s.H;
          int32_t kp = kind == KIND_O ? s.Qpad : kind == KIND_DOWN ? s.Fpad : s.Hpad;
          if (t.nrows < 1 || t.row0 < 0 || t.row0 + (int64_t)t.nrows > R)
            return fail(err, TILES_E_PLAN, "GEMV rows out of range");
          if (t.kpad != kp || kp % (CHUNK_BYTES / p.wb) != 0) return fail(err, TILES_E_PLAN, "bad GEMV width");
          spans.push_back({t.row0, t.nrows});
          covered += t.nrows;
          const int64_t bytes = tile_packed_bytes(p, t);
          if (t.woff % CHUNK_BYTES != 0 || t.woff < 0 || t.woff + bytes > p.packed_bytes)
            return fail(err, TILES_E_PLAN, "packed weights out of bounds or misaligned");
          packed_ranges.push_back({t.woff, t.woff + bytes});
          const int64_t lo = t.row0, hi = t.row0 + t.nrows;
          if (kind == KIND_O) {
            x.reads.push_back({in_buf, 0, wave_out_words(s, p.S, p.waves[wv - 1].kind)});
            x.writes.push_back({out_buf, lo, hi});
          } else if (kind == KIND_DOWN) {
            x.reads.push_back({in_buf, 0, s.F});
            x.writes.push_back({out_buf, lo, hi});
          } else if (kind == KIND_LM) {
            x.reads.push_back({in_buf, 0, s.H});
            x.writes.push_back({BUF_LOGITS, lo, hi});
          } else {
            x.writes.push_back({out_buf, lo, hi});  // QKV, GU: inputs listed above
          }
          break;
        }
        case KIND_ATTN: {
          const int32_t hs = p.T > 0 ? (t.aux0 - t.row0 * s.G) / p.T : -1;
          if (p.T < 1 || t.row0 < 0 || t.row0 >= s.n_kv || t.nrows < 0 || t.nrows >= p.S || t.aux0 < t.row0 * s.G ||
              (t.aux0 - t.row0 * s.G) % p.T != 0 || hs >= s.G / p.T)
            return fail(err, TILES_E_PLAN, "attention tile out of range");
          seen.push_back((t.row0 * (s.G / p.T) + hs) * p.S + t.nrows);
          x.reads.push_back({in_buf, 0, s.qkv_rows});
          // cached positions of this KV head (all positions before the current one)
          const int64_t kvbase = ((int64_t)layer * s.n_kv + t.row0) * s.max_positions;
          x.reads.push_back({BUF_KV, kvbase, kvbase + s.max_positions - 1});
          // The current position is written by exactly one split (the one holding L-1, checked
          // for every L below) of the KV head's first query-head group; the model gives that write
          // to split 0 and a slot past every read.
          if (t.nrows == 0 && hs == 0) x.writes.push_back({BUF_KV, kvbase + s.max_positions - 1, kvbase + s.max_positions});
          for (int g2 = 0; g2 < p.T; ++g2) {  // one (hd + 4)-word record per query head
            const int64_t h = (int64_t)t.aux0 + g2, rec = (h * p.S + t.nrows) * (s.hd + 4);
            x.writes.push_back({out_buf, rec, rec + s.hd + 4});
          }
          break;
        }
        case KIND_COMBINE: {
          if (t.row0 < 0 || t.row0 >= s.n_heads) return fail(err, TILES_E_PLAN, "combine tile out of range");
          seen.push_back(t.row0);
          x.reads.push_back({in_buf, (int64_t)t.row0 * p.S * (s.hd + 4), (int64_t)(t.row0 + 1) * p.S * (s.hd + 4)});
          x.writes.push_back({out_buf, (int64_t)t.row0 * s.hd, (int64_t)(t.row0 + 1) * s.hd});
          break;
        }
        default:
          return fail(err, TILES_E_PLAN, "unknown tile kind");
      }
    }
    if (kind == KIND_ATTN || kind == KIND_COMBINE) {
      std::sort(seen.begin(), seen.end());
      const int want_n = kind == KIND_ATTN ? s.n_kv * (s.G / p.T) * p.S : s.n_heads;
      if ((int)seen.size() != want_n) return fail(err, TILES_E_PLAN, "attention/combine tiles do not cover every head");
      for (int i = 0; i < want_n; ++i)
        if (seen[i] != i) return fail(err, TILES_E_PLAN, "attention/combine tile duplicated or missing");
    } else {
      int64_t R = kind == KIND_QKV ? s.qkv_rows : kind == KIND_GU ? s.F : kind == KIND_LM ? s.V : s.H;
      std::sort(spans.begin(), spans.end());
      int64_t expect_next = 0;
      for (const auto& sp : spans) {
        if (sp.first != expect_next) return fail(err, TILES_E_PLAN, "GEMV rows not covered exactly once");
        expect_next = sp.first + sp.second;
      }
      if (covered != R || expect_next != R) return fail(err, TILES_E_PLAN, "GEMV rows not covered exactly once");
    }
    // Dataflow: every tagged value a worker reads was published by the wave right before this one
    // in the same step (the kernel's gathers poll that buffer and no other), inside that buffer; the
    // LM partials of the previous step are read only at the start of a step.
    for (int w = 0; w < W; ++w)
      for (const Interval& r : io[w].reads) {
        if (r.buf >= BUF_WAVE) {
          const int j = r.buf - BUF_WAVE;
          if (j != wv - 1) return fail(err, TILES_E_PLAN, "a tile reads a tagged buffer other than the previous wave's");
          if (r.lo < 0 || r.hi > wave_out_words(s, p.S, p.waves[j].kind))
            return fail(err, TILES_E_PLAN, "a read falls outside its producer's buffer");
        } else if (r.buf == BUF_LMPART && wv != 0) {
          return fail(err, TILES_E_PLAN, "LM-head partials read outside the first wave of a step");
        }
      }
    // Every word of this wave's output buffer (the LM partials: every worker's slot) is written by
    // exactly one tile per step: a word nobody writes would leave its consumers polling forever, a
    // word written twice would race.
    {
      const int32_t target = kind == KIND_LM ? BUF_LMPART : out_buf;
      const int64_t n = kind == KIND_LM ? W : wave_out_words(s, p.S, kind);
      std::vector<std::pair<int64_t, int64_t>> ws;
      for (int w = 0; w < W; ++w)
        for (const Interval& x : io[w].writes) {
          if (x.buf == target) ws.push_back({x.lo, x.hi});
          else if (x.buf >= BUF_WAVE) return fail(err, TILES_E_PLAN, "a tile writes another wave's buffer");
        }
      std::sort(ws.begin(), ws.end());
      int64_t next = 0;
      for (const auto& iv : ws) {
        if (iv.first != next) {
          os << "output buffer of wave " << wv << " not written exactly once per step";
          return fail(err, TILES_E_PLAN, os.str());
        }
        next = iv.second;
      }
      if (next != n) {
        os << "output buffer of wave " << wv << " not written exactly once per step";
        return fail(err, TILES_E_PLAN, os.str());
      }
    }
    // hazards: a write of one worker may not meet a read or write of another worker in the same wave
    for (int a = 0; a < W; ++a)
      for (const Interval& wr : io[a].writes)
        for (int b = 0; b < W; ++b) {
          if (b == a) continue;
          for (const Interval& o : io[b].reads)
            if (o.buf == wr.buf && o.lo < wr.hi && wr.lo < o.hi) {
              os << "read/write hazard in wave " << wv << " between workers " << a << " and " << b;
              return fail(err, TILES_E_PLAN, os.str());
            }
          for (const Interval& o : io[b].writes)
            if (o.buf == wr.buf && o.lo < wr.hi && wr.lo < o.hi) {
              os << "write/write hazard in wave " << wv << " between workers " << a << " and " << b;
              return fail(err, TILES_E_PLAN, os.str());
            }
        }
  }

  // byte balance: max/mean over the wave's busy workers within one row of a perfect split
  for (int wv = 0; wv < nw; ++wv) {
    int64_t tot = 0, mx = 0, row_bytes = 0;
    int busy = 0;
    for (int w = 0; w < W; ++w) {
      const TileDesc& t = p.tiles[(size_t)wv * W + w];
      if (t.kind == KIND_NONE || t.kind == KIND_ATTN || t.kind == KIND_COMBINE) continue;
      const int64_t b = (int64_t)t.nrows * (t.kind == KIND_GU ? 2 : 1) * t.kpad * p.wb;
      ++busy;
      tot += b;
      mx = std::max(mx, b);
      row_bytes = std::max<int64_t>(row_bytes, (int64_t)t.kpad * p.wb * (t.kind == KIND_GU ? 2 : 1));
    }
    if (busy == 0) continue;
    if ((double)mx > (double)tot / busy + row_bytes + 0.5) {
      os << "worker bytes unbalanced in wave " << wv;
      return fail(err, TILES_E_PLAN, os.str());
    }
  }

  // packed ranges of different tiles never overlap
  std::sort(packed_ranges.begin(), packed_ranges.end());
  for (size_t i = 1; i < packed_ranges.size(); ++i)
    if (packed_ranges[i].first < packed_ranges[i - 1].second) return fail(err, TILES_E_PLAN, "packed tiles overlap");

  // Packing round trip: every row of every source tensor is copied exactly once, with its full
  // width, inside the packed buffer, and every GEMV tile row finds there the source row it computes
  // with (QKV rows from Wq, Wk, Wv in turn; gate/up rows alternating; LM-head rows from the embedding
  // when tied), so that a packing mistake cannot go unnoticed until the numbers come out wrong.
  {
    struct Src { int32_t tensor, layer; int64_t row, cols, scale; };  // scale: its offset (quantized copy) or -1
    std::unordered_map<int64_t, Src> at;  // destination byte offset of a packed row -> its source
    at.reserve(1 << 16);
    // source rows copied, per (tensor, layer, form): a tied INT8 head copies the embedding twice, as
    // INT8 codes for the head and as BF16 rows for the lookup
    std::map<std::tuple<int32_t, int32_t, int32_t>, std::vector<std::pair<int64_t, int64_t>>> rows_of;
    for (const CopySeg& c : p.copies) {
      int64_t R = 0, C = 0;
      const bool quant = c.scale_off >= 0;
      const int64_t eb = quant ? 1 : 2;  // bytes per packed value of this copy
      const bool gain = c.tensor == SRC_ATTN_NORM || c.tensor == SRC_MLP_NORM || c.tensor == SRC_Q_NORM ||
                        c.tensor == SRC_K_NORM || c.tensor == SRC_FINAL_NORM;
      if (!source_geometry(s, c.tensor, R, C) || c.cols != C || c.nrows < 1 || c.src_row < 0 || c.src_row + c.nrows > R ||
          c.dst_off < 0 || c.dst_pitch < c.cols * eb || c.dst_off + (c.nrows - 1) * c.dst_pitch + c.cols * eb > p.packed_bytes ||
          (quant && (!p.q8 || gain || c.scale_off + (c.nrows - 1) * c.scale_pitch + 4 > p.packed_bytes)))
        return fail(err, TILES_E_PLAN, "packing copy out of range");
      rows_of[std::make_tuple(c.tensor, c.layer, quant ? 1 : 0)].push_back({c.src_row, c.src_row + c.nrows});
      for (int64_t r = 0; r < c.nrows; ++r)
        if (!at.emplace(c.dst_off + r * c.dst_pitch,
                        Src{c.tensor, c.layer, c.src_row + r, c.cols, quant ? c.scale_off + r * c.scale_pitch : -1})
                 .second)
          return fail(err, TILES_E_PLAN, "two packing copies write the same packed row");
    }
    for (auto& kvp : rows_of) {
      int64_t R = 0, C = 0;
      source_geometry(s, std::get<0>(kvp.first), R, C);
      auto& v = kvp.second;
      std::sort(v.begin(), v.end());
      int64_t next = 0;
      for (const auto& iv : v) {
        if (iv.first != next) return fail(err, TILES_E_PLAN, "source rows not packed exactly once");
        next = iv.second;
      }
      if (next != R) return fail(err, TILES_E_PLAN, "source rows not packed exactly once");
    }
    // every source tensor the model has is packed
    const size_t per_layer = s.qk_norm ? 11 : 9;
    const size_t want = (size_t)s.n_layers * per_layer + 2 /*final norm, embedding or LM head*/ +
                        (s.tied && !p.q8 ? 0 : 1) /*a lookup table of its own*/;
    if (rows_of.size() != want) return fail(err, TILES_E_PLAN, "source rows not packed exactly once");
    for (int wv = 0; wv < nw; ++wv) {
      const int32_t kind = p.waves[wv].kind;
      if (kind == KIND_ATTN || kind == KIND_COMBINE) continue;
      for (int w = 0; w < W; ++w) {
        const TileDesc& t = p.tiles[(size_t)wv * W + w];
        if (t.kind == KIND_NONE) continue;
        const int64_t nr = (int64_t)t.nrows * (kind == KIND_GU ? 2 : 1);
        for (int64_t r = 0; r < nr; ++r) {
          int32_t tensor, layer;
          int64_t srow;
          expected_source(s, kind, p.waves[wv].layer, s.tied, t.row0 + (kind == KIND_GU ? r / 2 : r), r, tensor, layer, srow);
          auto it = at.find(t.woff + r * t.kpad * p.wb);
          const int64_t want_scale = p.q8 ? t.woff + nr * t.kpad + r * 4 : -1;  // INT8: scales follow the rows
          if (it == at.end() || it->second.tensor != tensor || it->second.layer != layer || it->second.row != srow ||
              it->second.cols > (int64_t)t.kpad || it->second.scale != want_scale) {
            os << "packed row " << r << " of worker " << w << "'s tile in wave " << wv << " is not its source row";
            return fail(err, TILES_E_PLAN, os.str());
          }
        }
      }
    }
    // the embedding rows the first wave reads, and the gains, are where the plan says
    auto it = at.find(p.embed_off + (int64_t)(s.V - 1) * p.embed_stride);
    if (it == at.end() || it->second.tensor != SRC_EMBED || it->second.row != s.V - 1 || it->second.scale != -1)
      return fail(err, TILES_E_PLAN, "embedding rows not where the plan reads them");
    it = at.find(p.final_norm_off);
    if (it == at.end() || it->second.tensor != SRC_FINAL_NORM) return fail(err, TILES_E_PLAN, "final-norm gain misplaced");
    for (int l = 0; l < s.n_layers; ++l) {
      const LayerSmall& g = p.small[l];
      auto a1 = at.find(g.attn_norm), m1 = at.find(g.mlp_norm);
      if (a1 == at.end() || a1->second.tensor != SRC_ATTN_NORM || a1->second.layer != l || m1 == at.end() ||
          m1->second.tensor != SRC_MLP_NORM || m1->second.layer != l)
        return fail(err, TILES_E_PLAN, "norm gains misplaced");
      if (s.qk_norm) {
        auto q1 = at.find(g.q_norm), k1 = at.find(g.k_norm);
        if (q1 == at.end() || q1->second.tensor != SRC_Q_NORM || q1->second.layer != l || k1 == at.end() ||
            k1->second.tensor != SRC_K_NORM || k1->second.layer != l)
          return fail(err, TILES_E_PLAN, "norm gains misplaced");
      }
    }
  }

  // split-KV: for every attended length the splits partition [0, L) and exactly one holds L-1
  for (int64_t L = 1; L <= s.max_positions; ++L) {
    int64_t next = 0;
    int holders = 0;
    for (int sp = 0; sp < p.S; ++sp) {
      int64_t lo, hi;
      split_range(L, p.S, sp, lo, hi);
      if (hi > lo) {
        if (lo != next) return fail(err, TILES_E_PLAN, "KV splits do not partition the positions");
        next = hi;
        if (lo <= L - 1 && L - 1 < hi) ++holders;
      }
    }
    if (next != L || holders != 1) return fail(err, TILES_E_PLAN, "KV splits do not partition the positions");
    // the KV write happens in the split holding L-1; the kernel makes that split write
  }

  // multi-token steps
  if (p.mt < 1 || p.mt > MAX_STEP_TOKENS) return fail(err, TILES_E_PLAN, "tokens per step must be 1 .. 4");
  if (p.mt > 1 && (p.top_k > 0 || p.T * p.mt > MAX_GROUP))
    return fail(err, TILES_E_PLAN, "multi-token plan with an unsupported option");
  if (p.mt > 1 && p.combine_in_o && (int64_t)p.mt * p.lds_vec_floats + p.lds_part_floats < mt_merge_floats(p))
    return fail(err, TILES_E_PLAN, "LDS too small for the split merge of every position");
  // LDS capacity for every wave's staging
  if (p.lds_part_floats / (NCOMP * p.mt) < 2) return fail(err, TILES_E_PLAN, "LDS partial area too small");
  // the kernel's GEMV row blocks (see the worker); INT8 scales and sampled candidates cover MAX_BLOCK_ROWS
  // rows of a block
  {
    const int32_t br = p.mt > 1 ? std::min((p.lds_part_floats / (NCOMP * p.mt)) & ~1, MAX_BLOCK_ROWS)
                                : (p.lds_part_floats / NCOMP) & ~1;
    if ((p.q8 || p.top_k > 0) && br > MAX_BLOCK_ROWS)
      for (const TileDesc& t : p.tiles)
        if ((t.kind == KIND_QKV || t.kind == KIND_O || t.kind == KIND_GU || t.kind == KIND_DOWN || t.kind == KIND_LM) &&
            t.nrows * (t.kind == KIND_GU ? 2 : 1) > MAX_BLOCK_ROWS)
          return fail(err, TILES_E_PLAN, "a GEMV tile of more than 640 rows in an INT8 or sampling plan");
  }
  if (p.stage_batches < 0 || p.stage_batches > MAX_STAGE_BATCHES ||
      p.lds_stage_floats != p.stage_batches * NCOMP * STREAM_BATCH * CHUNK_BYTES / 4 || p.lds_bytes > LDS_LIMIT ||
      p.lds_stage_floats * 4 > 65536)
    return fail(err, TILES_E_PLAN, "bad LDS staging area");
  // a one-position step stages one batch of a compute wavefront's own range whatever stage_batches says
  if (p.mt == 1 && p.stage_batches < 1) return fail(err, TILES_E_PLAN, "no LDS room for a staging batch");
  if (p.lds_vec_floats < std::max({s.Hpad, s.Qpad, s.Fpad})) return fail(err, TILES_E_PLAN, "LDS vector area too small");
  if (p.combine_in_o && p.mt == 1 && (int64_t)s.n_heads * p.S * (s.hd + 4) > p.lds_part_floats)
    return fail(err, TILES_E_PLAN, "LDS too small for the split merge");
  if ((int64_t)p.mt * p.S * (s.hd + 4) > p.lds_part_floats) return fail(err, TILES_E_PLAN, "LDS too small for a combine tile");
  if (attn_lds_floats(p) > p.lds_part_floats) return fail(err, TILES_E_PLAN, "LDS too small for an attention tile");
  if (p.lds_xres_floats < p.mt * round_up(s.Hpad, 64) + (p.q8 ? MAX_BLOCK_ROWS : 0))
    return fail(err, TILES_E_PLAN, "LDS residual area too small");
  if (p.kv8) {
    const int64_t np = (s.max_positions + p.S - 1) / p.S;
    if (np > p.kv8_span || p.kv8_span > MAX_SPLIT_POSITIONS_KV8 || p.kv8_span % 64 != 0)
      return fail(err, TILES_E_PLAN, "INT8 KV: a split longer than its LDS scale area, or than 4096 positions");
    if (p.lds_part_floats < attn_lds_floats(p) + 2 * (int64_t)p.kv8_span)
      return fail(err, TILES_E_PLAN, "LDS too small for an INT8 KV split's scales");
  }
  if (p.top_k < 0 || p.top_k > MAX_TOP_K || p.top_k > s.V || (p.top_k > 0 && p.W > 256))
    return fail(err, TILES_E_PLAN, "top_k out of range (1..32, <= vocab, at most 256 workers)");
  if (p.top_k > 0 && (int64_t)p.lds_vec_floats + p.lds_part_floats < ((int64_t)p.W * p.top_k + 1) / 2 * 4)
    return fail(err, TILES_E_PLAN, "LDS too small for the sampled token gather (W x top_k pairs)");
  return TILES_OK;
}

int debug_mutate_plan(HostPlan& p, int32_t m, std::string& err) {
  const int32_t W = p.W;
  const int nw = (int)p.waves.size();
  auto tile = [&](int wv, int w) -> TileDesc& { return p.tiles[(size_t)wv * W + w]; };
  auto first_wave = [&](int32_t kind) {
    for (int wv = 0; wv < nw; ++wv)
      if (p.waves[wv].kind == kind) return wv;
    return -1;
  };
  // two workers of a GEMV wave whose tiles are adjacent in rows (a's rows end where b's begin)
  auto adjacent = [&](int wv, int& a, int& b, int min_b_rows) {
    for (a = 0; a < W; ++a) {
      if (tile(wv, a).kind == KIND_NONE) continue;
      for (b = 0; b < W; ++b)
        if (b != a && tile(wv, b).kind != KIND_NONE && tile(wv, b).row0 == tile(wv, a).row0 + tile(wv, a).nrows &&
            tile(wv, b).nrows > min_b_rows)
          return true;
    }
    return false;
  };
  int a = 0, b = 0;
  switch (m) {
    case DBG_NONE:
      return TILES_OK;
    case DBG_ROW_OVERLAP: {
      const int wv = first_wave(KIND_GU);
      if (!adjacent(wv, a, b, 0)) break;
      tile(wv, a).nrows += 1;
      return TILES_OK;
    }
    case DBG_ROW_GAP: {
      const int wv = first_wave(KIND_GU);
      for (a = 0; a < W; ++a)
        if (tile(wv, a).kind != KIND_NONE && tile(wv, a).nrows >= 2) {
          tile(wv, a).nrows -= 1;
          return TILES_OK;
        }
      break;
    }
    case DBG_ATTN_DUPLICATE: case DBG_ATTN_MISSING: {
      const int wv = first_wave(KIND_ATTN);
      for (a = 0; a < W; ++a)
        if (tile(wv, a).kind == KIND_ATTN) break;
      if (a == W) break;
      if (m == DBG_ATTN_MISSING) {
        std::memset(&tile(wv, a), 0, sizeof(TileDesc));
        return TILES_OK;
      }
      for (b = 0; b < W; ++b)
        if (tile(wv, b).kind == KIND_NONE) {
          tile(wv, b) = tile(wv, a);
          return TILES_OK;
        }
      break;
    }
    case DBG_SPLIT_OUT_OF_RANGE: {
      const int wv = first_wave(KIND_ATTN);
      for (a = 0; a < W; ++a)
        if (tile(wv, a).kind == KIND_ATTN) {
          tile(wv, a).nrows = p.S;
          return TILES_OK;
        }
      break;
    }
    case DBG_TAGGED_OVERLAP:
      if (nw < 3) break;
      p.waves[1].ll_off = p.waves[0].ll_off;
      return TILES_OK;
    case DBG_TAGGED_OUT_OF_BOUNDS:
      p.waves[0].ll_off = (int32_t)p.ll_words;
      return TILES_OK;
    case DBG_UNBALANCED: {
      // worker a takes the first two rows of worker b: coverage and packing stay exact, the bytes do not
      const int wv = first_wave(KIND_DOWN);
      if (!adjacent(wv, a, b, 2)) break;
      const int64_t row_bytes = (int64_t)tile(wv, b).kpad * p.wb;
      tile(wv, a).nrows += 2;
      tile(wv, b).row0 += 2;
      tile(wv, b).nrows -= 2;
      tile(wv, b).woff += 2 * row_bytes;
      return TILES_OK;
    }
    case DBG_WAVE_ORDER:
      if (nw < 3) break;
      std::swap(p.waves[1], p.waves[2]);
      return TILES_OK;
    case DBG_LM_NOT_LAST:
      p.waves.back().kind = KIND_DOWN;
      return TILES_OK;
    case DBG_PACKED_OVERLAP: {
      const int wv = first_wave(KIND_QKV);
      if (!adjacent(wv, a, b, 0)) break;
      tile(wv, b).woff = tile(wv, a).woff;
      return TILES_OK;
    }
    case DBG_PACKED_SWAPPED: {
      // two tiles of the LM-head wave with equal row counts exchange their packed rows
      const int wv = nw - 1;
      for (a = 0; a < W; ++a)
        for (b = a + 1; b < W; ++b)
          if (tile(wv, a).kind == KIND_LM && tile(wv, b).kind == KIND_LM && tile(wv, a).nrows == tile(wv, b).nrows) {
            std::swap(tile(wv, a).woff, tile(wv, b).woff);
            return TILES_OK;
          }
      break;
    }
    case DBG_COPY_DROPPED:
      if (p.copies.empty()) break;
      p.copies.erase(p.copies.begin() + (long)(p.copies.size() / 2));
      return TILES_OK;
    case DBG_GAIN_MISPLACED:
      if (p.small.size() < 2) break;
      p.small[1].mlp_norm = p.small[0].mlp_norm;
      return TILES_OK;
    case DBG_STAGING:
      p.stage_batches = MAX_STAGE_BATCHES + 1;
      return TILES_OK;
    default:
      return fail(err, TILES_E_ARG, "unknown plan mutation");
  }
  return fail(err, TILES_E_ARG, "plan mutation not applicable to this plan");
}

}  // namespace tiles
