// C-ABI runtime: plan creation (device probe, planning, validation, weight packing,
// uploads), cooperative launches of the persistent worker, status and debug read-back.
//
// Follows "Tiles: Scheduling LLM Decoding as a Graph of Tiles", "What the code contains"
// (the split between an offline plan builder and a runtime that checks a plan before each
// use and runs many tokens per cooperative launch).  Here the checks are: before every
// launch the host re-hashes its copy of the schedule and compares device and CU count; in
// every launch each worker re-hashes the schedule it actually loaded from device memory and
// compares it, and the build id stored with the plan, against what the plan recorded and
// against its own compiled-in build id.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstddef>
#include <mutex>
#include <thread>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/tiles.h"
#include "plan_types.h"
#include "planner.h"

#ifndef TILES_BUILD_ID
#define TILES_BUILD_ID 0x0ull
#endif

namespace tiles {
const void* worker_kernel(int head_dim, int group, bool short_watchdog, bool q8, bool sampled, bool kv8, int mt);
hipError_t launch_kv_convert(const uint16_t* k, const uint16_t* v, int64_t cap, int64_t length, int hd, int64_t nheads,
                             int8_t* codes, float* ks, float* vs, float* sigma, hipStream_t stream);
hipError_t launch_pack(const PackSeg* segs, int nseg, uint8_t* dst, hipStream_t stream);
hipError_t launch_fill(uint32_t* p, int64_t n, uint32_t v, hipStream_t stream);
hipError_t launch_fill_blocks(uint16_t* p, int nblk, int64_t stride, int64_t count, uint16_t v, hipStream_t stream);
hipError_t launch_stream_read(const uint8_t* p, int64_t bytes, int n_groups, uint32_t* sink, hipStream_t stream);
hipError_t launch_edge_latency(uint32_t* words, int peer, int iters, uint32_t spin_limit, uint64_t* out,
                               hipStream_t stream);
hipError_t noalloc_scratch(int device, uint32_t** out);
}

using namespace tiles;

namespace {

thread_local std::string g_err;

int set_err(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIP_TRY(expr)                                                                    \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess) {                                                              \
      return set_err(TILES_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_));   \
    }                                                                                    \
  } while (0)

constexpr int MAX_STEPS = 64;

}  // namespace

struct tiles_plan {
  HostPlan hp;
  tiles_config_t cfg;
  int device = -1;
  int cu_count = 0;
  char arch[64] = {0};
  char pci[32] = {0};
  uint64_t build_id = TILES_BUILD_ID;
  const void* kernel = nullptr;
  int occupancy = 0;
  uint32_t spin_limit = DEFAULT_SPIN_LIMIT;  // polling rounds before a wait gives up (watchdog)
  const void* kernel_wd = nullptr;            // test instantiation checking the watchdog every round
  hipStream_t stream = nullptr;
  // device memory
  uint8_t* packed = nullptr;
  TileDesc* d_tiles = nullptr;
  WaveDesc* d_waves = nullptr;
  LayerSmall* d_small = nullptr;
  float* d_rope = nullptr;
  uint8_t* scratch = nullptr;
  size_t scratch_bytes = 0;
  uint32_t* ll = nullptr;      // tagged-data buffers; lmpart follows them in the same fill range
  uint32_t* lmpart = nullptr;
  int64_t fill_words = 0;      // ll .. lmpart end, refilled before every launch
  uint32_t* sync = nullptr;
  size_t sync_bytes = 0;
  int32_t* d_forced = nullptr;        // [MAX_STEPS]: the given tokens of a verify step
  uint64_t* d_table_check = nullptr;  // [W] per-worker schedule hashes, then the build id
  uint32_t* last_sync = nullptr;      // status words of the last launch (plan-owned or the static scratch)
  float* dbg_hidden = nullptr;
  uint64_t* trace = nullptr;
  int last_steps = 0;
};

namespace {

int probe_device(tiles_plan* p) {
  HIP_TRY(hipGetDevice(&p->device));
  hipDeviceProp_t pr;
  HIP_TRY(hipGetDeviceProperties(&pr, p->device));
  std::snprintf(p->arch, sizeof(p->arch), "%s", pr.gcnArchName);
  std::snprintf(p->pci, sizeof(p->pci), "%04x:%02x:%02x", pr.pciDomainID, pr.pciBusID, pr.pciDeviceID);
  p->cu_count = pr.multiProcessorCount;
  if (std::strncmp(pr.gcnArchName, "gfx950", 6) != 0)
    return set_err(TILES_E_DEVICE, std::string("worker kernel is built for gfx950, device is ") + pr.gcnArchName);
  if (!pr.cooperativeLaunch) return set_err(TILES_E_DEVICE, "device does not support cooperative launches");
  return TILES_OK;
}

const void* src_ptr(const tiles_weights_t* w, int32_t tensor, int32_t layer) {
  const tiles_layer_weights_t* L = layer >= 0 ? &w->layers[layer] : nullptr;
  switch (tensor) {
    case SRC_EMBED: return w->embed;
    case SRC_FINAL_NORM: return w->final_norm;
    case SRC_LM_HEAD: return w->lm_head;
    case SRC_ATTN_NORM: return L->attn_norm;
    case SRC_WQ: return L->wq;
    case SRC_WK: return L->wk;
    case SRC_WV: return L->wv;
    case SRC_Q_NORM: return L->q_norm;
    case SRC_K_NORM: return L->k_norm;
    case SRC_WO: return L->wo;
    case SRC_MLP_NORM: return L->mlp_norm;
    case SRC_WGATE: return L->w_gate;
    case SRC_WUP: return L->w_up;
    case SRC_WDOWN: return L->w_down;
  }
  return nullptr;
}

void release(tiles_plan* p) {
  if (!p) return;
  if (p->stream || p->device >= 0) (void)hipStreamSynchronize(p->stream);
  void* bufs[] = {p->packed, p->d_tiles, p->d_waves, p->d_small, p->d_rope, p->scratch, p->dbg_hidden, p->trace,
                  p->d_table_check};
  for (void* b : bufs)
    if (b) (void)hipFree(b);
  delete p;
}

// Weight-only INT8 plans: the packed image (INT8 codes and scales of every linear layer, BF16 gains
// and embedding rows) is built on the host -- device-resident sources are read back one copy
// segment at a time -- by a few threads over disjoint segments, and uploaded in one copy.
int pack_int8_on_host(tiles_plan* p, const tiles_weights_t* w) {
  const HostPlan& hp = p->hp;
  std::vector<uint8_t> img((size_t)hp.packed_bytes, 0);
  std::atomic<size_t> next{0};
  std::atomic<int> failed{0};
  std::string first_err;
  std::mutex err_mu;
  int dev = p->device;
  auto work = [&]() {
    if (w->on_device && hipSetDevice(dev) != hipSuccess) {
      failed = 1;
      return;
    }
    std::vector<uint16_t> tmp;
    for (size_t i = next++; i < hp.copies.size() && !failed; i = next++) {
      const CopySeg& c = hp.copies[i];
      const uint8_t* src = static_cast<const uint8_t*>(src_ptr(w, c.tensor, c.layer));
      if (!src) {
        std::lock_guard<std::mutex> g(err_mu);
        first_err = "missing weight tensor for packing";
        failed = 1;
        return;
      }
      src += c.src_row * c.cols * 2;
      const uint16_t* rows = reinterpret_cast<const uint16_t*>(src);
      if (w->on_device) {
        tmp.resize((size_t)(c.nrows * c.cols));
        const hipError_t e = hipMemcpy(tmp.data(), src, (size_t)(c.nrows * c.cols * 2), hipMemcpyDeviceToHost);
        if (e != hipSuccess) {
          std::lock_guard<std::mutex> g(err_mu);
          first_err = std::string("reading back weights: ") + hipGetErrorString(e);
          failed = 1;
          return;
        }
        rows = tmp.data();
      }
      if (c.scale_off >= 0) {
        quantize_rows_int8(rows, c.cols, c.nrows, c.cols, reinterpret_cast<int8_t*>(img.data() + c.dst_off), c.dst_pitch,
                           reinterpret_cast<float*>(img.data() + c.scale_off), c.scale_pitch / 4);
      } else {
        for (int64_t r = 0; r < c.nrows; ++r)
          std::memcpy(img.data() + c.dst_off + r * c.dst_pitch, rows + r * c.cols, (size_t)(c.cols * 2));
      }
    }
  };
  const unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  std::vector<std::thread> threads;
  for (unsigned t = 0; t < nt; ++t) threads.emplace_back(work);
  for (auto& t : threads) t.join();
  if (failed) return set_err(first_err.empty() ? TILES_E_HIP : TILES_E_ARG, first_err.empty() ? "packing failed" : first_err);
  HIP_TRY(hipSetDevice(dev));
  HIP_TRY(hipMemcpy(p->packed, img.data(), (size_t)hp.packed_bytes, hipMemcpyHostToDevice));
  return TILES_OK;
}

int create_impl(const tiles_config_t* cfg, const tiles_weights_t* w, tiles_plan** out) {
  *out = nullptr;
  if (!cfg || !w) return set_err(TILES_E_ARG, "null config or weights");
  if (!w->embed || !w->final_norm || !w->layers) return set_err(TILES_E_ARG, "missing weight tensor");
  if (!cfg->tie_embeddings && !w->lm_head) return set_err(TILES_E_ARG, "untied model without lm_head");
  for (int l = 0; l < cfg->n_layers; ++l) {
    const tiles_layer_weights_t& L = w->layers[l];
    if (!L.attn_norm || !L.wq || !L.wk || !L.wv || !L.wo || !L.mlp_norm || !L.w_gate || !L.w_up || !L.w_down)
      return set_err(TILES_E_ARG, "missing layer weight tensor");
    if (cfg->qk_norm && (!L.q_norm || !L.k_norm)) return set_err(TILES_E_ARG, "missing q_norm/k_norm");
  }
  tiles_plan* p = new tiles_plan();
  p->cfg = *cfg;
  p->stream = static_cast<hipStream_t>(cfg->stream);
  int rc = probe_device(p);
  if (rc != TILES_OK) {
    release(p);
    return rc;
  }
  if (cfg->n_workers != 0 && cfg->n_workers != p->cu_count) {
    release(p);
    return set_err(TILES_E_DEVICE, "n_workers must equal the CU count on the GPU");
  }
  std::string err;
  rc = build_plan(*cfg, p->cu_count, p->hp, err);
  if (rc != TILES_OK) {
    release(p);
    return set_err(rc, err);
  }
  const HostPlan& hp = p->hp;
  // occupancy probe of the worker binary
  p->kernel = worker_kernel(hp.s.hd, hp.T, false, hp.q8 != 0, hp.top_k > 0, hp.kv8 != 0, hp.mt);
  if (!p->kernel) {
    release(p);
    return set_err(TILES_E_CONFIG, "no worker instantiation for this head_dim / group size");
  }
  hipError_t e = hipFuncSetAttribute(p->kernel, hipFuncAttributeMaxDynamicSharedMemorySize, hp.lds_bytes);
  if (e != hipSuccess) {
    release(p);
    return set_err(TILES_E_HIP, std::string("hipFuncSetAttribute: ") + hipGetErrorString(e));
  }
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&p->occupancy, p->kernel, BLOCK_THREADS, hp.lds_bytes);
  if (e != hipSuccess || p->occupancy < 1) {
    release(p);
    return set_err(TILES_E_DEVICE, "worker kernel cannot be resident (occupancy < 1)");
  }

#define TRY(expr)                                                                    \
  do {                                                                               \
    hipError_t e_ = (expr);                                                          \
    if (e_ != hipSuccess) {                                                          \
      std::string m = std::string(#expr) + ": " + hipGetErrorString(e_);             \
      release(p);                                                                    \
      return set_err(TILES_E_HIP, m);                                                \
    }                                                                                \
  } while (0)

  // packed weights
  TRY(hipMalloc(&p->packed, hp.packed_bytes));
  TRY(hipMemsetAsync(p->packed, 0, hp.packed_bytes, p->stream));
  if (hp.q8) {
    rc = pack_int8_on_host(p, w);
    if (rc != TILES_OK) {
      release(p);
      return rc;
    }
  } else if (w->on_device) {
    // device-resident sources: one packing kernel for every segment
    std::vector<PackSeg> segs;
    segs.reserve(hp.copies.size());
    for (const CopySeg& c : hp.copies) {
      const uint8_t* src = static_cast<const uint8_t*>(src_ptr(w, c.tensor, c.layer));
      if (!src) {
        release(p);
        return set_err(TILES_E_ARG, "missing weight tensor for packing");
      }
      segs.push_back({src + c.src_row * c.cols * 2, c.cols * 2, c.dst_off, c.dst_pitch, c.nrows, c.cols * 2});
    }
    PackSeg* d_segs = nullptr;
    TRY(hipMalloc(&d_segs, segs.size() * sizeof(PackSeg)));
    hipError_t e1 = hipMemcpyAsync(d_segs, segs.data(), segs.size() * sizeof(PackSeg), hipMemcpyHostToDevice, p->stream);
    if (e1 == hipSuccess) e1 = launch_pack(d_segs, (int)segs.size(), p->packed, p->stream);
    if (e1 == hipSuccess) e1 = hipStreamSynchronize(p->stream);
    (void)hipFree(d_segs);
    if (e1 != hipSuccess) {
      std::string m = std::string("weight packing: ") + hipGetErrorString(e1);
      release(p);
      return set_err(TILES_E_HIP, m);
    }
  } else {
    for (const CopySeg& c : hp.copies) {
      const uint8_t* src = static_cast<const uint8_t*>(src_ptr(w, c.tensor, c.layer));
      if (!src) {
        release(p);
        return set_err(TILES_E_ARG, "missing weight tensor for packing");
      }
      src += c.src_row * c.cols * 2;
      TRY(hipMemcpy2DAsync(p->packed + c.dst_off, c.dst_pitch, src, c.cols * 2, c.cols * 2, c.nrows,
                           hipMemcpyHostToDevice, p->stream));
    }
  }
  // schedule
  TRY(hipMalloc(&p->d_tiles, hp.tiles.size() * sizeof(TileDesc)));
  TRY(hipMemcpyAsync(p->d_tiles, hp.tiles.data(), hp.tiles.size() * sizeof(TileDesc), hipMemcpyHostToDevice, p->stream));
  TRY(hipMalloc(&p->d_waves, hp.waves.size() * sizeof(WaveDesc)));
  TRY(hipMemcpyAsync(p->d_waves, hp.waves.data(), hp.waves.size() * sizeof(WaveDesc), hipMemcpyHostToDevice, p->stream));
  TRY(hipMalloc(&p->d_small, hp.small.size() * sizeof(LayerSmall)));
  TRY(hipMemcpyAsync(p->d_small, hp.small.data(), hp.small.size() * sizeof(LayerSmall), hipMemcpyHostToDevice, p->stream));
  {
    std::vector<uint64_t> chk = worker_table_hashes(hp);
    chk.push_back(p->build_id);
    TRY(hipMalloc(&p->d_table_check, chk.size() * sizeof(uint64_t)));
    TRY(hipMemcpy(p->d_table_check, chk.data(), chk.size() * sizeof(uint64_t), hipMemcpyHostToDevice));
  }
  // RoPE table: angles p * theta^(-2i/hd) in double, cos/sin rounded to float
  {
    const int half = hp.s.hd / 2;
    std::vector<float> rope((size_t)hp.s.max_positions * half * 2);
    for (int pos = 0; pos < hp.s.max_positions; ++pos)
      for (int i = 0; i < half; ++i) {
        const double inv = std::pow((double)cfg->rope_theta, -2.0 * i / hp.s.hd);
        const double ang = (double)pos * inv;
        rope[((size_t)pos * half + i) * 2] = (float)std::cos(ang);
        rope[((size_t)pos * half + i) * 2 + 1] = (float)std::sin(ang);
      }
    TRY(hipMalloc(&p->d_rope, rope.size() * sizeof(float)));
    TRY(hipMemcpy(p->d_rope, rope.data(), rope.size() * sizeof(float), hipMemcpyHostToDevice));
  }
  // scratch (one allocation, 256-byte aligned pieces)
  {
    size_t off = 0;
    auto piece = [&](size_t bytes) {
      size_t o = off;
      off += (bytes + 255) / 256 * 256;
      return o;
    };
    // (multi-token plans: one set of tagged buffers and LM-head partials per position of a step)
    const size_t o_ll = piece((size_t)hp.ll_words * 4 * hp.mt);
    const size_t o_lm = piece((size_t)hp.W * 8 * (hp.top_k > 0 ? hp.top_k : 1) * hp.mt);
    const size_t lm_end = off;
    p->sync_bytes = (size_t)SYNC_WORDS * 4;
    const size_t o_sync = piece(p->sync_bytes);
    const size_t o_forced = piece((size_t)MAX_STEPS * 4);
    p->scratch_bytes = off;
    TRY(hipMalloc(&p->scratch, p->scratch_bytes));
    TRY(hipMemsetAsync(p->scratch, 0, p->scratch_bytes, p->stream));
    p->ll = reinterpret_cast<uint32_t*>(p->scratch + o_ll);
    p->lmpart = reinterpret_cast<uint32_t*>(p->scratch + o_lm);
    p->fill_words = (int64_t)(lm_end - o_ll) / 4;
    p->sync = reinterpret_cast<uint32_t*>(p->scratch + o_sync);
    p->d_forced = reinterpret_cast<int32_t*>(p->scratch + o_forced);
  }
  if (cfg->flags & TILES_DEBUG_HIDDEN) {
    const size_t n = (size_t)MAX_STEPS * hp.s.n_layers * hp.s.H;
    TRY(hipMalloc(&p->dbg_hidden, n * sizeof(float)));
    TRY(hipMemsetAsync(p->dbg_hidden, 0, n * sizeof(float), p->stream));
  }
  if (cfg->flags & TILES_TRACE) {
    const size_t n = (size_t)MAX_STEPS * hp.waves.size() * hp.W * TRACE_WORDS;
    TRY(hipMalloc(&p->trace, n * sizeof(uint64_t)));
    TRY(hipMemsetAsync(p->trace, 0, n * sizeof(uint64_t), p->stream));
  }
  TRY(hipStreamSynchronize(p->stream));
#undef TRY
  *out = p;
  return TILES_OK;
}

int check_identity(const tiles_plan* p) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev != p->device) return set_err(TILES_E_DEVICE, "plan was created for another device");
  if (p->hp.W != p->cu_count) return set_err(TILES_E_DEVICE, "plan worker count differs from the CU count");
  if (plan_checksum(p->hp) != p->hp.checksum) return set_err(TILES_E_PLAN, "plan checksum mismatch (schedule modified)");
  return TILES_OK;
}

// One cooperative launch of the worker over n_steps positions (a multi-token plan runs them
// tokens_per_step at a time: n_steps / tokens_per_step kernel steps).  `noalloc`: the launch's
// tagged-data buffers, LM-head partials and status words live in the file-scope scratch array of
// this GPU (see noalloc_scratch) instead of the plan's own buffers; the layout is the same.
int decode_impl(tiles_plan_t* p, tiles_kv_t* kv, int32_t token, int32_t n_steps, int32_t* out_tokens,
                float* out_logits, bool noalloc, const float* uniforms, const int32_t* forced = nullptr) {
  if (!p || !kv || !out_tokens) return set_err(TILES_E_ARG, "null plan, kv or out_tokens");
  if (p->hp.mt > 1 && !forced)
    return set_err(TILES_E_ARG, "this plan runs multi-token verify steps (tokens_per_step > 1): use tiles_verify");
  if (p->hp.top_k > 0 && !uniforms)
    return set_err(TILES_E_ARG, "this plan samples (top_k > 0): use tiles_decode_sampled with the step uniforms");
  if (p->hp.top_k == 0 && uniforms) return set_err(TILES_E_ARG, "this plan is greedy (top_k = 0): use tiles_decode");
  if (!kv->k || (!kv->v && !p->hp.kv8)) return set_err(TILES_E_ARG, "null KV buffers");
  if (p->hp.kv8 && (!kv->k_scale || !kv->v_scale || !kv->k_smooth))
    return set_err(TILES_E_ARG, "an INT8 KV plan needs the cache's k_scale, v_scale and k_smooth");
  if (n_steps < 1 || n_steps > MAX_STEPS) return set_err(TILES_E_ARG, "n_steps must be in [1, 64]");
  const HostPlan& hp = p->hp;
  if (token < 0 || token >= hp.s.V) return set_err(TILES_E_ARG, "token out of range");
  if (kv->length < 0 || kv->capacity < 1) return set_err(TILES_E_ARG, "bad KV length or capacity");
  const int64_t limit = kv->capacity < hp.s.max_positions ? kv->capacity : hp.s.max_positions;
  if (kv->length + n_steps > limit) return set_err(TILES_E_ARG, "KV length + n_steps exceeds capacity / max_positions");
  int rc = check_identity(p);
  if (rc != TILES_OK) return rc;

  KernelArgs a;
  std::memset(&a, 0, sizeof(a));
  a.tiles = p->d_tiles;
  a.waves = p->d_waves;
  a.small = p->d_small;
  a.packed = p->packed;
  a.rope = p->d_rope;
  a.final_norm_off = hp.final_norm_off;
  a.embed_off = hp.embed_off;
  a.embed_stride = hp.embed_stride;
  uint32_t* ll = p->ll;
  uint32_t* lmpart = p->lmpart;
  uint32_t* sync = p->sync;
  if (noalloc) {
    const int64_t ll_bytes = ((int64_t)hp.ll_words * 4 * hp.mt + 255) / 256 * 256;
    const int64_t lm_bytes = ((int64_t)hp.W * 8 * (hp.top_k > 0 ? hp.top_k : 1) * hp.mt + 255) / 256 * 256;
    const int64_t need = ll_bytes + lm_bytes + SYNC_WORDS * 4;
    if (need > NOALLOC_SCRATCH_BYTES)
      return set_err(TILES_E_ARG, "this plan's tagged scratch (" + std::to_string(need) +
                                      " bytes) exceeds the allocation-free entry point's " +
                                      std::to_string(NOALLOC_SCRATCH_BYTES) + " bytes; use tiles_decode");
    uint32_t* base = nullptr;
    HIP_TRY(noalloc_scratch(p->device, &base));
    ll = base;
    lmpart = base + ll_bytes / 4;
    sync = lmpart + lm_bytes / 4;
  }
  a.ll = ll;
  a.lmpart = lmpart;
  a.sync = sync;
  a.table_check = p->d_table_check;
  a.kv_k = static_cast<uint16_t*>(kv->k);
  a.kv_v = static_cast<uint16_t*>(p->hp.kv8 ? kv->k : kv->v);  // (INT8 KV: one interleaved array)
  a.kv_ks = hp.kv8 ? kv->k_scale : nullptr;
  a.kv_vs = hp.kv8 ? kv->v_scale : nullptr;
  a.kv_sigma = hp.kv8 ? kv->k_smooth : nullptr;
  a.kv_cap = kv->capacity;
  a.out_tokens = out_tokens;
  a.out_logits = out_logits;
  a.uniforms = uniforms;
  a.top_k = hp.top_k;
  a.temperature = hp.temperature;
  a.top_p = hp.top_p;
  a.forced = forced;
  a.dbg_hidden = p->dbg_hidden;
  a.trace = p->trace;
  a.token0 = token;
  a.pos0 = (int32_t)kv->length;
  a.n_steps = n_steps / hp.mt;
  a.mt = hp.mt;
  a.ll_tok = hp.ll_words;
  a.kv8_span = hp.kv8_span;
  a.n_waves = (int32_t)hp.waves.size();
  a.W = hp.W;
  a.n_layers = hp.s.n_layers;
  a.H = hp.s.H;
  a.Hpad = hp.s.Hpad;
  a.n_heads = hp.s.n_heads;
  a.n_kv = hp.s.n_kv;
  a.head_dim = hp.s.hd;
  a.F = hp.s.F;
  a.Fpad = hp.s.Fpad;
  a.V = hp.s.V;
  a.qkv_rows = hp.s.qkv_rows;
  a.Qpad = hp.s.Qpad;
  a.S = hp.S;
  a.combine_in_o = hp.combine_in_o;
  a.eps = p->cfg.rms_eps;
  a.qscale = (float)(1.4426950408889634 / std::sqrt((double)hp.s.hd));
  a.spin_limit = p->spin_limit;
  a.lds_vec_floats = hp.lds_vec_floats;
  a.lds_part_floats = hp.lds_part_floats;
  a.lds_xres_floats = hp.lds_xres_floats;
  a.lds_stage_floats = hp.lds_stage_floats;
  a.stage_batches = hp.stage_batches;

  // Kernels rather than memsets, so that the launch sequence can be captured in a graph.
  HIP_TRY(launch_fill(ll, p->fill_words, TAG_FILL, p->stream));
  HIP_TRY(launch_fill(sync, SYNC_WORDS, 0u, p->stream));
  if (p->cfg.flags & TILES_POISON) {
    // NaN into the rows this launch writes: a read before the write would surface as NaN
    const int nblk = hp.s.n_layers * hp.s.n_kv;
    if (hp.kv8) {  // INT8 codes cannot be NaN: the rows' scales are (two BF16 NaN halves make an FP32 NaN)
      const int64_t stride = kv->capacity * 2, first = kv->length * 2, count = (int64_t)n_steps * 2;
      HIP_TRY(launch_fill_blocks(reinterpret_cast<uint16_t*>(a.kv_ks) + first, nblk, stride, count, 0x7fc0, p->stream));
      HIP_TRY(launch_fill_blocks(reinterpret_cast<uint16_t*>(a.kv_vs) + first, nblk, stride, count, 0x7fc0, p->stream));
    } else {
      const int64_t stride = kv->capacity * hp.s.hd, first = kv->length * hp.s.hd, count = (int64_t)n_steps * hp.s.hd;
      HIP_TRY(launch_fill_blocks(a.kv_k + first, nblk, stride, count, 0x7fc0, p->stream));
      HIP_TRY(launch_fill_blocks(a.kv_v + first, nblk, stride, count, 0x7fc0, p->stream));
    }
  }
  void* args[] = {&a};
  // (the worker checks its watchdog every 32 polling rounds; a short test watchdog runs the test
  // instantiation, which checks every round)
  const void* kern = p->spin_limit < 32 ? p->kernel_wd : p->kernel;
  HIP_TRY(hipLaunchCooperativeKernel(kern, dim3(hp.W), dim3(BLOCK_THREADS), args, hp.lds_bytes, p->stream));
  kv->length += n_steps;
  p->last_steps = n_steps;
  p->last_sync = sync;
  return TILES_OK;
}


}  // namespace

extern "C" {

tiles_plan_t* tiles_plan_create(const tiles_config_t* cfg, const tiles_weights_t* w) {
  g_err.clear();
  tiles_plan* p = nullptr;
  int rc = create_impl(cfg, w, &p);
  if (rc != TILES_OK) return nullptr;
  return p;
}

int tiles_decode(tiles_plan_t* p, tiles_kv_t* kv, int32_t token, int32_t n_steps, int32_t* out_tokens,
                 float* out_logits) {
  return decode_impl(p, kv, token, n_steps, out_tokens, out_logits, false, nullptr);
}

int tiles_decode_sampled(tiles_plan_t* p, tiles_kv_t* kv, int32_t token, int32_t n_steps, const float* uniforms,
                         int32_t* out_tokens, float* out_logits) {
  if (p && p->hp.top_k == 0) return set_err(TILES_E_ARG, "this plan is greedy (top_k = 0): use tiles_decode");
  if (!uniforms) return set_err(TILES_E_ARG, "null uniforms");
  return decode_impl(p, kv, token, n_steps, out_tokens, out_logits, false, uniforms);
}

int tiles_decode_noalloc(tiles_plan_t* p, tiles_kv_t* kv, int32_t token, int32_t n_steps, int32_t* out_tokens,
                         float* out_logits) {
  return decode_impl(p, kv, token, n_steps, out_tokens, out_logits, true, nullptr);
}

int tiles_verify(tiles_plan_t* p, tiles_kv_t* kv, const int32_t* tokens, int32_t m, int32_t* out_argmax,
                 float* out_logits) {
  if (!p || !tokens) return set_err(TILES_E_ARG, "null plan or tokens");
  if (p->hp.top_k > 0) return set_err(TILES_E_ARG, "verify steps are greedy: this plan samples (top_k > 0)");
  if (m < 1 || m > MAX_STEPS) return set_err(TILES_E_ARG, "m must be in [1, 64]");
  if (m % p->hp.mt != 0) return set_err(TILES_E_ARG, "m must be a multiple of the plan's tokens_per_step");
  for (int32_t i = 0; i < m; ++i)
    if (tokens[i] < 0 || tokens[i] >= p->hp.s.V) return set_err(TILES_E_ARG, "token out of range");
  if (m > 1) HIP_TRY(hipMemcpyAsync(p->d_forced, tokens + 1, (size_t)(m - 1) * 4, hipMemcpyHostToDevice, p->stream));
  return decode_impl(p, kv, tokens[0], m, out_argmax, out_logits, false, nullptr, p->d_forced);
}

int tiles_kv_convert_int8(tiles_plan_t* p, const void* k_bf16, const void* v_bf16, int64_t capacity, int64_t length,
                          tiles_kv_t* dst) {
  if (!p || !k_bf16 || !v_bf16 || !dst) return set_err(TILES_E_ARG, "null plan, source or destination");
  if (!p->hp.kv8) return set_err(TILES_E_ARG, "the plan's KV format is BF16");
  if (!dst->k || !dst->k_scale || !dst->v_scale || !dst->k_smooth) return set_err(TILES_E_ARG, "null INT8 KV buffers");
  if (capacity < 1 || length < 0 || length > capacity || dst->capacity != capacity)
    return set_err(TILES_E_ARG, "bad capacity or length (dst->capacity must equal capacity)");
  const Shape& s = p->hp.s;
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev != p->device) return set_err(TILES_E_DEVICE, "plan was created for another device");
  HIP_TRY(launch_kv_convert(static_cast<const uint16_t*>(k_bf16), static_cast<const uint16_t*>(v_bf16), capacity, length,
                            s.hd, (int64_t)s.n_layers * s.n_kv, static_cast<int8_t*>(dst->k), dst->k_scale,
                            dst->v_scale, dst->k_smooth, p->stream));
  dst->length = length;
  return TILES_OK;
}

void tiles_plan_destroy(tiles_plan_t* p) { release(p); }

const char* tiles_last_error(void) { return g_err.c_str(); }

static void fill_info(const HostPlan& hp, int occupancy, uint64_t build_id, tiles_plan_info_t* info) {
  std::memset(info, 0, sizeof(*info));
  info->n_workers = hp.W;
  info->block_threads = BLOCK_THREADS;
  info->lds_bytes = hp.lds_bytes;
  info->waves_per_step = (int32_t)hp.waves.size();
  int32_t n = 0;
  for (const TileDesc& t : hp.tiles) n += t.kind != KIND_NONE;
  info->n_tiles = n;
  info->kv_splits = hp.S;
  info->combine_mode = hp.combine_in_o ? 1 : 2;
  info->attn_heads = hp.T;
  info->weight_format = hp.q8 ? TILES_WEIGHTS_INT8 : TILES_WEIGHTS_BF16;
  info->top_k = hp.top_k;
  info->kv_format = hp.kv8 ? TILES_KV_INT8 : TILES_KV_BF16;
  info->tokens_per_step = hp.mt;
  info->stage_batches = hp.stage_batches;
  for (size_t wv = 0; wv < hp.waves.size(); ++wv)
    if (hp.waves[wv].kind == KIND_O) {
      info->o_workers = hp.wave_busy[wv];
      break;
    }
  info->occupancy = occupancy;
  info->packed_bytes = hp.packed_bytes;
  info->weight_bytes_per_step = hp.weight_bytes_per_step;
  info->max_over_mean = hp.max_over_mean;
  info->checksum = hp.checksum;
  info->build_id = build_id;
}

int tiles_plan_info(const tiles_plan_t* p, tiles_plan_info_t* info) {
  if (!p || !info) return set_err(TILES_E_ARG, "null plan or info");
  fill_info(p->hp, p->occupancy, p->build_id, info);
  return TILES_OK;
}

int tiles_plan_wave(const tiles_plan_t* p, int32_t wave, tiles_wave_info_t* out) {
  if (!p || !out) return set_err(TILES_E_ARG, "null plan or output");
  if (wave < 0 || wave >= (int32_t)p->hp.waves.size()) return set_err(TILES_E_ARG, "wave out of range");
  std::memset(out, 0, sizeof(*out));
  out->kind = p->hp.waves[wave].kind;
  out->layer = p->hp.waves[wave].layer;
  out->busy_workers = p->hp.wave_busy[wave];
  out->weight_bytes = p->hp.wave_bytes[wave];
  out->max_worker_bytes = p->hp.wave_max_bytes[wave];
  return TILES_OK;
}

int tiles_plan_dry_run(const tiles_config_t* cfg, int32_t n_workers, tiles_plan_info_t* info) {
  if (!cfg || !info) return set_err(TILES_E_ARG, "null config or info");
  HostPlan hp;
  std::string err;
  int rc = build_plan(*cfg, n_workers, hp, err);
  if (rc != TILES_OK) return set_err(rc, err);
  fill_info(hp, 0, TILES_BUILD_ID, info);
  return TILES_OK;
}

int tiles_plan_debug_validate(const tiles_config_t* cfg, int32_t n_workers, int32_t mutation) {
  if (!cfg) return set_err(TILES_E_ARG, "null config");
  HostPlan hp;
  std::string err;
  int rc = build_plan(*cfg, n_workers, hp, err);
  if (rc != TILES_OK) return set_err(rc, err);
  rc = debug_mutate_plan(hp, mutation, err);
  if (rc != TILES_OK) return set_err(rc, err);
  rc = validate_plan(hp, err);
  if (rc != TILES_OK) return set_err(rc, err);
  g_err.clear();
  return TILES_OK;
}

int tiles_plan_set_stream(tiles_plan_t* p, void* stream) {
  if (!p) return set_err(TILES_E_ARG, "null plan");
  p->stream = static_cast<hipStream_t>(stream);
  return TILES_OK;
}

int tiles_plan_status(tiles_plan_t* p) {
  if (!p) return set_err(TILES_E_ARG, "null plan");
  HIP_TRY(hipStreamSynchronize(p->stream));
  uint32_t status = 0;
  uint32_t* sync = p->last_sync ? p->last_sync : p->sync;
  HIP_TRY(hipMemcpy(&status, sync + SYNC_STATUS_WORD, 4, hipMemcpyDeviceToHost));
  if (status != 0) {
    HIP_TRY(hipMemset(sync, 0, p->sync_bytes));
    if (status == STATUS_TABLES)
      return set_err(TILES_E_PLAN, "a worker's device-resident schedule or build id failed its check in the last launch");
    return set_err(TILES_E_KERNEL, "a wait's watchdog expired in the last launch");
  }
  return TILES_OK;
}

int tiles_read_debug(tiles_plan_t* p, float* hidden, uint64_t* trace, int32_t* n_steps_out) {
  if (!p) return set_err(TILES_E_ARG, "null plan");
  HIP_TRY(hipStreamSynchronize(p->stream));
  const HostPlan& hp = p->hp;
  if (n_steps_out) *n_steps_out = p->last_steps;
  if (hidden) {
    if (!p->dbg_hidden) return set_err(TILES_E_ARG, "plan was created without TILES_DEBUG_HIDDEN");
    HIP_TRY(hipMemcpy(hidden, p->dbg_hidden, (size_t)p->last_steps * hp.s.n_layers * hp.s.H * sizeof(float),
                      hipMemcpyDeviceToHost));
  }
  if (trace) {
    if (!p->trace) return set_err(TILES_E_ARG, "plan was created without TILES_TRACE");
    // one record per kernel step (a verify plan's step runs hp.mt positions)
    HIP_TRY(hipMemcpy(trace, p->trace,
                      (size_t)(p->last_steps / hp.mt) * hp.waves.size() * hp.W * TRACE_WORDS * sizeof(uint64_t),
                      hipMemcpyDeviceToHost));
  }
  return TILES_OK;
}

int tiles_plan_debug_spin_limit(tiles_plan_t* p, uint32_t rounds) {
  if (!p) return set_err(TILES_E_ARG, "null plan");
  const uint32_t limit = rounds ? rounds : DEFAULT_SPIN_LIMIT;
  if (limit < 32 && !p->kernel_wd) {
    const void* k = worker_kernel(p->hp.s.hd, p->hp.T, true, p->hp.q8 != 0, p->hp.top_k > 0, p->hp.kv8 != 0, p->hp.mt);
    if (!k)
      return set_err(TILES_E_CONFIG, "a watchdog under 32 rounds needs BF16 weights and KV, greedy decoding, one "
                                     "query head per attention tile and one position per step");
    HIP_TRY(hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, p->hp.lds_bytes));
    int occ = 0;
    HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k, BLOCK_THREADS, p->hp.lds_bytes));
    if (occ < 1) return set_err(TILES_E_DEVICE, "test worker kernel cannot be resident (occupancy < 1)");
    p->kernel_wd = k;
  }
  p->spin_limit = limit;
  return TILES_OK;
}

int tiles_plan_debug_corrupt(tiles_plan_t* p) {
  if (!p) return set_err(TILES_E_ARG, "null plan");
  if (p->hp.tiles.empty()) return set_err(TILES_E_PLAN, "empty plan");
  p->hp.tiles[p->hp.tiles.size() / 2].woff ^= 0x400;
  return TILES_OK;
}

int tiles_plan_debug_corrupt_device(tiles_plan_t* p) {
  if (!p) return set_err(TILES_E_ARG, "null plan");
  if (p->hp.tiles.empty() || !p->d_tiles) return set_err(TILES_E_PLAN, "empty plan");
  // one bit of the woff field of a tile in the middle of the table (device copy only)
  const size_t idx = p->hp.tiles.size() / 2;
  uint8_t* byte = reinterpret_cast<uint8_t*>(p->d_tiles + idx) + offsetof(TileDesc, woff) + 1;
  uint8_t v = 0;
  HIP_TRY(hipStreamSynchronize(p->stream));
  HIP_TRY(hipMemcpy(&v, byte, 1, hipMemcpyDeviceToHost));
  v ^= 0x04;
  HIP_TRY(hipMemcpy(byte, &v, 1, hipMemcpyHostToDevice));
  return TILES_OK;
}

int tiles_quantize_rows_int8(const uint16_t* bf16, int64_t rows, int64_t cols, int8_t* q, float* scales) {
  if (!bf16 || !q || !scales) return set_err(TILES_E_ARG, "null pointer");
  if (rows < 0 || cols < 0) return set_err(TILES_E_ARG, "negative size");
  quantize_rows_int8(bf16, cols, rows, cols, q, cols, scales, 1);
  return TILES_OK;
}

int tiles_stream_read(const void* buf, int64_t bytes, int32_t n_groups, uint32_t* sink, void* stream) {
  if (!buf || !sink) return set_err(TILES_E_ARG, "null buffer or sink");
  if (n_groups < 1 || n_groups > 65536) return set_err(TILES_E_ARG, "n_groups out of range [1, 65536]");
  const int64_t unit = (int64_t)n_groups * NWAVES * STREAM_DEPTH * CHUNK_BYTES;
  if (bytes <= 0 || bytes % unit != 0)
    return set_err(TILES_E_ARG, "bytes must be a positive multiple of n_groups * 8 wavefronts * 8 KB");
  if (bytes / ((int64_t)n_groups * NWAVES) > (int64_t)0xffffffffll)
    return set_err(TILES_E_ARG, "more than 4 GB per wavefront");
  HIP_TRY(launch_stream_read(static_cast<const uint8_t*>(buf), bytes, n_groups, sink, static_cast<hipStream_t>(stream)));
  return TILES_OK;
}

int tiles_edge_latency(uint32_t* words, int32_t peer, int32_t iters, uint32_t spin_limit, uint64_t* out,
                       void* stream) {
  if (!words || !out) return set_err(TILES_E_ARG, "null words or out");
  if (peer < 1 || peer > 255) return set_err(TILES_E_ARG, "peer out of range [1, 255]");
  if (iters < 1 || iters > (1 << 20)) return set_err(TILES_E_ARG, "iters out of range [1, 2^20]");
  if (spin_limit == 0) return set_err(TILES_E_ARG, "spin_limit must be positive");
  HIP_TRY(launch_edge_latency(words, peer, iters, spin_limit, out, static_cast<hipStream_t>(stream)));
  return TILES_OK;
}

}  // extern "C"
