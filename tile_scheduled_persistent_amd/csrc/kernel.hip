// The persistent tile worker for gfx950 (CDNA4).
//
// One workgroup per compute unit executes the static per-step schedule built by the
// host planner: for every decoded token, for every wave, gather the tile's inputs, run
// the tile (if any) and publish its outputs.  The kernel makes no scheduling decision of
// its own ("Tiles: Scheduling LLM Decoding as a Graph of Tiles", intro): tiles, workers,
// wave order and split boundaries are all fixed by the plan and the attended length.
//
// Synchronisation between waves is carried by the data itself.  Every FP32 value a tile
// publishes for other workers holds the step's parity in the lowest mantissa bit (the
// value consumers use is the published one with that bit cleared); consumers poll the
// producer wave's output buffer with device-coherent 16-byte loads until every element
// they need shows the current parity.  One memory round trip thus both signals and moves
// the data: there is no grid barrier, no flag and no wait for store completion on the
// critical path.  Each wave has its own output buffer, written exactly once per step.  The
// generations are separated by one all-to-all per step: every worker ends a step with a
// release store of its LM-head partial, and every worker begins the next step by reading all
// W partials (the token gather) followed by an acquire.  So when any worker starts step s + 1,
// every worker has finished step s (each of its reads and writes), and every store of step s
// is visible to it: a producer never overwrites a value a consumer still needs, and a consumer
// polling at step s + 1 sees each buffer's step-s value (the other parity) until the
// step-(s+1) value arrives, never an older one of its own parity.  The buffers are filled with
// a quiet NaN of parity 0 before every launch; step 0 publishes parity 1.
//
// Workgroup organisation (512 threads = 8 wavefronts):
//   * all eight wavefronts share the input gather of every wave (each polls its share of
//     the 16-byte units) and the LDS-only prologue work (norm scale, q/k norm + RoPE,
//     split merge);
//   * wavefront 0 is the control wave: it runs the epilogues (residual add, SwiGLU,
//     partial argmax), the KV write and every global store;
//   * wavefronts 1..7 are compute waves: each streams its share of the worker's packed
//     weights into registers (16-byte loads, double-buffered) and, before a tile's last
//     batch is consumed, issues the loads of its next GEMV tile, so those bytes arrive
//     while the workgroup gathers the next inputs: weights do not depend on activations,
//     only the dot products do (the Tiles page credits this prefetch idea to the
//     megakernel it builds on).
//
// Tile bodies:
//   * GEMV tiles: one "chunk" = 64 lanes x 16 B = 512 columns of one row; FP32 dot
//     products against the LDS input vector, reduced across the wavefront with DPP
//     ("History and roadmap", TileInfer.jl, "M8 so far": residual add + RMSNorm and
//     SwiGLU fused into the GEMV).
//   * Attention tiles: one split of grouped-query attention over the BF16 KV cache with
//     an online softmax; the compute waves' states are merged through LDS and the
//     splits are merged in the o_proj prologue or in a wave of their own (roadmap
//     "Milestones", M5: split-KV decode; "Tried and not kept": no combine inside the
//     split kernel).
//   * LM head: logits and a (max, lowest index) partial per worker; the next step's
//     first wave reduces all partials in worker order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "plan_types.h"

#ifndef TILES_BUILD_ID
#define TILES_BUILD_ID 0x0ull
#endif

namespace tiles {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int SC1 = 16;  // buffer-instruction cache policy bit: device-coherent access
constexpr int NT = 2;    // buffer-instruction cache policy bit: non-temporal (streamed once)

// ---------------------------------------------------------------------------
// coherent memory helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t ld_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The per-step LM-head partial is a release: every store this wavefront made earlier in the step
// (all of the worker's published values and its KV rows: the control wavefront makes every global
// store) is visible before the partial is.
__device__ __forceinline__ void st_u64_release(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Buffer descriptor over a scratch array (byte offsets < 4 GB).  Device-coherent buffer
// loads through it are plain (non-atomic) loads the compiler can issue back to back.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0xffffffffu, 0x00020000);
}
__device__ __forceinline__ u32x4 cld4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, SC1);
}
#define COMPILER_FENCE() asm volatile("" ::: "memory")


__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round-to-nearest-even FP32 -> BF16 (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_round(float f) { return __uint_as_float(f32_to_bf16_bits(f) << 16); }

// ---------------------------------------------------------------------------
// tagged data: parity in the lowest mantissa bit
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t step_parity(int step) { return (uint32_t)((step + 1) & 1); }
// the value every consumer (and the producer itself) uses
__device__ __forceinline__ float tag_clear(float v) { return __uint_as_float(__float_as_uint(v) & ~1u); }
__device__ __forceinline__ void publish(uint32_t* buf, int64_t i, float v, uint32_t par) {
  st_u32(buf + i, (__float_as_uint(v) & ~1u) | par);
}
__device__ __forceinline__ bool unit_ready(const u32x4 v, uint32_t par) {
  return par ? ((v.x & v.y & v.z & v.w) & 1u) != 0 : ((v.x | v.y | v.z | v.w) & 1u) == 0;
}
__device__ __forceinline__ f32x4 unit_values(const u32x4 v) {
  return f32x4{__uint_as_float(v.x & ~1u), __uint_as_float(v.y & ~1u), __uint_as_float(v.z & ~1u),
               __uint_as_float(v.w & ~1u)};
}

// ---------------------------------------------------------------------------
// wavefront reductions (DPP butterflies; every lane ends with the same value)
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <-> 7-i within 8
constexpr int DPP_MIRROR = 0x140;       // lane i <-> 15-i within 16

__device__ __forceinline__ float sum4(float v) {
  v += dpp<DPP_XOR1>(v);
  v += dpp<DPP_XOR2>(v);
  return v;
}
__device__ __forceinline__ float sum8(float v) {
  v += dpp<DPP_XOR1>(v);
  v += dpp<DPP_XOR2>(v);
  v += dpp<DPP_HALF_MIRROR>(v);
  return v;
}
__device__ __forceinline__ float sum16(float v) {
  v = sum8(v);
  v += dpp<DPP_MIRROR>(v);
  return v;
}
// Lane exchanges across 4, 8, 16 and 32 lanes without the LDS crossbar: DPP rotations by 4 and 8
// within each 16-lane row (for sums and maxima over lanes of equal residue a rotation does what an
// exchange does), and the gfx950 permlane swaps of 16-lane rows and 32-lane halves.
__device__ __forceinline__ float xor4(float v) { return dpp<0x124>(v); }  // row_ror:4
__device__ __forceinline__ float xor8(float v) { return dpp<0x128>(v); }  // row_ror:8
__device__ __forceinline__ float xor16(float v, int lane) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(((lane >> 4) & 1) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32(float v, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(lane >= 32 ? r[0] : r[1]);
}
template <int OFF>
__device__ __forceinline__ float lane_xor(float v, int lane) {
  static_assert(OFF == 4 || OFF == 8 || OFF == 16 || OFF == 32, "lane_xor offsets: 4, 8, 16, 32");
  if constexpr (OFF == 4) return xor4(v);
  else if constexpr (OFF == 8) return xor8(v);
  else if constexpr (OFF == 16) return xor16(v, lane);
  else return xor32(v, lane);
}

// the largest value of the wavefront, in every lane
__device__ __forceinline__ float wave_max(float v, int lane) {
  v = fmaxf(v, dpp<DPP_XOR1>(v));
  v = fmaxf(v, dpp<DPP_XOR2>(v));
  v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_MIRROR>(v));
  v = fmaxf(v, lane_xor<16>(v, lane));
  return fmaxf(v, lane_xor<32>(v, lane));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = sum16(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// ---------------------------------------------------------------------------
// LDS layout (dynamic, from LDS address 0): stage | vec | part | xres | small | segs | tiles |
// waves | lsmall.
//   stage per compute wavefront, staged chunks of its next GEMV range (direct-to-LDS loads; first,
//         so that their LDS addresses stay below 64 KB)
//   vec   GEMV input vector (or the raw q/k/v of an attention tile)
//   part  GEMV row partials, attention work areas, gathered split partials
//   xres  the residual stream x as last gathered (read by the o_proj / down epilogues)
//   small per-wave words: the abort flag and the per-wavefront sums of squares
// ---------------------------------------------------------------------------
constexpr int SM_ABORT = 0;  // int: some wavefront gave up waiting (all leave after barrier P)
constexpr int SM_SS = 8;     // float[NWAVES]: sums of squares of each wavefront's share of x
constexpr int SM_CTRACE = 32;  // uint64[2][8]: first compute wavefront's timestamps of a tile (set = tile parity)
constexpr int SM_WDONE = 64;   // uint64[2][8]: each compute wavefront's done stamp of a tile (set = tile parity)
constexpr int SM_ROPE = 256;   // float[head_dim]: (cos, sin) pairs of the current position (attention tiles)
constexpr int SM_QGAIN = 512;  // float[head_dim]: q-norm gains (attention tiles with q/k norm)
constexpr int SM_KGAIN = 640;  // float[head_dim]: k-norm gains
constexpr int SM_KSMOOTH = 768;  // float[head_dim]: INT8 KV key smoothing factors of the tile's KV head
constexpr int SM_KVCUR = 896;    // float[2]: INT8 KV scales of the current position's K and V rows
constexpr int SM_SS2 = 960;      // float[3][NWAVES]: as SM_SS, for positions 1 .. 3 of a multi-token step
// (multi-token steps, INT8 KV: SM_KVCUR holds the (K, V) scales of every position of the step, 2 x 4 at most)
// (multi-token steps keep one (cos, sin) row per position of the step after the attention tile's areas
// instead: see rope_rows)
__device__ __forceinline__ int sm_ss(int t) { return t == 0 ? SM_SS : SM_SS2 + (t - 1) * NWAVES; }

struct Lds {
  float* vec;
  float* part;
  float* xres;
  float* scl;           // weight-only INT8: the scales of the rows of the GEMV block being worked
  float* stage;
  float* small;
  SegDesc* segs;
  TileDesc* tiles;      // this worker's tile of every wave
  WaveDesc* waves;      // every wave's descriptor
  LayerSmall* lsmall;   // per-layer gain offsets
};

// The schedule tables live in LDS for the whole launch: read from global memory they are cold
// every time (each entry is used once per token) and each read would wait behind the weight
// stream.  Values read from LDS are per-lane to the compiler; readfirstlane makes them scalar.
__device__ __forceinline__ int sc(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t sc64(int64_t v) {
  return ((int64_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
}
__device__ __forceinline__ TileDesc tile_of(const Lds& L, int k) {
  const TileDesc x = L.tiles[k];
  TileDesc t;
  t.kind = sc(x.kind);
  t.row0 = sc(x.row0);
  t.nrows = sc(x.nrows);
  t.kpad = sc(x.kpad);
  t.woff = sc64(x.woff);
  t.aux0 = sc(x.aux0);  // attention: first query head of the tile
  t.aux1 = 0;
  return t;
}
__device__ __forceinline__ WaveDesc wave_of(const Lds& L, int k) {
  const WaveDesc x = L.waves[k];
  WaveDesc w;
  w.kind = sc(x.kind);
  w.layer = sc(x.layer);
  w.max_rows = sc(x.max_rows);
  w.ll_off = sc(x.ll_off);
  return w;
}
__device__ __forceinline__ int64_t gain_off(const Lds& L, int layer, int which) {  // 0 attn, 1 mlp, 2 q, 3 k
  const LayerSmall& x = L.lsmall[layer];
  return sc64(which == 0 ? x.attn_norm : which == 1 ? x.mlp_norm : which == 2 ? x.q_norm : x.k_norm);
}

__device__ __forceinline__ bool is_gemv(int kind) {
  return kind == KIND_QKV || kind == KIND_O || kind == KIND_GU || kind == KIND_DOWN || kind == KIND_LM;
}
// chunk range of compute wave c over n chunks
__device__ __forceinline__ int chunk_lo(int n, int c) { return (int)((uint32_t)(n * c) / NCOMP); }

// ---------------------------------------------------------------------------
// waiting: every poll loop is bounded (watchdog) and leaves when any worker has aborted
// ---------------------------------------------------------------------------

// WD: the test instantiation of the worker, whose waits check every round (a short watchdog set
// from the host then makes ordinary waits give up); the worker proper checks every 32 rounds.
template <bool WD>
__device__ __forceinline__ bool watch_tick(const KernelArgs& a, uint32_t& spins, int lane) {
  ++spins;
  if ((spins & (WD ? 0u : 31u)) == 0) {
    if (ld_u32(a.sync + SYNC_ABORT_WORD) != 0) return true;
    if (spins > a.spin_limit) {
      if (lane == 0) {
        st_u32(a.sync + SYNC_STATUS_WORD, 1u);
        st_u32(a.sync + SYNC_ABORT_WORD, 1u);
      }
      return true;
    }
  }
  return false;
}

// Poll-gather `nunits` 16-byte units of tagged floats.  Unit u of the gathered vector sits at
// unit map(u) of `src`; the units are dealt to `nslots` wavefronts, this one taking
// u = (i * nslots + slot) * 64 + lane.  prep(i, u) runs once per owned unit before polling
// (to issue independent loads early), sink(i, u, x) once the unit shows parity `par`.
// Only units not yet seen are re-read.  Returns true when the wait was abandoned.
template <int GB, bool WD, typename Map, typename Prep, typename Sink>
__device__ __forceinline__ bool gather(const KernelArgs& a, const uint32_t* src, int nunits, int slot, int nslots, uint32_t par,
                       int lane, Map map, Prep prep, Sink sink) {
  const __amdgpu_buffer_rsrc_t r = rsrc(src);
  for (int base = 0; base < nunits; base += GB * nslots * 64) {
    uint32_t pending = 0;
#pragma unroll
    for (int i = 0; i < GB; ++i) {
      const int u = base + (i * nslots + slot) * 64 + lane;
      if (u < nunits) {
        pending |= 1u << i;
        prep(i, u);
      }
    }
    uint32_t spins = 0;
    for (;;) {
      u32x4 v[GB];
      COMPILER_FENCE();
#pragma unroll
      for (int i = 0; i < GB; ++i) {
        v[i] = u32x4{0u, 0u, 0u, 0u};
        if ((pending >> i) & 1u) v[i] = cld4(r, (uint32_t)map(base + (i * nslots + slot) * 64 + lane) * 16u);
      }
      COMPILER_FENCE();
#pragma unroll
      for (int i = 0; i < GB; ++i) {
        if (((pending >> i) & 1u) && unit_ready(v[i], par)) {
          sink(i, base + (i * nslots + slot) * 64 + lane, unit_values(v[i]));
          pending &= ~(1u << i);
        }
      }
      if (__all(pending == 0)) break;
      if (watch_tick<WD>(a, spins, lane)) return true;
      // a long wait polls less often: less polling traffic on the fabric for the other workers
      if (spins > 4) __builtin_amdgcn_s_sleep(8);
    }
  }
  return false;
}

// The same over the MT positions of a multi-token step in one polling loop: position t's n units
// are those of src + t * tok_words (units t * n .. t * n + n - 1 of the combined range); map, prep
// and sink see the position and the unit within it.
template <int GB, int MT, bool WD, typename Map, typename Prep, typename Sink>
__device__ __forceinline__ bool gather_mt(const KernelArgs& a, const uint32_t* src, int n, int64_t tok_words, int slot,
                                          int nslots, uint32_t par, int lane, Map map, Prep prep, Sink sink) {
  const int tok_units = (int)(tok_words / 4);
  auto split = [&](int u, int& t) {
    t = 0;
#pragma unroll
    for (int k = 1; k < MT; ++k) t += u >= k * n ? 1 : 0;
    return u - t * n;
  };
  return gather<GB, WD>(
      a, src, MT * n, slot, nslots, par, lane,
      [&](int u) {
        int t;
        const int w = split(u, t);
        return t * tok_units + map(w);
      },
      [&](int i, int u) {
        int t;
        const int w = split(u, t);
        prep(i, t, w);
      },
      [&](int i, int u, const f32x4 x) {
        int t;
        const int w = split(u, t);
        sink(i, t, w, x);
      });
}

constexpr int GATHER_UNITS = 4;  // units per lane per polling pass (8 wavefronts x 64 lanes x 4 = 8192 floats)
// Plain gathers (split partials into the o_proj prologue, the down input) poll twice as many
// units per pass: the partials of 32 heads x 5 splits then arrive in one round trip.
constexpr int GATHER_UNITS_PLAIN = 2 * GATHER_UNITS;

struct Identity {
  __device__ int operator()(int u) const { return u; }
};
struct NoPrep {
  __device__ void operator()(int, int) const {}
};

// Columns of one packed chunk: 512 BF16 weights, or 1024 INT8 codes.
template <bool Q8>
constexpr int chunk_cols() { return Q8 ? CHUNK_COLS_I8 : CHUNK_COLS; }

// LDS position of GEMV input element i.  In a packed chunk lane l holds VPL = columns / 64
// consecutive columns, 4 per dword (INT8) or per two dwords (BF16); group h (of 4 columns) of
// lane l is stored at chunk offset 256 h + 4 l, so that the 64 lanes' 16-byte reads of one group
// are consecutive in LDS (no bank conflicts; consecutive columns 4 apart by lane would collide).
// Groups of four stay contiguous, so 16-byte aligned writes of four elements stay 16-byte writes.
template <bool Q8>
__device__ __forceinline__ int vperm(int i) {
  constexpr int CC = chunk_cols<Q8>(), VPL = CC / 64;
  return (i & ~(CC - 1)) | (((i & (VPL - 1)) >> 2) << 8) | (((i & (CC - 1)) / VPL) << 2) | (i & 3);
}

// x (n floats, tagged) -> xres = x, vec = x * gain (GEMV input order, vperm), and this
// wavefront's sum of squares of its share
template <bool WD, bool Q8>
__device__ __forceinline__ bool gather_norm(const KernelArgs& a, float* vec, float* xres, const uint32_t* src, int n,
                                            const uint16_t* gain, int slot, int lane, uint32_t par, float& ss) {
  uint2 gv[GATHER_UNITS];
  float s = 0.f;
  const bool ab = gather<GATHER_UNITS, WD>(
      a, src, n / 4, slot, NWAVES, par, lane, Identity{},
      [&](int i, int u) { gv[i] = *reinterpret_cast<const uint2*>(gain + u * 4); },
      [&](int i, int u, const f32x4 x) {
        *reinterpret_cast<f32x4*>(xres + u * 4) = x;
        const f32x4 v = {x.x * bf16_lo(gv[i].x), x.y * bf16_hi(gv[i].x), x.z * bf16_lo(gv[i].y), x.w * bf16_hi(gv[i].y)};
        *reinterpret_cast<f32x4*>(vec + vperm<Q8>(u * 4)) = v;
        s += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
      });
  ss = wave_sum(s);
  return ab;
}

// plain tagged vector -> dst (in GEMV input order, vperm, when `perm`)
template <bool WD, bool Q8>
__device__ __forceinline__ bool gather_plain(const KernelArgs& a, float* dst, const uint32_t* src, int n, int slot, int lane,
                             uint32_t par, bool perm) {
  return gather<GATHER_UNITS_PLAIN, WD>(a, src, n / 4, slot, NWAVES, par, lane, Identity{}, NoPrep{},
                              [&](int, int u, const f32x4 x) {
                                *reinterpret_cast<f32x4*>(dst + (perm ? vperm<Q8>(u * 4) : u * 4)) = x;
                              });
}

// Multi-token steps: gather_norm for the MT positions in one polling loop (position t into
// vec + t * vs, xres + t * xs, its sum of squares in ss[t]).
template <bool WD, bool Q8, int MT>
__device__ __forceinline__ bool gather_norm_mt(const KernelArgs& a, float* vec, float* xres, int vs, int xs,
                                               const uint32_t* src, int n, const uint16_t* gain, int slot, int lane,
                                               uint32_t par, float (&ss)[MT]) {
  uint2 gv[GATHER_UNITS];
  float s[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) s[t] = 0.f;
  const bool ab = gather_mt<GATHER_UNITS, MT, WD>(
      a, src, n / 4, a.ll_tok, slot, NWAVES, par, lane, Identity{},
      [&](int i, int, int u) { gv[i] = *reinterpret_cast<const uint2*>(gain + u * 4); },
      [&](int i, int t, int u, const f32x4 x) {
        *reinterpret_cast<f32x4*>(xres + t * xs + u * 4) = x;
        const f32x4 v = {x.x * bf16_lo(gv[i].x), x.y * bf16_hi(gv[i].x), x.z * bf16_lo(gv[i].y), x.w * bf16_hi(gv[i].y)};
        *reinterpret_cast<f32x4*>(vec + t * vs + vperm<Q8>(u * 4)) = v;
        const float q = x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
#pragma unroll
        for (int k = 0; k < MT; ++k) s[k] += t == k ? q : 0.f;
      });
#pragma unroll
  for (int t = 0; t < MT; ++t) ss[t] = wave_sum(s[t]);
  return ab;
}

// Multi-token steps: gather_plain for the MT positions in one polling loop (position t into
// dst + t * dstride)
template <bool WD, bool Q8, int MT>
__device__ __forceinline__ bool gather_plain_mt(const KernelArgs& a, float* dst, int dstride, const uint32_t* src, int n,
                                                int slot, int lane, uint32_t par, bool perm) {
  return gather_mt<GATHER_UNITS_PLAIN, MT, WD>(a, src, n / 4, a.ll_tok, slot, NWAVES, par, lane, Identity{},
                                               [&](int, int, int) {},
                                               [&](int, int t, int u, const f32x4 x) {
                                                 *reinterpret_cast<f32x4*>(dst + t * dstride +
                                                                           (perm ? vperm<Q8>(u * 4) : u * 4)) = x;
                                               });
}

// embedding row of `tok` (BF16, exact in FP32) -> xres, vec = x * gain (vperm order); returns the
// sum of squares
template <bool Q8>
__device__ __forceinline__ float stage_embedding(const KernelArgs& a, float* vec, float* xres, int tok, const uint16_t* gain,
                                                 int lane) {
  const uint16_t* erow = reinterpret_cast<const uint16_t*>(a.packed + a.embed_off + (int64_t)tok * a.embed_stride);
  constexpr int B = 8;
  float ss = 0.f;
  for (int base = 0; base < a.H; base += B * 256) {
    uint2 ev[B], gv[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int i = base + u * 256 + lane * 4;
      ev[u] = uint2{0u, 0u};
      gv[u] = uint2{0u, 0u};
      if (i < a.H) {
        ev[u] = *reinterpret_cast<const uint2*>(erow + i);
        gv[u] = *reinterpret_cast<const uint2*>(gain + i);
      }
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int i = base + u * 256 + lane * 4;
      if (i < a.H) {
        const f32x4 x = {bf16_lo(ev[u].x), bf16_hi(ev[u].x), bf16_lo(ev[u].y), bf16_hi(ev[u].y)};
        *reinterpret_cast<f32x4*>(xres + i) = x;
        const f32x4 v = {x.x * bf16_lo(gv[u].x), x.y * bf16_hi(gv[u].x), x.z * bf16_lo(gv[u].y), x.w * bf16_hi(gv[u].y)};
        *reinterpret_cast<f32x4*>(vec + vperm<Q8>(i)) = v;
        ss += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
      }
    }
  }
  return wave_sum(ss);
}

// Next token: reduce the W LM-head partials (value, index | parity << 31) of the step with
// parity `par`, greater value first, lower index on ties.  Returns true when abandoned.
// (Multi-token steps: the partials of position t of the step, at lmpart + t * W * 2.)
template <bool WD>
__device__ __forceinline__ bool gather_token(const KernelArgs& a, int lane, uint32_t par, int& tok, int t = 0) {
  constexpr int B = 4;  // up to 4 x 128 workers
  const __amdgpu_buffer_rsrc_t r = rsrc(a.lmpart + (int64_t)t * a.W * 2);
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  uint32_t pending = 0;
#pragma unroll
  for (int u = 0; u < B; ++u)
    if (u * 128 + lane * 2 < a.W) pending |= 1u << u;
  uint32_t spins = 0;
  for (;;) {
    u32x4 pv[B];
    COMPILER_FENCE();
#pragma unroll
    for (int u = 0; u < B; ++u) {
      pv[u] = u32x4{0u, 0u, 0u, 0u};
      if ((pending >> u) & 1u) pv[u] = cld4(r, (uint32_t)(u * 128 + lane * 2) * 8u);
    }
    COMPILER_FENCE();
#pragma unroll
    for (int u = 0; u < B; ++u) {
      if (!((pending >> u) & 1u)) continue;
      const int w = u * 128 + lane * 2;
      const bool two = w + 1 < a.W;
      const bool ok = (pv[u].y >> 31) == par && (!two || (pv[u].w >> 31) == par);
      if (!ok) continue;
      pending &= ~(1u << u);
      for (int e = 0; e < (two ? 2 : 1); ++e) {
        const float v = __uint_as_float(e ? pv[u].z : pv[u].x);
        const int ix = (int)((e ? pv[u].w : pv[u].y) & 0x7fffffffu);
        if (v > best || (v == best && ix < bidx)) {
          best = v;
          bidx = ix;
        }
      }
    }
    if (__all(pending == 0)) break;
    if (watch_tick<WD>(a, spins, lane)) return true;
  }
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(best, off);
    const int oi = __shfl_xor(bidx, off);
    if (ov > best || (ov == best && oi < bidx)) {
      best = ov;
      bidx = oi;
    }
  }
  if (bidx < 0 || bidx >= a.V) bidx = 0;  // only reachable with non-finite logits
  tok = bidx;
  // The acquire side of the per-step all-to-all: having seen every worker's (released) partial of
  // the step, this worker sees every store any worker made in that step, so one parity bit separates
  // generations -- when a consumer polls a buffer at step s + 2, the buffer already shows step s + 1's
  // value (the other parity) or a newer one, never step s's (nor, at step 1, the fill value).  No
  // cache invalidation is needed for that: every later load of another worker's data is issued after
  // these loads returned and either reads the device-coherent level (the polls) or is a KV row that no
  // worker read before it was written in this launch (see load_kv); only the compiler must not move
  // loads above this point.
  COMPILER_FENCE();
  return false;
}

// ---------------------------------------------------------------------------
// sampled decoding (top-k / top-p): every worker publishes its top_k logits; every worker then
// merges all W lists and draws the same token with the step's uniform
// ---------------------------------------------------------------------------

// A candidate as one 64-bit key: larger logit first, then lower token id (the order of ranking and
// of ties); 0 stands for "none" (no real candidate has key 0: its low word ~id is >= 2^31).
__device__ __forceinline__ uint64_t cand_key(float v, int idx) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;  // -0 ranks as +0
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint32_t)~(uint32_t)idx;
}
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t b = (uint32_t)(k >> 32);
  return __uint_as_float((b & 0x80000000u) ? (b & 0x7fffffffu) : ~b);
}
__device__ __forceinline__ int key_index(uint64_t k) { return (int)~(uint32_t)k; }
__device__ __forceinline__ uint64_t key_max(uint64_t a, uint64_t b) { return a > b ? a : b; }
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t xor16_64(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  const auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  const bool up = (lane >> 4) & 1;
  return ((uint64_t)(up ? b[0] : b[1]) << 32) | (up ? a[0] : a[1]);
}
__device__ __forceinline__ uint64_t xor32_64(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  const auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  const bool up = lane >= 32;
  return ((uint64_t)(up ? b[0] : b[1]) << 32) | (up ? a[0] : a[1]);
}
// the largest key of the wavefront, in every lane
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k, int lane) {
  k = key_max(k, dpp64<DPP_XOR1>(k));
  k = key_max(k, dpp64<DPP_XOR2>(k));
  k = key_max(k, dpp64<DPP_HALF_MIRROR>(k));
  k = key_max(k, dpp64<DPP_MIRROR>(k));
  k = key_max(k, xor16_64(k, lane));
  return key_max(k, xor32_64(k, lane));
}

// The K largest of a running list (lane i holds its i-th entry, 0 if none) and this lane's NC
// candidates c[] (0 = none): K rounds of a wavefront maximum, each removing its winner.
template <int NC>
__device__ __forceinline__ void topk_merge(uint64_t& run, uint64_t (&c)[NC], int K, int lane) {
  uint64_t nk = 0;
  for (int r = 0; r < K; ++r) {
    uint64_t m = run;
#pragma unroll
    for (int j = 0; j < NC; ++j) m = key_max(m, c[j]);
    const uint64_t w = wave_max_key(m, lane);
    if (w == 0) break;  // (uniform) nothing left
    if (run == w) run = 0;
#pragma unroll
    for (int j = 0; j < NC; ++j) c[j] = c[j] == w ? 0 : c[j];
    nk = lane == r ? w : nk;
  }
  run = nk;
}

// Poll the W x top_k candidate words of the step with parity `par` (value bits, id | parity << 31)
// into LDS (from L.vec on, in worker-major order): one wavefront, GB 16-byte units per lane in
// flight.  Returns true when the wait was abandoned.
template <bool WD>
__device__ __forceinline__ bool poll_candidates(const KernelArgs& a, const Lds& L, int lane, uint32_t par) {
  constexpr int GB = 16;
  constexpr int slot = 0, nslots = 1;
  const int nwords = a.W * a.top_k;
  const int nunits = (nwords + 1) / 2;
  const __amdgpu_buffer_rsrc_t r = rsrc(a.lmpart);
  for (int base = 0; base < nunits; base += GB * nslots * 64) {
    uint32_t pending = 0;
#pragma unroll
    for (int i = 0; i < GB; ++i)
      if (base + (i * nslots + slot) * 64 + lane < nunits) pending |= 1u << i;
    uint32_t spins = 0;
    for (;;) {
      u32x4 v[GB];
      COMPILER_FENCE();
#pragma unroll
      for (int i = 0; i < GB; ++i) {
        v[i] = u32x4{0u, 0u, 0u, 0u};
        if ((pending >> i) & 1u) v[i] = cld4(r, (uint32_t)(base + (i * nslots + slot) * 64 + lane) * 16u);
      }
      COMPILER_FENCE();
#pragma unroll
      for (int i = 0; i < GB; ++i) {
        const int u = base + (i * nslots + slot) * 64 + lane;
        const bool two = 2 * u + 1 < nwords;
        if (((pending >> i) & 1u) && (v[i].y >> 31) == par && (!two || (v[i].w >> 31) == par)) {
          *reinterpret_cast<u32x4*>(L.vec + 4 * u) = v[i];
          pending &= ~(1u << i);
        }
      }
      if (__all(pending == 0)) break;
      if (watch_tick<WD>(a, spins, lane)) return true;
    }
  }
  return false;
}

// The sampled token from the candidates in LDS (control wavefront, after poll_candidates): the W
// sorted lists merged into the global top_k (K rounds of a wavefront maximum over the list heads;
// lane l merges lists l, l + 64, l + 128, l + 192), then the top-k / temperature / top-p draw with
// the uniform u, in FP32, the running sums taken in ranking order.
__device__ __forceinline__ int draw_token(const KernelArgs& a, const Lds& L, int lane, float u) {
  constexpr int NL = 4;  // W <= 256
  const int K = a.top_k;
  auto load = [&](int w, int i) -> uint64_t {
    if (w >= a.W || i >= K) return 0;
    const uint2 c = *reinterpret_cast<const uint2*>(L.vec + 2 * (w * K + i));
    return cand_key(__uint_as_float(c.x), (int)(c.y & 0x7fffffffu));
  };
  int ptr[NL];
  uint64_t head[NL], next[NL];
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    ptr[q] = 0;
    head[q] = load(lane + 64 * q, 0);
    next[q] = load(lane + 64 * q, 1);
  }
  uint64_t mine = 0;  // lane r: the r-th largest candidate
  for (int r = 0; r < K; ++r) {
    uint64_t m = head[0];
#pragma unroll
    for (int q = 1; q < NL; ++q) m = key_max(m, head[q]);
    const uint64_t w = wave_max_key(m, lane);
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      if (w != 0 && head[q] == w) {
        head[q] = next[q];
        ++ptr[q];
        next[q] = load(lane + 64 * q, ptr[q] + 1);
      }
    }
    mine = lane == r ? w : mine;
  }
  const bool valid = lane < K && mine != 0;
  const float z = valid ? key_value(mine) : 0.f;
  const float z0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), 0));
  const float wgt = valid ? expf((z - z0) / a.temperature) : 0.f;
  float run = 0.f, cum = 0.f;
  for (int r = 0; r < K; ++r) {
    run += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), r));
    cum = lane == r ? run : cum;
  }
  const int nvalid = __popcll(__ballot(valid));
  // the shortest prefix whose sum reaches top_p of the total (at least one candidate)
  const float need = a.top_p * run;
  int n = __popcll(__ballot(valid && cum < need)) + 1;
  n = n < nvalid ? n : nvalid;
  if (n < 1) n = 1;
  const float pref = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), n - 1));
  u = fminf(fmaxf(u, 0.f), 0x1.fffffep-1f);  // [0, 1); NaN -> 0
  const float target = u * pref;
  int pos = __popcll(__ballot(lane < n && cum <= target));  // the first prefix entry whose sum exceeds it
  pos = pos < n ? pos : n - 1;
  const uint64_t pick = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mine >> 32), pos) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mine, pos);
  int tok = pick ? key_index(pick) : 0;
  if (tok < 0 || tok >= a.V) tok = 0;  // only reachable with non-finite logits
  // the acquire side of the per-step all-to-all, as for the greedy token (see gather_token)
  COMPILER_FENCE();
  return tok;
}

// ---------------------------------------------------------------------------
// compute wave: weight streaming.  Each compute wave reads its share of a GEMV block (a
// contiguous chunk range) with 16-byte loads into registers, in batches of STREAM_BATCH
// chunks that rotate through a ring of NB register sets: while one batch is consumed the
// other NB - 1 are in flight (the per-wave depth sets how many bytes a compute unit keeps in
// flight, and so its share of the HBM bandwidth).  The reloads issued after a range's last
// batches fetch the first NB batches of the wave's next range -- the next block, the next GEMV
// tile or the (K, V) rows of
// its next attention split -- so those bytes arrive while the workgroup publishes this tile's
// outputs and gathers the next inputs: weights (and cached KV rows) do not depend on
// activations, only the dot products do (the Tiles page credits this prefetch idea to the
// megakernel it builds on).
//
// Every load of these loops is issued unconditionally (addresses clamped into the range, or a
// dummy chunk when there is nothing to fetch) and the bounds are wave-uniform: that lets the
// compiler count outstanding loads exactly; loads behind per-slot branches make it wait for
// all of them before the first use.
// ---------------------------------------------------------------------------


// Trace stamps of the first compute wavefront, kept in LDS (a global store would hold up the
// wavefront's next wait on its loads, which counts stores too) and written out by the control
// wavefront after barrier B.
enum { TS_GATHERED, TS_AFTER_A, TS_ENTRY, TS_FIRST, TS_DONE, TS_COUNT };
__device__ __forceinline__ void stamp(uint64_t* ts, int i, int lane) {
  if (ts && lane == 0) ts[i] = wall_clock64();
}

__device__ __forceinline__ float dot8(const u32x4 w, const float* v) {
  const f32x4 v0 = *reinterpret_cast<const f32x4*>(v);
  const f32x4 v1 = *reinterpret_cast<const f32x4*>(v + 4);
  float s0 = bf16_lo(w.x) * v0.x;
  float s1 = bf16_hi(w.x) * v0.y;
  s0 = fmaf(bf16_lo(w.y), v0.z, s0);
  s1 = fmaf(bf16_hi(w.y), v0.w, s1);
  s0 = fmaf(bf16_lo(w.z), v1.x, s0);
  s1 = fmaf(bf16_hi(w.z), v1.y, s1);
  s0 = fmaf(bf16_lo(w.w), v1.z, s0);
  s1 = fmaf(bf16_hi(w.w), v1.w, s1);
  return s0 + s1;
}

// 16 INT8 codes (one 16-byte load, weight-only INT8 tiles) times 16 FP32 inputs: the codes are
// converted in registers and the row's scale is applied once to the row's total (by the control
// wavefront).
__device__ __forceinline__ float i8(uint32_t x, int k) { return (float)(int8_t)(uint8_t)(x >> (8 * k)); }
__device__ __forceinline__ float dot16_i8(const u32x4 w, const float* v) {
  const f32x4 v0 = *reinterpret_cast<const f32x4*>(v);
  const f32x4 v1 = *reinterpret_cast<const f32x4*>(v + 4);
  const f32x4 v2 = *reinterpret_cast<const f32x4*>(v + 8);
  const f32x4 v3 = *reinterpret_cast<const f32x4*>(v + 12);
  float s0 = i8(w.x, 0) * v0.x;
  float s1 = i8(w.x, 1) * v0.y;
  s0 = fmaf(i8(w.x, 2), v0.z, s0);
  s1 = fmaf(i8(w.x, 3), v0.w, s1);
  s0 = fmaf(i8(w.y, 0), v1.x, s0);
  s1 = fmaf(i8(w.y, 1), v1.y, s1);
  s0 = fmaf(i8(w.y, 2), v1.z, s0);
  s1 = fmaf(i8(w.y, 3), v1.w, s1);
  s0 = fmaf(i8(w.z, 0), v2.x, s0);
  s1 = fmaf(i8(w.z, 1), v2.y, s1);
  s0 = fmaf(i8(w.z, 2), v2.z, s0);
  s1 = fmaf(i8(w.z, 3), v2.w, s1);
  s0 = fmaf(i8(w.w, 0), v3.x, s0);
  s1 = fmaf(i8(w.w, 1), v3.y, s1);
  s0 = fmaf(i8(w.w, 2), v3.z, s0);
  s1 = fmaf(i8(w.w, 3), v3.w, s1);
  return s0 + s1;
}

// Chunk range [i, ihi) of compute wave c in block r0 of a GEMV segment.
struct Range {
  int k;         // schedule wave (-1: none)
  int r0;        // first row of the block
  int C;         // chunks per row
  int i, ihi;
  int64_t base;  // byte offset of the block's first chunk
};

// (Values read from LDS are per-lane to the compiler; readfirstlane makes the bounds scalar.)
__device__ __forceinline__ Range block_range(const SegDesc& s, int k, int r0, int block_rows, int c) {
  Range r;
  r.k = k;
  r.r0 = r0;
  const int cpr = __builtin_amdgcn_readfirstlane(s.chunks_per_row);
  const int rows = __builtin_amdgcn_readfirstlane(s.rows);
  const int64_t woff = ((int64_t)__builtin_amdgcn_readfirstlane((int)(s.woff >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)s.woff);
  r.C = cpr;
  const int nr = min(block_rows, rows - r0);
  const int n = nr * cpr;
  r.i = chunk_lo(n, c);
  r.ihi = chunk_lo(n, c + 1);
  r.base = woff + (int64_t)r0 * cpr * CHUNK_BYTES;
  return r;
}

__device__ __forceinline__ Range no_range() {
  Range r;
  r.k = -1;
  r.r0 = 0;
  r.C = 1;
  r.i = r.ihi = 0;
  r.base = 0;
  return r;
}

// First block of the next GEMV wave after `k` (wrapping into the next step) in which compute
// wave c has chunks; k = -1 when there is none.
__device__ __forceinline__ Range next_gemv(const SegDesc* segs, int n_waves, int k, int block_rows, int c) {
  for (int d = 1; d <= n_waves; ++d) {
    const int kk = (k + d) % n_waves;
    if (segs[kk].rows == 0) continue;
    const Range r = block_range(segs[kk], kk, 0, block_rows, c);
    if (r.i < r.ihi) return r;
  }
  return no_range();
}

// The NB batch register sets of a compute wave: batch slot h = v[h * B, (h + 1) * B).
template <int B, int NB>
struct Stream {
  u32x4 v[NB * B];
  int k;   // wave whose data the registers hold (-1: none)
  int r0;  // GEMV block of that wave
  int sk;  // wave whose first block has batches NB .. NB + ls staged in the wave's LDS area (-1: none)
  int ls;
};

// Source of the B loads of one batch: per slot a buffer descriptor, a per-lane byte offset and a
// wave-uniform byte offset.  The loads themselves are always the same instruction sequence;
// only these operands are selected (uniformly, without branches) between the sources.
template <int B>
struct BatchSrc {
  __amdgpu_buffer_rsrc_t d[B];
  uint32_t vo[B];
  uint32_t so[B];
};

// Batch q of GEMV range r: chunks r.i + q*B + u, clamped to the range's last chunk (a range
// with no chunks reads the first KB of the packed buffer).
template <int B>
__device__ __forceinline__ BatchSrc<B> gemv_src(const uint8_t* packed, const Range& r, int q, int lane) {
  BatchSrc<B> b;
  const bool any = r.i < r.ihi;
  const __amdgpu_buffer_rsrc_t rs = rsrc(packed + (any ? r.base : 0));
#pragma unroll
  for (int u = 0; u < B; ++u) {
    const int j = r.i + q * B + u;
    const int jc = any ? (j < r.ihi ? j : r.ihi - 1) : 0;
    b.d[u] = rs;
    b.vo[u] = (uint32_t)lane * 16u;
    b.so[u] = (uint32_t)jc * CHUNK_BYTES;
  }
  return b;
}

template <int B>
__device__ __forceinline__ BatchSrc<B> select_src(bool first, const BatchSrc<B>& x, const BatchSrc<B>& y) {
  BatchSrc<B> b;
#pragma unroll
  for (int u = 0; u < B; ++u) {
    b.d[u] = first ? x.d[u] : y.d[u];
    b.vo[u] = first ? x.vo[u] : y.vo[u];
    b.so[u] = first ? x.so[u] : y.so[u];
  }
  return b;
}

// Non-temporal 16-byte loads for every stream (weights and KV rows alike; see load_kv for why
// that is coherent for KV rows): one load form for all sources.
template <int B>
__device__ __forceinline__ void load_batch(u32x4* w, const BatchSrc<B>& b) {
#pragma unroll
  for (int u = 0; u < B; ++u) w[u] = __builtin_amdgcn_raw_buffer_load_b128(b.d[u], b.vo[u], b.so[u], NT);
}

template <int B>
__device__ __forceinline__ void load_gemv_batch(u32x4* w, const uint8_t* packed, const Range& r, int q, int lane) {
  load_batch<B>(w, gemv_src<B>(packed, r, q, lane));
}

// Batch q of GEMV range r (chunks clamped into the range, as in gemv_src) straight into LDS at
// byte address lds + u * CHUNK_BYTES for slot u: gfx950's 16-byte direct-to-LDS load puts lane i's
// 16 bytes at M0 + 16 i, so a staged chunk has the same lane layout as a register batch.  The
// compiler does not see these loads: a consumer waits for them explicitly (they complete in issue
// order with the wavefront's other vector-memory loads).
template <int B>
__device__ __forceinline__ void stage_batch(const uint8_t* packed, const Range& r, int q, int lane, uint32_t lds) {
  const uint8_t* base = packed + r.base + (uint32_t)lane * 16u;
#pragma unroll
  for (int u = 0; u < B; ++u) {
    const int j = r.i + q * B + u;
    const int jc = j < r.ihi ? j : r.ihi - 1;
    const uint8_t* g = base + (int64_t)jc * CHUNK_BYTES;
    const uint32_t dst = lds + u * CHUNK_BYTES;
    uint32_t saved;  // M0 is the compiler's: kept across the statement
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt\n\ts_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(dst)
        : "memory");
  }
}
// One 4-byte direct-to-LDS load per lane: lane i's word lands at LDS byte address lds + 4 i (lanes
// outside EXEC write nothing).  Like the 16-byte form, it is invisible to the compiler: a consumer
// waits for it explicitly.
__device__ __forceinline__ void stage_dword(const float* g, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds)
      : "memory");
}
// Stage batches NB .. NB + n of GEMV range r (n = what the range has beyond its first NB
// batches, at most `limit`); returns n.  The area's previous contents must have been read.
template <int B, int NB>
__device__ __forceinline__ int stage_range(const uint8_t* packed, const Range& r, int limit, int lane, uint32_t lds) {
  if (limit <= 0 || r.i >= r.ihi) return 0;
  const int nb = (r.ihi - r.i + B - 1) / B;
  const int n = nb - NB < limit ? (nb - NB > 0 ? nb - NB : 0) : limit;
  if (n > 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // earlier reads of the area have completed
  for (int t = 0; t < n; ++t) stage_batch<B>(packed, r, NB + t, lane, lds + t * B * CHUNK_BYTES);
  return n;
}

// s_waitcnt with only the vector-memory count N enforced (gfx9 encoding: vmcnt[3:0] in bits
// 3:0 and vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Consume chunks [r.i, r.ihi) in batches; st holds batches 0 .. NB - 1 when `have` (else they
// are loaded first).  Per-row partial sums go to part[row * NCOMP + c].  The reloads after the
// last NB batches fetch next_src(0) .. next_src(NB - 1) into the NB register sets.
// Q8: the chunks hold INT8 codes (16 per lane, 1024 columns) instead of BF16 weights (8, 512).
// MT > 1 (multi-token steps): every chunk is multiplied with the MT input vectors of the step (vs
// floats apart in LDS), and row partials of position t go to part[t * pt + row * NCOMP + c].
template <int B, int NB, bool Q8, int MT, typename NextSrc>
__device__ __forceinline__ void stream_range(const Lds& L, const uint8_t* packed, const Range& r, int c, int lane,
                                             Stream<B, NB>& st, bool have, NextSrc next_src, const float* stage,
                                             uint64_t* ts, int vs, int pt) {
  constexpr int VPL = Q8 ? 16 : 8;            // input values per lane per chunk
  constexpr int CC = chunk_cols<Q8>();
  const int C = r.C;
  const int i = r.i;
  const int ihi = r.ihi;
  int row = i / C, seg = i - row * C;
  float acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = 0.f;
  const float* vlane = L.vec + lane * 4;  // group q of this lane's columns of chunk s: vlane[s * CC + 256 q] (vperm)
  // Every slot is consumed (a slot past the range contributes zero and does not advance the
  // row), so no branch sits between a load and the use of its registers.
  auto consume = [&](const u32x4& w, bool valid, const float* xv) {  // xv: [MT][VPL]
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float d = Q8 ? dot16_i8(w, xv + t * VPL) : dot8(w, xv + t * VPL);
      acc[t] += valid ? d : 0.f;
    }
    seg += valid ? 1 : 0;
    if (seg == C) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const float s = wave_sum(acc[t]);
        if (lane == 0) L.part[t * pt + row * NCOMP + c] = s;
        acc[t] = 0.f;
      }
      seg = 0;
      ++row;
    }
  };
  // The input-vector slices of a batch's chunks are read from LDS before any of them is used,
  // so their latencies overlap (the row-end branches would otherwise serialise them).  A slot
  // past the range reads a slice too (in bounds, masked).
  auto consume_batch = [&](const u32x4* w, int jb) {
    float xv[B][MT * VPL];
    int s = seg;
#pragma unroll
    for (int u = 0; u < B; ++u) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const float* px = vlane + t * vs + s * CC;
#pragma unroll
        for (int q = 0; q < VPL / 4; ++q) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(px + 256 * q);
          float* xo = xv[u] + t * VPL + 4 * q;
          xo[0] = x.x; xo[1] = x.y; xo[2] = x.z; xo[3] = x.w;
        }
      }
      s = s + 1 == C ? 0 : s + 1;
    }
#pragma unroll
    for (int u = 0; u < B; ++u) consume(w[u], jb + u < ihi, xv[u]);
  };
  // Batches 0 .. NB - 1 come from the register sets, batches NB .. NB + ls from the wave's LDS
  // area (staged while the tile's inputs were outstanding), the rest stream through the register
  // sets again: register batch q is batch rb(q).
  const int ls = st.sk == r.k && r.r0 == 0 ? st.ls : 0;
  const int nb = (ihi - i + B - 1) / B;
  const int nrb = nb - ls;
  const int nbe = (nrb + NB - 1) / NB * NB;  // whole ring passes: the last NB reloads fetch what follows
  auto rb = [&](int q) { return q < NB ? q : q + ls; };
  const float* stg = stage + lane * 4;
  auto consume_staged = [&]() {
    if (ls > 0) {
      // the staging loads were issued before the NB * B reloads of the first ring pass, the last
      // vector-memory instructions: once at most NB * B are outstanding, they have landed
      wait_vmcnt<NB * B>();
      for (int t = 0; t < ls; ++t) {
        u32x4 w[B];
#pragma unroll
        for (int u = 0; u < B; ++u) w[u] = *reinterpret_cast<const u32x4*>(stg + (t * B + u) * (CHUNK_BYTES / 4));
        consume_batch(w, i + (NB + t) * B);
      }
    }
  };
  if (!have) {
#pragma unroll
    for (int h = 0; h < NB; ++h) load_gemv_batch<B>(st.v + h * B, packed, r, h, lane);
  }
  stamp(ts, TS_ENTRY, lane);
  int b = 0;
  for (; b + NB < nbe; b += NB) {
#pragma unroll
    for (int h = 0; h < NB; ++h) {
      consume_batch(st.v + h * B, i + rb(b + h) * B);
      load_gemv_batch<B>(st.v + h * B, packed, r, rb(b + h + NB), lane);
      __builtin_amdgcn_sched_barrier(0);  // keep each reload ahead of the next slot's consumption
      if (b == 0 && h == 0) stamp(ts, TS_FIRST, lane);
    }
    if (b == 0) consume_staged();
  }
  // the last ring pass: its reloads fetch what follows the range
#pragma unroll
  for (int h = 0; h < NB; ++h) {
    consume_batch(st.v + h * B, i + rb(b + h) * B);
    load_batch<B>(st.v + h * B, next_src(h));
    __builtin_amdgcn_sched_barrier(0);
    if (b == 0 && h == 0) stamp(ts, TS_FIRST, lane);
  }
  if (b == 0) consume_staged();
  if (ls > 0) st.sk = -1;
  if (seg != 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const float s = wave_sum(acc[t]);
      if (lane == 0) L.part[t * pt + row * NCOMP + c] = s;
    }
  }
}

// total of row r of a block: partials of the compute waves whose ranges touch it, in order.
// Every slot of the row is read (independent loads); those of waves that did not write it are
// dropped by a select.
__device__ __forceinline__ float row_total(const float* part, int nr, int C, int r) {
  const int n = nr * C;
  const int first = r * C, last = r * C + C - 1;
  float v[NCOMP];
#pragma unroll
  for (int c = 0; c < NCOMP; ++c) v[c] = part[r * NCOMP + c];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCOMP; ++c) {
    const int lo = chunk_lo(n, c), hi = chunk_lo(n, c + 1);
    s += (lo < hi && lo <= last && first < hi) ? v[c] : 0.f;
  }
  return s;
}

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------

// Split partial record of one query head: m, l, acc[HD], two pad words (16-byte units).
template <int HD>
constexpr int pstride() { return HD + 4; }

// merge the S splits of one query head (Ph -> [S][HD + 4]) for output dim d, fixed split order
// Merge the S split partials (m, l, acc[HD], pad) of heads [0, nh) -- head h's at
// part + h * S * (HD + 4) -- into out[h * HD + d]: acc weighted by 2^(m_s - max m) over the
// weighted l ("Tiles", split-KV attention combine).  Each thread takes four consecutive
// dimensions of one head; a split's (m, l) pair and accumulator slice are read with
// independent loads, and both loops over the splits are unrolled, so the LDS latencies overlap.  Empty splits (l = 0) carry no weight; a head
// with no positions gives 0.  `perm`: out is a GEMV input (vperm order).
template <int HD, bool Q8>
__device__ __forceinline__ void merge_heads(const float* part, int nh, int S, int tid, float* out, bool perm) {
  constexpr int PS = pstride<HD>();
  for (int o = tid * 4; o < nh * HD; o += BLOCK_THREADS * 4) {
    const int h = o / HD, d = o % HD;
    const float* P = part + h * S * PS;
    float mm = -INFINITY;
#pragma unroll 4
    for (int sp = 0; sp < S; ++sp) {
      // (m, l) as one 8-byte read (the compiler would read l, branch, then read m)
      const uint2 ml = *reinterpret_cast<const uint2*>(P + sp * PS);
      mm = __uint_as_float(ml.y) > 0.f ? fmaxf(mm, __uint_as_float(ml.x)) : mm;
    }
    float ll = 0.f, a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 4
    for (int sp = 0; sp < S; ++sp) {
      const float* st = P + sp * PS;
      const float2 ml = *reinterpret_cast<const float2*>(st);
      const float2 v01 = *reinterpret_cast<const float2*>(st + 2 + d);
      const float2 v23 = *reinterpret_cast<const float2*>(st + 4 + d);
      const float f = ml.y > 0.f ? __builtin_amdgcn_exp2f(ml.x - mm) : 0.f;
      ll = fmaf(f, ml.y, ll);
      a0 = fmaf(f, v01.x, a0);
      a1 = fmaf(f, v01.y, a1);
      a2 = fmaf(f, v23.x, a2);
      a3 = fmaf(f, v23.y, a3);
    }
    const float inv = ll > 0.f ? 1.0f / ll : 0.f;
    *reinterpret_cast<f32x4*>(out + (perm ? vperm<Q8>(o) : o)) = f32x4{a0 * inv, a1 * inv, a2 * inv, a3 * inv};
  }
}

// Attention tile LDS layout (inside `part`): q[G][HD] (normed, roped, scaled to the base-2
// domain) | kc[HD] (normed, roped, BF16-rounded) | vc[HD] (BF16-rounded) | compute-wave states
// [NCOMP][G][HD + 4] | merged partial [G][HD + 4].  The raw q/k/v are gathered into `vec`.
// Multi-token steps (MT positions): q holds MT * G rows, row t * G + h being query head h at
// position t of the step, and kc / vc one row per position: q[MT * G][HD] | kc[MT][HD] |
// vc[MT][HD] | states [NCOMP][MT * G][HD + 4] | merged [MT * G][HD + 4]; position t's raw q/k/v
// are at vec + t * lds_vec_floats.
template <int HD, int G, int MT = 1>
__device__ __forceinline__ float* attn_ws(const Lds& L) { return L.part + MT * G * HD + 2 * MT * HD; }
template <int HD, int G, int MT = 1>
__device__ __forceinline__ float* attn_merged(const Lds& L) { return attn_ws<HD, G, MT>(L) + NCOMP * MT * G * pstride<HD>(); }
// INT8 KV: the split's K scales, then its V scales (kv8_span positions apart: the plan's longest
// split, rounded up to 64), by position - split start
template <int HD, int G, int MT = 1>
__device__ __forceinline__ float* attn_kscales(const Lds& L) { return attn_merged<HD, G, MT>(L) + MT * G * pstride<HD>(); }

// The (cos, sin) RoPE rows of an attention tile: the current position's in the small area (one-position
// steps), or one row per position of a multi-token step after the tile's work areas (and, INT8 KV,
// after the split's scales).
template <int HD, int G, bool KV8, int MT>
__device__ __forceinline__ float* rope_rows(const Lds& L, int kv8_span) {
  return MT == 1 ? L.small + SM_ROPE : attn_kscales<HD, G, MT>(L) + (KV8 ? 2 * kv8_span : 0);
}

// The split [lo, hi) that split sp of S covers at attended length L_att (positions < 2^31).
__device__ __forceinline__ void split_bounds(int S, int sp, int L_att, int& lo, int& hi) {
  const int ch = (int)((uint32_t)(L_att + S - 1) / (uint32_t)S);
  lo = sp * ch;
  hi = lo + ch < L_att ? lo + ch : L_att;
  if (lo > L_att) lo = L_att;
}

// INT8 KV: symmetric INT8 code of r at scale s (r / s rounded half to even, clamped; 0 when s = 0),
// the divisions correctly rounded
__device__ __forceinline__ float kv_code(float r, float s) {
  return s > 0.f ? fminf(fmaxf(rintf(__fdiv_rn(r, s)), -127.f), 127.f) : 0.f;
}

// all wavefronts: raw q (the tile's G query heads, from head qa), k, v of KV head g into vec from
// the QKV wave's output
template <int HD, int G, bool WD>
__device__ __forceinline__ bool gather_qkv(const KernelArgs& a, float* vec, const uint32_t* src, int g, int qa, int slot,
                                           int lane, uint32_t par) {
  constexpr int NQ = G * HD / 4, NK = HD / 4;
  const int q0 = qa * HD / 4;
  const int k0 = (a.n_heads * HD + g * HD) / 4;
  const int v0 = (a.n_heads * HD + a.n_kv * HD + g * HD) / 4;
  return gather<2, WD>(
      a, src, NQ + 2 * NK, slot, NWAVES, par, lane,
      [&](int u) { return u < NQ ? q0 + u : u < NQ + NK ? k0 + (u - NQ) : v0 + (u - NQ - NK); }, NoPrep{},
      [&](int, int u, const f32x4 x) { *reinterpret_cast<f32x4*>(vec + u * 4) = x; });
}

// Multi-token steps: gather_qkv for the MT positions in one polling loop (position t into vec + t * vs)
template <int HD, int G, bool WD, int MT>
__device__ __forceinline__ bool gather_qkv_mt(const KernelArgs& a, float* vec, int vs, const uint32_t* src, int g, int qa,
                                              int slot, int lane, uint32_t par) {
  constexpr int NQ = G * HD / 4, NK = HD / 4;
  const int q0 = qa * HD / 4;
  const int k0 = (a.n_heads * HD + g * HD) / 4;
  const int v0 = (a.n_heads * HD + a.n_kv * HD + g * HD) / 4;
  return gather_mt<2, MT, WD>(
      a, src, NQ + 2 * NK, a.ll_tok, slot, NWAVES, par, lane,
      [&](int u) { return u < NQ ? q0 + u : u < NQ + NK ? k0 + (u - NQ) : v0 + (u - NQ - NK); }, [&](int, int, int) {},
      [&](int, int t, int u, const f32x4 x) { *reinterpret_cast<f32x4*>(vec + t * vs + u * 4) = x; });
}

// all wavefronts, between barriers P and A: wave u < G normalises (optional) and rotates query
// head u, wave G the key; wave G + 1 rounds the value.  LDS only (plus read-only tables).
// INT8 KV (KV8): the query heads are also multiplied by the key smoothing factors (a score is then the
// key row's scale times the dot product of these with its codes), and the current K and V rows are
// quantized: kc / vc hold their codes, SM_KVCUR their scales (also put at the split's scale area
// when the split holds the current position, split sp).
// MT > 1: the same for every position t of the step (pos = its first position), each with its own
// RoPE row (and, INT8 KV, its own scales at SM_KVCUR + 2 t).
template <int HD, int G, bool KV8, int MT = 1>
__device__ __forceinline__ void attn_lds_prep(const KernelArgs& a, const Lds& L, int wave_index, int lane, int layer, int pos,
                                              int sp) {
  constexpr int HALF = HD / 2;
  float* q = L.part;
  float* kc = q + MT * G * HD;
  float* vc = kc + MT * HD;
  int slo = 0, shi = 0;
  if (KV8) split_bounds(a.S, sp, pos + MT, slo, shi);
  float* kss = attn_kscales<HD, G, MT>(L);
  float* vss = kss + a.kv8_span;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const bool own_cur = KV8 && slo <= pos + t && pos + t < shi;
    const float* raw = L.vec + t * a.lds_vec_floats;
    if (wave_index <= G) {
      const int u = wave_index;
      float u0 = 0.f, u1 = 0.f;
      if (lane < HALF) {
        u0 = raw[u * HD + lane];
        u1 = raw[u * HD + lane + HALF];
      }
      if (gain_off(L, layer, 2) >= 0) {
        const float ss = wave_sum(u0 * u0 + u1 * u1);
        const float rs = 1.0f / sqrtf(ss / (float)HD + a.eps);
        const float* gn = L.small + (u < G ? SM_QGAIN : SM_KGAIN);
        if (lane < HALF) {
          u0 = u0 * rs * gn[lane];
          u1 = u1 * rs * gn[lane + HALF];
        }
      }
      float r0 = 0.f, r1 = 0.f;
      if (lane < HALF) {
        const float* cs = rope_rows<HD, G, KV8, MT>(L, a.kv8_span) + t * HD + lane * 2;
        const float co = cs[0], si = cs[1];
        r0 = u0 * co - u1 * si;
        r1 = u1 * co + u0 * si;
      }
      if constexpr (KV8) {
        const float* sg = L.small + SM_KSMOOTH;
        if (u < G) {
          if (lane < HALF) {
            q[(t * G + u) * HD + lane] = r0 * a.qscale * sg[lane];
            q[(t * G + u) * HD + lane + HALF] = r1 * a.qscale * sg[lane + HALF];
          }
        } else {  // the key: smoothed, then quantized per row
          const float k0 = lane < HALF ? __fdiv_rn(r0, sg[lane]) : 0.f;
          const float k1 = lane < HALF ? __fdiv_rn(r1, sg[lane + HALF]) : 0.f;
          const float sk = __fdiv_rn(wave_max(fmaxf(fabsf(k0), fabsf(k1)), lane), 127.f);
          if (lane < HALF) {
            kc[t * HD + lane] = kv_code(k0, sk);
            kc[t * HD + lane + HALF] = kv_code(k1, sk);
          }
          if (lane == 0) {
            L.small[SM_KVCUR + 2 * t] = sk;
            if (own_cur) kss[pos + t - slo] = sk;
          }
        }
      } else if (lane < HALF) {
        if (u < G) {
          q[(t * G + u) * HD + lane] = r0 * a.qscale;
          q[(t * G + u) * HD + lane + HALF] = r1 * a.qscale;
        } else {
          kc[t * HD + lane] = bf16_round(r0);
          kc[t * HD + lane + HALF] = bf16_round(r1);
        }
      }
    } else if (wave_index == G + 1) {
      if constexpr (KV8) {
        constexpr int NV = (HD + 63) / 64;
        float v[NV], am = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          v[i] = lane + 64 * i < HD ? raw[(G + 1) * HD + lane + 64 * i] : 0.f;
          am = fmaxf(am, fabsf(v[i]));
        }
        const float sv = __fdiv_rn(wave_max(am, lane), 127.f);
#pragma unroll
        for (int i = 0; i < NV; ++i)
          if (lane + 64 * i < HD) vc[t * HD + lane + 64 * i] = kv_code(v[i], sv);
        if (lane == 0) {
          L.small[SM_KVCUR + 2 * t + 1] = sv;
          if (own_cur) vss[pos + t - slo] = sv;
        }
      } else {
        for (int i = lane; i < HD; i += 64) vc[t * HD + i] = bf16_round(raw[(G + 1) * HD + i]);
      }
    }
  }
}

// control wave, after barrier A: the split holding the current position writes its K/V row (the
// tile of the KV head's first query heads, when the heads are spread over several tiles).  MT > 1:
// the rows of the step's MT positions (L_att - MT .. L_att - 1), each by the split that holds it.
template <int HD, int G, bool KV8, int MT = 1>
__device__ __forceinline__ void cw_attn_kv_write(const KernelArgs& a, const Lds& L, int lane, int layer, int g, int sp,
                                 int qa, int64_t L_att) {
  if (qa != g * (a.n_heads / a.n_kv)) return;
  const float* kc0 = L.part + MT * G * HD;
  const float* vc0 = kc0 + MT * HD;
  const int64_t ch = (L_att + a.S - 1) / a.S;
  const int64_t lo = (int64_t)sp * ch;
  const int64_t hi = lo + ch < L_att ? lo + ch : L_att;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const float* kc = kc0 + t * HD;
    const float* vc = vc0 + t * HD;
    const int64_t cur = L_att - MT + t;
    if (KV8 && lo <= cur && cur < hi) {  // the interleaved codes, four per lane, and the two scales
      const int64_t row = ((int64_t)layer * a.n_kv + g) * a.kv_cap + cur;
      if (lane < HD / 2) {
        // word `lane` of the row: group lane / 4 of 8 dimensions, its K codes in words 0-1, V in 2-3
        const int grp = lane >> 2, part = lane & 3;
        const float* c = (part < 2 ? kc : vc) + grp * 8 + (part & 1) * 4;
        const uint32_t w = ((uint32_t)(uint8_t)(int8_t)(int)c[0]) | ((uint32_t)(uint8_t)(int8_t)(int)c[1] << 8) |
                           ((uint32_t)(uint8_t)(int8_t)(int)c[2] << 16) | ((uint32_t)(uint8_t)(int8_t)(int)c[3] << 24);
        st_u32(reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.kv_k) + row * HD * 2) + lane, w);
      }
      if (lane == 0) {
        st_u32(reinterpret_cast<uint32_t*>(a.kv_ks + row), __float_as_uint(L.small[SM_KVCUR + 2 * t]));
        st_u32(reinterpret_cast<uint32_t*>(a.kv_vs + row), __float_as_uint(L.small[SM_KVCUR + 2 * t + 1]));
      }
    } else if (!KV8 && lo <= cur && cur < hi && lane < HD / 2) {
      const int64_t row = ((int64_t)layer * a.n_kv + g) * a.kv_cap + cur;
      const uint32_t kb = f32_to_bf16_bits(kc[2 * lane]) | (f32_to_bf16_bits(kc[2 * lane + 1]) << 16);
      const uint32_t vb = f32_to_bf16_bits(vc[2 * lane]) | (f32_to_bf16_bits(vc[2 * lane + 1]) << 16);
      st_u32(reinterpret_cast<uint32_t*>(a.kv_k + row * HD) + lane, kb);
      st_u32(reinterpret_cast<uint32_t*>(a.kv_v + row * HD) + lane, vb);
    }
  }
}

// Positions [wlo, whi) of a split that compute wave c handles at attended length L_att.
// Positions are below 2^31 (the planner bounds the cache capacity), so 32-bit arithmetic.
struct AttnRange {
  int wlo, whi;
  int lo;  // the split's first position
};
__device__ __forceinline__ AttnRange attn_range(const KernelArgs& a, int sp, int c, int64_t L_att64) {
  const int L_att = (int)L_att64;
  const int S = a.S;
  const int ch = (int)((uint32_t)(L_att + S - 1) / (uint32_t)S);
  int lo = sp * ch;
  const int hi = lo + ch < L_att ? lo + ch : L_att;
  if (lo > L_att) lo = L_att;
  const int n = hi > lo ? hi - lo : 0;
  AttnRange r;
  r.lo = lo;
  r.wlo = lo + (int)((uint32_t)(n * c) / NCOMP);
  r.whi = lo + (int)((uint32_t)(n * (c + 1)) / NCOMP);
  return r;
}

// K and V of position j of KV head (layer, g) for this lane's 16-byte segment.  Every stream
// of the compute waves (weights and KV rows alike) uses the same non-temporal 16-byte load, so
// that one instruction sequence serves whichever source a batch comes from.  That is coherent
// for KV rows because, within a launch, no row is read before this launch writes it: real
// reads only touch positions before the current one (written in earlier steps, completed
// before any output this worker's readers depend on), and a slot that has no position -- past
// the range, or the current position, taken from LDS -- reads the cache's last row
// (capacity - 1) instead, which is never read for real (a position is read only in later
// steps, and none follows the last one); rows from earlier launches are covered by the cache
// maintenance at kernel boundaries.  The consumer discards what such a slot read (its weight
// and V values are selected away, not multiplied by 0), so that row's contents never matter:
// it may hold anything, NaN included.
// Lanes per position: a lane's 16-byte load holds 8 dimensions of a position -- 8 BF16 values of a K
// or a V row, or (INT8 KV) 8 K codes followed by the same 8 dimensions' V codes (the INT8 cache
// interleaves K and V per group of 8 dimensions, one row of 2 x head_dim bytes per position).
template <int HD, bool KV8>
constexpr int kv_lpp() { return HD / 8; }
template <int HD>
__device__ __forceinline__ void load_kv(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int j, int whi,
                                        int cur, int dummy, int dseg, u32x4& kw, u32x4& vw) {
  constexpr int LPP = HD / 8;
  const int jj = (j < whi && j != cur) ? j : dummy;
  const uint32_t off = ((uint32_t)jj * LPP + dseg) * 16u;
  kw = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, NT);
  vw = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, NT);
}
// INT8 KV: one load per position group (each position's interleaved K and V codes)
template <int HD>
__device__ __forceinline__ void load_kv8(__amdgpu_buffer_rsrc_t rkv, int j, int whi, int cur, int dummy, int dseg,
                                         u32x4& w) {
  constexpr int LPP = HD / 8;
  const int jj = (j < whi && j != cur) ? j : dummy;
  w = __builtin_amdgcn_raw_buffer_load_b128(rkv, ((uint32_t)jj * LPP + dseg) * 16u, 0, NT);
}
// The first row of a KV head's cache (row bytes: head_dim BF16 values of K or of V, or (INT8 KV)
// 2 x head_dim interleaved K and V codes)
template <bool KV8>
__device__ __forceinline__ const uint8_t* kv_head_base(const uint16_t* cache, int64_t kvrow0, int hd) {
  return reinterpret_cast<const uint8_t*>(cache) + kvrow0 * hd * 2;
}

// The opening loads of an attention split -- the first NP (K, V) position-group pairs of this
// wave's range, one per ring slot -- prepared ahead: the KV head's row bases and each pair's
// per-lane byte offset (a slot without a position reads the dummy row, as in load_kv).
template <int NP>
struct KvOpen {
  const uint8_t* kbase;
  const uint8_t* vbase;
  uint32_t off[NP];
};
template <int HD, int NP, bool KV8, int MT = 1>
__device__ __forceinline__ KvOpen<NP> kv_open(const KernelArgs& a, int layer, int g, int sp, int64_t L_att, int c,
                                             int lane) {
  constexpr int LPP = kv_lpp<HD, KV8>(), P = 64 / LPP;
  const int pp = lane / LPP, dseg = lane % LPP;
  KvOpen<NP> o;
  const AttnRange r = attn_range(a, sp, c, L_att);
  const int64_t kvrow0 = ((int64_t)layer * a.n_kv + g) * a.kv_cap;
  o.kbase = kv_head_base<KV8>(a.kv_k, kvrow0, HD);
  o.vbase = kv_head_base<KV8>(a.kv_v, kvrow0, HD);
  const int cur = (int)L_att - 1, dummy = (int)a.kv_cap - 1;
  const int cut = (int)L_att - MT;  // (MT > 1) the step's own positions, from cut on, come from LDS
#pragma unroll
  for (int s = 0; s < NP; ++s) {
    const int j = r.wlo + s * P + pp;
    const bool real = MT == 1 ? (j < r.whi && j != cur) : (j < r.whi && j < cut);
    const int jj = real ? j : dummy;
    o.off[s] = ((uint32_t)jj * LPP + dseg) * 16u;
  }
  return o;
}

// Part h of the opening (pairs h*B/2 .. h*B/2 + B/2 - 1) as one batch of B loads: the start of
// the ring compute_attention runs on, loaded while the previous tile (QKV) streams.  The cache
// rows do not depend on this step's q; the current position's row is never loaded (it comes
// from LDS).
template <int B, int NP>
__device__ __forceinline__ BatchSrc<B> kv_half_src(const KvOpen<NP>& o, int h) {
  BatchSrc<B> b;
  const __amdgpu_buffer_rsrc_t rk = rsrc(o.kbase), rv = rsrc(o.vbase);
#pragma unroll
  for (int s = 0; s < B / 2; ++s) {
    b.d[2 * s] = rk;
    b.d[2 * s + 1] = rv;
    b.vo[2 * s] = b.vo[2 * s + 1] = o.off[h * (B / 2) + s];
    b.so[2 * s] = b.so[2 * s + 1] = 0;
  }
  return b;
}

// Values prepared before a wait are passed through an empty asm statement so that they are
// computed there (the compiler would otherwise sink the arithmetic to the first use, after the
// barrier that ends the wait).
__device__ __forceinline__ void pin(int& x) { asm volatile("" : "+s"(x)); }
__device__ __forceinline__ void pin(int64_t& x) { asm volatile("" : "+s"(x)); }
__device__ __forceinline__ void pin(const uint16_t*& p) { asm volatile("" : "+s"(p)); }
__device__ __forceinline__ void pin(const uint8_t*& p) { asm volatile("" : "+s"(p)); }
__device__ __forceinline__ void pin_v(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(Range& r) {
  pin(r.k);
  pin(r.r0);
  pin(r.C);
  pin(r.i);
  pin(r.ihi);
  pin(r.base);
}
template <int NP>
__device__ __forceinline__ void pin(KvOpen<NP>& o) {
  pin(o.kbase);
  pin(o.vbase);
#pragma unroll
  for (int s = 0; s < NP; ++s) pin_v(o.off[s]);
}

// The values of a 16-byte K or V load: 8 BF16 values, or (INT8 KV) 16 codes
template <bool KV8>
__device__ __forceinline__ void unpack_kv(const u32x4 w, float* f) {
  if constexpr (KV8) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      f[b] = i8(w.x, b);
      f[4 + b] = i8(w.y, b);
      f[8 + b] = i8(w.z, b);
      f[12 + b] = i8(w.w, b);
    }
  } else {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
  }
}

// compute wave: one share of an attention split.  The position groups run through a ring of
// D = NB * B / 2 (K, V) register pairs -- the stream registers themselves, filled with the first D groups
// while the previous tile streamed: each step consumes one slot and reloads it with the group D
// steps ahead (past the range the reload reads the dummy row; every load is unconditional, see
// the weight streaming above).  after(h) reuses the registers of batch slot h to fetch batch h
// of the next GEMV tile.
// INT8 KV (KV8): a slot is the first register of its pair, one load of the position group's
// interleaved K and V codes (the second register is left alone in the loop: the ring keeps the BF16
// shape, which the register budget needs; the opening fills it with the same row); a score
// is the position's K scale times the dot product of the smoothed query (prepared in LDS) with the
// K codes, and a V row contributes its codes times its scale times the weight; the split's scales
// are staged in LDS.
// MT > 1 (multi-token steps): MT * G query rows (row t * G + h: head h at position t of the step);
// the ring covers the cached positions (before the step's first), and each of the step's own
// positions (K/V rows in LDS) is added, by the wave whose range holds it, to the rows at that
// position or later (causal).
template <int HD, int G, int B, int NB, bool KV8, int MT, typename After>
__device__ __forceinline__ void compute_attention(const KernelArgs& a, const Lds& L, int k, int c, int lane, int layer,
                                                  int g, int sp, int64_t L_att, Stream<B, NB>& pf, After after,
                                                  uint64_t* ts) {
  constexpr int PS = pstride<HD>();
  constexpr int D = NB * B / 2;  // ring slots: register pairs in the NB * B stream registers
  constexpr int SPB = B / 2;     // slots per batch of stream registers
  constexpr int GM = G * MT;     // query rows
  const float* q = L.part;
  const float* kc = q + GM * HD;
  const float* vc = kc + MT * HD;
  float* ws = attn_ws<HD, G, MT>(L);
  const int cur = (int)L_att - 1;
  const int cut = (int)L_att - MT;  // first position of the step
  const int64_t kvrow0 = ((int64_t)layer * a.n_kv + g) * a.kv_cap;
  constexpr int LPP = HD / 8;  // lanes per position
  constexpr int P = 64 / LPP;  // positions per load
  const AttnRange rg = attn_range(a, sp, c, L_att);
  const int wlo = rg.wlo, whi = rg.whi;
  // the ring's positions: the whole range (MT = 1: the current position is masked in it), or
  // (MT > 1) the range's cached positions
  const int whr = MT == 1 ? whi : (whi < cut ? whi : cut);
  const int curr = MT == 1 ? cur : -1;
  const int ngroups = whr > wlo ? (whr - wlo + P - 1) / P : 0;
  const int pp = lane / LPP, dseg = lane % LPP;
  const float* qlane = q + dseg * 8;  // q values are re-read from LDS per use (register budget)
  const __amdgpu_buffer_rsrc_t rk = rsrc(kv_head_base<KV8>(a.kv_k, kvrow0, HD));
  const __amdgpu_buffer_rsrc_t rv = rsrc(kv_head_base<KV8>(a.kv_v, kvrow0, HD));
  const float* kss = attn_kscales<HD, G, MT>(L) - rg.lo;  // (KV8) scales by position
  const float* vss = kss + a.kv8_span;
  const int dummy = (int)a.kv_cap - 1;
  // Running state per query head: m[h] is the same in every lane (the largest score the wave has
  // seen so far, base 2); l[h] and acc[h][] are this lane's sums over its positions, weighted
  // by 2^(score - m[h]).
  float m[GM], l[GM], acc[GM][8];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  // score of this lane's position for head h (its 8 dimensions, summed over the LPP lanes)
  auto score = [&](const float* kf, int h) -> float {
    const f32x4 q0 = *reinterpret_cast<const f32x4*>(qlane + h * HD);
    const f32x4 q1 = *reinterpret_cast<const f32x4*>(qlane + h * HD + 4);
    float d0 = q0.x * kf[0], d1 = q0.y * kf[1];
    d0 = fmaf(q0.z, kf[2], d0);
    d1 = fmaf(q0.w, kf[3], d1);
    d0 = fmaf(q1.x, kf[4], d0);
    d1 = fmaf(q1.y, kf[5], d1);
    d0 = fmaf(q1.z, kf[6], d0);
    d1 = fmaf(q1.w, kf[7], d1);
    const float sc = d0 + d1;
    return LPP == 8 ? sum8(sc) : sum16(sc);
  };
  // maximum over the wave's positions (lanes differing by multiples of LPP)
  auto pos_max = [&](float v) -> float {
    if constexpr (LPP == 8) v = fmaxf(v, lane_xor<8>(v, lane));
    v = fmaxf(v, lane_xor<16>(v, lane));
    return fmaxf(v, lane_xor<32>(v, lane));
  };
  // raise each head's running maximum to cover bm (this lane's candidates, -inf for none) and
  // rescale the sums to it
  auto raise = [&](const float* bm) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      const float mn = fmaxf(m[h], pos_max(bm[h]));
      const float al = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m[h] - mn);
      l[h] *= al;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= al;
      m[h] = mn;
    }
  };
  // weighted V of one position (sv: its scale, INT8 KV; 1 for BF16 rows).  A slot without a
  // position contributes exactly nothing: its weight is 0 and its V values are replaced by 0
  // (selects, not a multiplication by 0, so that whatever the masked load read -- a NaN in an
  // unwritten cache row included -- cannot reach the sums).
  auto accumulate = [&](bool valid, const float* sc, float* vf, float sv) {
#pragma unroll
    for (int e = 0; e < 8; ++e) vf[e] = valid ? vf[e] : 0.0f;
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      const float p = valid ? __builtin_amdgcn_exp2f(sc[h] - m[h]) : 0.0f;
      l[h] += p;
      const float pv = KV8 ? p * sv : p;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pv, vf[e], acc[h][e]);
    }
  };
  // slot s: its K and V values (8 dimensions each) from the stream registers
  auto slot_k = [&](int s, float* kf) {
    if constexpr (KV8) {
      const u32x4 w = pf.v[2 * s];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        kf[b] = i8(w.x, b);
        kf[4 + b] = i8(w.y, b);
      }
    } else {
      unpack_kv<false>(pf.v[2 * s], kf);
    }
  };
  auto slot_v = [&](int s, float* vf) {
    if constexpr (KV8) {
      const u32x4 w = pf.v[2 * s];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        vf[b] = i8(w.z, b);
        vf[4 + b] = i8(w.w, b);
      }
    } else {
      unpack_kv<false>(pf.v[2 * s + 1], vf);
    }
  };
  auto slot_load = [&](int s, int j) {
    if constexpr (KV8) load_kv8<HD>(rk, j, whi, cur, dummy, dseg, pf.v[2 * s]);
    else load_kv<HD>(rk, rv, j, whr, curr, dummy, dseg, pf.v[2 * s], pf.v[2 * s + 1]);
  };
  if (pf.k != k) {  // no prefetch (e.g. this worker had no tile in the previous wave): fill the ring now
#pragma unroll
    for (int s = 0; s < D; ++s) slot_load(s, wlo + s * P + pp);
  }
  stamp(ts, TS_ENTRY, lane);
  // One pass per D position groups (the ring): scores of every slot from its K row, one raise of
  // the running maximum, then the weighted V rows.  Slots past the range, or holding the current
  // position (taken from LDS below), are masked.  In every pass but the last each slot is
  // reloaded (group + D) as soon as its V row is used; in the last pass each batch of SPB
  // slots, once used, fetches batch h of the next GEMV tile instead (after(h)).
  constexpr int SUB = D;
  auto pass = [&](int g0, bool last) {
#pragma unroll
    for (int s0 = 0; s0 < D; s0 += SUB) {
      float sc[SUB][GM], bm[GM], svs[SUB];
      bool valid[SUB];
#pragma unroll
      for (int h = 0; h < GM; ++h) bm[h] = -INFINITY;
#pragma unroll
      for (int t = 0; t < SUB; ++t) {
        const int s = s0 + t;
        const int j = wlo + (g0 + s) * P + pp;
        valid[t] = j < whr && j != curr;
        float ks = 1.f;
        svs[t] = 1.f;
        if constexpr (KV8) {  // the row's scales (a slot without a position reads the split's first)
          const int jj = valid[t] ? j : rg.lo;
          ks = kss[jj];
          svs[t] = vss[jj];
        }
        float kf[8];
        slot_k(s, kf);
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          sc[t][h] = KV8 ? ks * score(kf, h) : score(kf, h);
          bm[h] = valid[t] ? fmaxf(bm[h], sc[t][h]) : bm[h];
        }
      }
      raise(bm);
#pragma unroll
      for (int t = 0; t < SUB; ++t) {
        const int s = s0 + t;
        float vf[8];
        slot_v(s, vf);
        accumulate(valid[t], sc[t], vf, svs[t]);
        if (!last) {
          slot_load(s, wlo + (g0 + s + D) * P + pp);
          __builtin_amdgcn_sched_barrier(0);  // keep each reload right after its slot's use (the overlap)
        } else if (s % SPB == SPB - 1) {
          after(s / SPB);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (s == 0 && g0 == 0) stamp(ts, TS_FIRST, lane);
      }
    }
  };
  int g0 = 0;
  for (; g0 + D < ngroups; g0 += D) pass(g0, false);
  pass(g0, true);
  if constexpr (MT > 1) {
    // the step's positions (K/V rows in LDS), lane group 0: position u of the step reaches the
    // rows of positions u and later only
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      const int pu = cut + u;
      if (wlo <= pu && pu < whi) {
        float kf[8], vf[8], sc[GM], bm[GM];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kf[e] = kc[u * HD + dseg * 8 + e];
          vf[e] = pp == 0 ? vc[u * HD + dseg * 8 + e] : 0.f;
        }
        // (INT8 KV: kc / vc hold the row's codes, SM_KVCUR + 2 u its K and V scales)
        const float ks = KV8 ? L.small[SM_KVCUR + 2 * u] : 1.f;
        const float sv = KV8 ? L.small[SM_KVCUR + 2 * u + 1] : 1.f;
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          sc[h] = KV8 ? ks * score(kf, h) : score(kf, h);
          bm[h] = pp == 0 && u <= h / G ? sc[h] : -INFINITY;
        }
        raise(bm);
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          const float p = pp == 0 && u <= h / G ? __builtin_amdgcn_exp2f(sc[h] - m[h]) : 0.0f;
          l[h] += p;
          const float pv = KV8 ? p * sv : p;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pv, vf[e], acc[h][e]);
        }
      }
    }
  } else if (wlo <= cur && cur < whi) {  // the current position (its K/V row, or its codes, in LDS): lane group 0
    float kf[8], vf[8], sc[G], bm[G];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kf[e] = kc[dseg * 8 + e];
      vf[e] = vc[dseg * 8 + e];
    }
    const float ks = KV8 ? L.small[SM_KVCUR] : 1.f;
    const float sv = KV8 ? L.small[SM_KVCUR + 1] : 1.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sc[h] = KV8 ? ks * score(kf, h) : score(kf, h);
      bm[h] = pp == 0 ? sc[h] : -INFINITY;
    }
    raise(bm);
    accumulate(pp == 0, sc, vf, sv);
  }
  // every lane's sums are relative to the same maximum: add up the lanes of equal dimensions
  auto sum_lanes = [&](auto off_tag) {
    constexpr int OFF = decltype(off_tag)::value;
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      l[h] += lane_xor<OFF>(l[h], lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += lane_xor<OFF>(acc[h][e], lane);
    }
  };
  if constexpr (LPP == 8) sum_lanes(std::integral_constant<int, 8>{});
  sum_lanes(std::integral_constant<int, 16>{});
  sum_lanes(std::integral_constant<int, 32>{});
  if (pp == 0) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      float* st = ws + (c * GM + h) * PS;
      if (dseg == 0) {
        st[0] = m[h];
        st[1] = l[h];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) st[2 + dseg * 8 + e] = acc[h][e];
    }
  }
}

// all wavefronts, between barriers B and E: merge the compute waves' states in wave order into
// the tile's partial (m, l, acc, pad) per query head
template <int HD, int G, int MT = 1>
__device__ __forceinline__ void attn_merge_phase(const Lds& L, int wave_index, int lane) {
  constexpr int PS = pstride<HD>();
  constexpr int GM = G * MT;  // query rows
  const float* ws = attn_ws<HD, G, MT>(L);
  float* mrg = attn_merged<HD, G, MT>(L);
  for (int idx = wave_index * 64 + lane; idx < GM * HD; idx += BLOCK_THREADS) {
    const int h = idx / HD, d = idx % HD;
    // every compute wave's state of head h (independent loads), then one common maximum
    float mv[NCOMP], lv[NCOMP], av[NCOMP];
#pragma unroll
    for (int c = 0; c < NCOMP; ++c) {
      const float* st = ws + (c * GM + h) * PS;
      mv[c] = st[0];
      lv[c] = st[1];
      av[c] = st[2 + d];
    }
    float mm = -INFINITY;
#pragma unroll
    for (int c = 0; c < NCOMP; ++c) mm = fmaxf(mm, mv[c]);
    float ll = 0.f, aa = 0.f;
#pragma unroll
    for (int c = 0; c < NCOMP; ++c) {
      const float f = mv[c] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv[c] - mm);  // a wave without positions: weight 0
      ll = fmaf(f, lv[c], ll);
      aa = fmaf(f, av[c], aa);
    }
    float* dst = mrg + h * PS;
    if (d == 0) {
      dst[0] = mm;
      dst[1] = ll;
      dst[HD + 2] = 0.f;
      dst[HD + 3] = 0.f;
    }
    dst[2 + d] = aa;
  }
}

// control wave, after barrier E: publish the merged partials of query heads qa .. qa + G - 1, split sp
// (MT > 1: the rows of position t of the step go to out + t * ll_tok)
template <int HD, int G, int MT = 1>
__device__ __forceinline__ void cw_attn_publish(const KernelArgs& a, const Lds& L, uint32_t* out, int lane, int qa, int sp,
                                uint32_t par) {
  constexpr int PS = pstride<HD>();
  constexpr int GM = G * MT;  // query rows
  constexpr int N = (GM * PS + 63) / 64;  // values per lane
  const float* mrg = attn_merged<HD, G, MT>(L);
  float v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = lane + 64 * i < GM * PS ? mrg[lane + 64 * i] : 0.f;  // reads first, then the stores
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int idx = lane + 64 * i;
    if constexpr (MT == 1) {
      if (idx < G * PS) publish(out, ((int64_t)(qa + idx / PS) * a.S + sp) * PS + idx % PS, v[i], par);
    } else if (idx < GM * PS) {
      const int r = idx / PS, t = r / G;
      publish(out + t * a.ll_tok, ((int64_t)(qa + r - t * G) * a.S + sp) * PS + idx % PS, v[i], par);
    }
  }
}

// ---------------------------------------------------------------------------
// per-wave phases shared by all wavefronts.  The control wave (0) and the compute waves
// (1..7) run separate loops (so that each keeps only its own values in registers) with the
// same barrier sequence per wave: P (inputs staged), A (LDS prologue done; only for tiles whose
// prologue writes LDS the compute waves read), then for GEMV tiles B per row block (and C
// between blocks), for attention tiles B and E.
// ---------------------------------------------------------------------------

// Multi-token steps whose o_proj prologue merges the splits: the merged heads of position t are at
// vec + t * Qpad (the o_proj tile's input stride), and the split partials of every position sit
// after them (position t's n_heads * S records at vec + MT * Qpad + t * n_heads * S * (HD + 4),
// running on into the partial area, which o_proj's compute wavefronts write only after barrier A).
template <int MT>
__device__ __forceinline__ int o_in_stride(const KernelArgs& a) { return MT > 1 && a.combine_in_o ? a.Qpad : a.lds_vec_floats; }
template <int MT>
__device__ __forceinline__ float* o_partials(const KernelArgs& a, const Lds& L) {
  return MT > 1 ? L.vec + MT * a.Qpad : L.part;
}

// Gather this wavefront's share of wave k's inputs into LDS.  Returns true when a wait was
// abandoned.  The control wave also reduces the previous step's token (tok).
// MT > 1 (multi-token steps): the inputs of every position tp of the step, from the producer's
// buffer of that position (ll_tok words after the previous one's), in one polling loop: a GEMV input
// at vec + tp * lds_vec_floats (o_proj's merged heads: o_in_stride apart) and its residual row at
// xres + tp * XS; a combine tile's split partials at part + tp * S * (HD + 4), the o_proj prologue's
// at o_partials.  The step's tokens are the given ones (verify), and the previous step's argmaxes
// are recorded.
template <int HD, int G, bool CTRL, bool WD, bool Q8, bool SMP, bool KV8, int MT = 1>
__device__ __forceinline__ bool gather_inputs(const KernelArgs& a, const Lds& L, int bid, int wave, int lane, int k,
                                              const TileDesc& t, const WaveDesc& wd, int step, uint32_t par,
                                              int& tok) {
  constexpr int PS = pstride<HD>();
  static_assert(MT == 1 || !SMP, "multi-token steps are greedy verify steps");
  const int VS = a.lds_vec_floats, XS = (a.Hpad + 63) & ~63;
  const int layer = wd.layer;
  const uint32_t* in = a.ll + (k > 0 ? wave_of(L, k - 1).ll_off : 0);
  // Every worker gathers x in the QKV and gate/up waves, tile or not: the o_proj and down
  // epilogues add their rows to the residual staged there.
  const int gk = (wd.kind == KIND_QKV || wd.kind == KIND_GU) ? wd.kind : t.kind;
  bool ab = false;
  switch (gk) {
    case KIND_QKV:
    case KIND_GU:
    case KIND_LM: {
      const int64_t goff = gk == KIND_QKV ? gain_off(L, layer, 0)
                           : gk == KIND_GU ? gain_off(L, layer, 1)
                                           : a.final_norm_off;
      const uint16_t* gain = reinterpret_cast<const uint16_t*>(a.packed + goff);
      float ss[MT];
#pragma unroll
      for (int tp = 0; tp < MT; ++tp) ss[tp] = 0.f;
      bool ctrl_pads = false;  // the control wavefront alone zeroes the input's padding (after its LDS use)
      if (gk == KIND_QKV && layer == 0) {
        if (SMP && step > 0) {
          ctrl_pads = true;
          // sampled decoding: the control wavefront polls the previous step's candidates into LDS
          // (over the input-vector and row-partial areas: the compute wavefronts have left the LM
          // tile and wait at barrier P, and its own epilogue is done) and draws the token; its
          // uniform is loaded before the polls.  The compute wavefronts' code is the greedy one.
          if (CTRL) {
            const float u = a.uniforms[step - 1];
            ab = poll_candidates<WD>(a, L, lane, step_parity(step - 1));
            if (!ab) {
              tok = draw_token(a, L, lane, u);
              if (bid == 0 && lane == 0) a.out_tokens[step - 1] = tok;
            }
          }
        } else if (CTRL && step > 0) {
          if constexpr (MT == 1) {
            ab = gather_token<WD>(a, lane, step_parity(step - 1), tok);
            if (!ab && bid == 0 && lane == 0) a.out_tokens[step - 1] = tok;
            if (!ab && a.forced) tok = a.forced[step - 1];  // a verify step: the given token, not the argmax
          } else {
#pragma unroll
            for (int tp = 0; tp < MT; ++tp) {
              int am = 0;
              if (!ab) ab = gather_token<WD>(a, lane, step_parity(step - 1), am, tp);
              if (!ab && bid == 0 && lane == 0) a.out_tokens[(step - 1) * MT + tp] = am;
            }
          }
        }
        if (CTRL && !ab) {
          if constexpr (MT == 1) {
            ss[0] = stage_embedding<Q8>(a, L.vec, L.xres, tok, gain, lane);
          } else {
#pragma unroll
            for (int tp = 0; tp < MT; ++tp) {
              const int i = step * MT + tp;  // position of the launch
              ss[tp] = stage_embedding<Q8>(a, L.vec + tp * VS, L.xres + tp * XS, i == 0 ? a.token0 : a.forced[i - 1], gain,
                                           lane);
            }
          }
        }
      } else if constexpr (MT == 1) {
        ab = gather_norm<WD, Q8>(a, L.vec, L.xres, in, a.H, gain, wave, lane, par, ss[0]);
      } else {
        ab = gather_norm_mt<WD, Q8, MT>(a, L.vec, L.xres, VS, XS, in, a.H, gain, wave, lane, par, ss);
      }
      if (!ctrl_pads) {
#pragma unroll
        for (int tp = 0; tp < MT; ++tp)
          for (int i = a.H + wave * 64 + lane; i < t.kpad; i += BLOCK_THREADS) L.vec[tp * VS + vperm<Q8>(i)] = 0.f;
      } else if (CTRL) {  // (the candidates the control wavefront polled also covered the padding)
        for (int i = a.H + lane; i < t.kpad; i += 64) L.vec[vperm<Q8>(i)] = 0.f;
      }
      if (lane == 0) {
#pragma unroll
        for (int tp = 0; tp < MT; ++tp) L.small[sm_ss(tp) + wave] = ss[tp];
      }
      break;
    }
    case KIND_O:
    case KIND_DOWN:
    case KIND_COMBINE: {
      // one plain gather for all three (a single copy of the polling loop in the code): the
      // o_proj input (split partials, or merged heads), the SwiGLU rows, or one head's partials
      float* dst = L.vec;
      const uint32_t* src = in;
      int n = a.F, nz = a.F;
      int vs = VS;  // (MT > 1) floats between the positions' GEMV inputs
      if (gk == KIND_O) {
        dst = a.combine_in_o ? o_partials<MT>(a, L) : L.vec;
        n = a.combine_in_o ? a.n_heads * a.S * PS : a.n_heads * HD;
        nz = a.n_heads * HD;
        vs = o_in_stride<MT>(a);
      } else if (gk == KIND_COMBINE) {
        dst = L.part;
        src = in + (int64_t)t.row0 * a.S * PS;
        n = a.S * PS;
        nz = t.kpad;  // no GEMV input to pad
      }
      if constexpr (MT == 1) {
        ab = gather_plain<WD, Q8>(a, dst, src, n, wave, lane, par, dst == L.vec);
      } else {
        // per position: the GEMV input (vs apart), or split partials (n apart)
        const bool vin = gk != KIND_COMBINE && !(gk == KIND_O && a.combine_in_o);
        ab = gather_plain_mt<WD, Q8, MT>(a, dst, vin ? vs : n, src, n, wave, lane, par, vin);
      }
#pragma unroll
      for (int tp = 0; tp < MT; ++tp)
        for (int i = nz + wave * 64 + lane; i < t.kpad; i += BLOCK_THREADS) L.vec[tp * vs + vperm<Q8>(i)] = 0.f;
      break;
    }
    case KIND_ATTN: {
      // the control wave also stages the current position's RoPE row and the q/k-norm gains;
      // the loads are issued before the poll and complete while it waits for the producers
      constexpr int HALF = HD / 2;
      float2 cs[MT];
      float gq0 = 0.f, gq1 = 0.f, gk0 = 0.f, gk1 = 0.f;
      const int64_t qoff = gain_off(L, layer, 2);
#pragma unroll
      for (int tp = 0; tp < MT; ++tp) cs[tp] = {0.f, 0.f};
      if (CTRL && lane < HALF) {
#pragma unroll
        for (int tp = 0; tp < MT; ++tp)
          cs[tp] = *reinterpret_cast<const float2*>(a.rope + ((int64_t)(a.pos0 + step * MT + tp) * HALF + lane) * 2);
        if (qoff >= 0) {
          const uint16_t* gq = reinterpret_cast<const uint16_t*>(a.packed + qoff);
          const uint16_t* gkk = reinterpret_cast<const uint16_t*>(a.packed + gain_off(L, layer, 3));
          gq0 = bf16_to_f32(gq[lane]);
          gq1 = bf16_to_f32(gq[lane + HALF]);
          gk0 = bf16_to_f32(gkk[lane]);
          gk1 = bf16_to_f32(gkk[lane + HALF]);
        }
      }
      // INT8 KV: the control wave also loads the KV head's key smoothing factors, and every
      // wavefront stages a share of the split's K and V scales of the cached positions straight into
      // LDS (64 positions per load, no registers held across the polls; issued before the polls
      // like the others; the current position's come from the LDS prologue)
      constexpr int SPT = MAX_SPLIT_POSITIONS_KV8 / BLOCK_THREADS;  // 64-position loads per wavefront
      float sg0 = 0.f, sg1 = 0.f;
      if constexpr (KV8) {
        const int64_t kvrow0 = ((int64_t)layer * a.n_kv + t.row0) * a.kv_cap;
        if (CTRL && lane < HALF) {
          const float* sg = a.kv_sigma + ((int64_t)layer * a.n_kv + t.row0) * HD;
          sg0 = sg[lane];
          sg1 = sg[lane + HALF];
        }
        const int pos = a.pos0 + step * MT;  // the step's first position
        int slo = 0, shi = 0;
        split_bounds(a.S, t.nrows, pos + MT, slo, shi);
        const int sn = (shi < pos ? shi : pos) - slo;  // cached positions of the split
        const uint32_t kl = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)attn_kscales<HD, G, MT>(L);
        for (int i = 0; i < SPT; ++i) {
          const int e0 = (wave + i * (BLOCK_THREADS / 64)) * 64;  // wavefront-uniform
          if (e0 >= sn) break;
          if (e0 + lane < sn) {
            const int64_t g = kvrow0 + slo + e0 + lane;
            stage_dword(a.kv_ks + g, kl + 4u * (uint32_t)e0);
            stage_dword(a.kv_vs + g, kl + 4u * (uint32_t)(a.kv8_span + e0));
          }
        }
      }
      if constexpr (MT == 1) ab = gather_qkv<HD, G, WD>(a, L.vec, in, t.row0, t.aux0, wave, lane, par);
      else ab = gather_qkv_mt<HD, G, WD, MT>(a, L.vec, VS, in, t.row0, t.aux0, wave, lane, par);
      if constexpr (KV8) wait_vmcnt<0>();  // the staged scales are in LDS before the tile's barrier
      if (CTRL && lane < HALF) {
#pragma unroll
        for (int tp = 0; tp < MT; ++tp) {
          float* rr = rope_rows<HD, G, KV8, MT>(L, a.kv8_span) + tp * HD;
          rr[2 * lane] = cs[tp].x;
          rr[2 * lane + 1] = cs[tp].y;
        }
        L.small[SM_QGAIN + lane] = gq0;
        L.small[SM_QGAIN + lane + HALF] = gq1;
        L.small[SM_KGAIN + lane] = gk0;
        L.small[SM_KGAIN + lane + HALF] = gk1;
        if (KV8) {
          L.small[SM_KSMOOTH + lane] = sg0;
          L.small[SM_KSMOOTH + lane + HALF] = sg1;
        }
      }
      break;
    }
    default:
      break;
  }
  return ab;
}

// Barrier A is needed only where the prologue writes LDS the compute waves read (attention prep,
// split merges).  For the other tiles the prologue only forms the folded RMSNorm scale, which only
// the control wave's epilogue uses: their compute waves start streaming right after barrier P.
__device__ __forceinline__ bool needs_barrier_a(const KernelArgs& a, const TileDesc& t) {
  return t.kind == KIND_ATTN || t.kind == KIND_COMBINE || (t.kind == KIND_O && a.combine_in_o);
}

// The folded RMSNorm scale of position tp of the step (after barrier P).
__device__ __forceinline__ float norm_scale(const KernelArgs& a, const Lds& L, int tp) {
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) tot += L.small[sm_ss(tp) + w];
  return 1.0f / sqrtf(tot / (float)a.H + a.eps);
}

// LDS-only prologue work between barriers P and A; returns the folded RMSNorm scale (of the step's
// first position; MT > 1: norm_scale gives the others).  pos: the step's first position.
template <int HD, int G, bool Q8, bool KV8, int MT = 1>
__device__ __forceinline__ float lds_prologue(const KernelArgs& a, const Lds& L, int wave, int lane,
                                              const TileDesc& t, int layer, int pos) {
  float rs = 1.0f;
  if (t.kind == KIND_QKV || t.kind == KIND_GU || t.kind == KIND_LM) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) tot += L.small[SM_SS + w];
    rs = 1.0f / sqrtf(tot / (float)a.H + a.eps);
  } else if (t.kind == KIND_ATTN) {
    attn_lds_prep<HD, G, KV8, MT>(a, L, wave, lane, layer, pos, t.nrows);
  } else if ((t.kind == KIND_O && a.combine_in_o) || t.kind == KIND_COMBINE) {
    // all heads' splits (o_proj prologue) or one head's (combine tile): one copy of the merge
    // (MT > 1: one merge per position of the step)
    const bool o = t.kind == KIND_O;
    const int nh = o ? a.n_heads : 1;
    const float* src = o ? o_partials<MT>(a, L) : L.part;
    const int ostride = o ? o_in_stride<MT>(a) : a.lds_vec_floats;
#pragma unroll
    for (int tp = 0; tp < MT; ++tp)
      merge_heads<HD, Q8>(src + tp * nh * a.S * pstride<HD>(), nh, a.S, wave * 64 + lane, L.vec + tp * ostride, o);
  }
  return rs;
}


// ---------------------------------------------------------------------------
// control wave loop
// ---------------------------------------------------------------------------

// (weight-only INT8) The scales of rows [r0, r0 + block) of GEMV tile t, this lane's share (row
// lane + 64 i in register i): loaded into registers before the tile's input gather, so that they
// arrive while it waits, and put into LDS after it for the epilogue.
constexpr int SCALE_REGS = MAX_BLOCK_ROWS / 64;
constexpr int ROWS_PER_LANE = MAX_BLOCK_ROWS / 64;  // rows of a block per control-wave lane
__device__ __forceinline__ int tile_rows(const TileDesc& t) { return t.kind == KIND_GU ? 2 * t.nrows : t.nrows; }
__device__ __forceinline__ void load_scales(const KernelArgs& a, const TileDesc& t, int r0, int block_rows, int lane,
                                            float* sreg) {
  const int rows = tile_rows(t);
  const int nr = min(block_rows, rows - r0);
  const float* sp = reinterpret_cast<const float*>(a.packed + t.woff + (int64_t)rows * t.kpad) + r0;
#pragma unroll
  for (int i = 0; i < SCALE_REGS; ++i) {
    const int r = lane + 64 * i;
    sreg[i] = r < nr ? sp[r] : 0.f;
  }
}
__device__ __forceinline__ void put_scales(const Lds& L, const TileDesc& t, int r0, int block_rows, int lane,
                                           const float* sreg) {
  const int nr = min(block_rows, tile_rows(t) - r0);
#pragma unroll
  for (int i = 0; i < SCALE_REGS; ++i) {
    const int r = lane + 64 * i;
    if (r < nr) L.scl[r] = sreg[i];
  }
}

// MT > 1 (multi-token steps): each step runs positions pos0 + step * MT .. + MT - 1; every epilogue
// runs once per position (its partials at part + tp * block_rows * NCOMP, its outputs at out + tp *
// ll_tok), and the LM head publishes one (max, index) partial per position (lmpart + tp * W).
template <int HD, int G, bool WD, bool Q8, bool SMP, bool KV8, int MT = 1>
__device__ __forceinline__ void control_loop(const KernelArgs& a, const Lds& L, int bid, int lane, int block_rows) {
  // The abort word lives in LDS and is written and read only on either side of a barrier (which
  // orders them), so plain accesses: the compiler then emits LDS instructions.  A volatile access
  // through this generic pointer would be a FLAT access, whose wait also drains every outstanding
  // global load and store of the wavefront (its prefetch, its last publish).
  int* smi = reinterpret_cast<int*>(L.small);
  int tok = a.token0;
  const int H = a.H;
  const int VS = a.lds_vec_floats, XS = (a.Hpad + 63) & ~63, PT = block_rows * NCOMP;
  bool stop = false;
  for (int step = 0; step < a.n_steps && !stop; ++step) {
    const uint32_t par = step_parity(step);
    const int pos = a.pos0 + step * MT;  // the step's first position
    const int64_t L_att = (int64_t)pos + MT;
    float lm_best[MT];
    int lm_idx[MT];
#pragma unroll
    for (int tp = 0; tp < MT; ++tp) {
      lm_best[tp] = -INFINITY;
      lm_idx[tp] = 0x7fffffff;
    }
    uint64_t lm_run = 0;  // sampled decoding: lane i holds this worker's i-th largest logit so far
    for (int k = 0; k < a.n_waves; ++k) {
      const TileDesc t = tile_of(L, k);
      const WaveDesc wd = wave_of(L, k);
      const int layer = wd.layer;
      uint32_t* out = a.ll + (wd.ll_off >= 0 ? wd.ll_off : 0);
      uint64_t t0 = 0, t_pro = 0, t_cmp = 0;
      uint64_t cw[TS_COUNT] = {};  // the first compute wavefront's stamps, read after barrier B
      uint64_t t_preb = 0, t_last = 0;  // control wave ready for B; last compute wavefront done
      const uint64_t* wds = reinterpret_cast<const uint64_t*>(L.small + SM_WDONE) + (k & 1) * 8;
      const uint64_t* cts = reinterpret_cast<const uint64_t*>(L.small + SM_CTRACE) + (k & 1) * 8;
      if (a.trace) t0 = wall_clock64();
      float sreg[SCALE_REGS];
      if (gather_inputs<HD, G, true, WD, Q8, SMP, KV8, MT>(a, L, bid, 0, lane, k, t, wd, step, par, tok)) smi[SM_ABORT] = 1;
      __syncthreads();  // P: inputs staged in LDS
      if (smi[SM_ABORT]) {
        stop = true;
        break;
      }
      // (INT8) the first block's row scales, issued after the input gather (its polls would complete
      // behind them) and arriving while the compute wavefronts stream the block
      if constexpr (Q8) {
        if (is_gemv(t.kind)) load_scales(a, t, 0, block_rows, lane, sreg);
      }
      if (a.trace) t_pro = wall_clock64();
      float rs[MT];
      rs[0] = lds_prologue<HD, G, Q8, KV8, MT>(a, L, 0, lane, t, layer, pos);
#pragma unroll
      for (int tp = 1; tp < MT; ++tp)
        rs[tp] = t.kind == KIND_QKV || t.kind == KIND_GU || t.kind == KIND_LM ? norm_scale(a, L, tp) : 1.0f;
      if (needs_barrier_a(a, t)) __syncthreads();  // A: inputs ready
      const uint64_t t_a = a.trace ? wall_clock64() : 0;
      if (is_gemv(t.kind)) {
        const int rows = t.kind == KIND_GU ? 2 * t.nrows : t.nrows;
        const int C = t.kpad / chunk_cols<Q8>();
        for (int r0 = 0; r0 < rows; r0 += block_rows) {
          const int nr = min(block_rows, rows - r0);
          // a row's total over the compute wavefronts' partials, times its scale in an INT8 tile
          auto total = [&](const float* part, int r) {
            const float x = row_total(part, nr, C, r);
            return Q8 ? L.scl[r] * x : x;
          };
          if constexpr (Q8) {
            if (r0 > 0) load_scales(a, t, r0, block_rows, lane, sreg);  // a later block's scales
          }
          __syncthreads();  // B: partials of this block ready
          if constexpr (Q8) put_scales(L, t, r0, block_rows, lane, sreg);  // (read by this wavefront only)
          if (a.trace && r0 == 0) {
            t_cmp = wall_clock64();
            for (int i = 0; i < TS_COUNT; ++i) cw[i] = cts[i];
            for (int w = 1; w < NWAVES; ++w) t_last = wds[w] > t_last ? wds[w] : t_last;
          }
#pragma unroll
          for (int tp = 0; tp < MT; ++tp) {  // (the step's positions)
            uint32_t* o = out + tp * a.ll_tok;
            const float* pa = L.part + tp * PT;
            const float* xr = L.xres + tp * XS;
            const int64_t srow = (int64_t)step * MT + tp;  // position of the launch
            switch (t.kind) {
              case KIND_QKV:
                for (int r = lane; r < nr; r += 64) publish(o, t.row0 + r0 + r, rs[tp] * total(pa, r), par);
                break;
              case KIND_O:
                for (int r = lane; r < nr; r += 64) {
                  const int j = t.row0 + r0 + r;
                  publish(o, j, xr[j] + total(pa, r), par);
                }
                break;
              case KIND_GU:  // interleaved gate/up rows
                for (int p = lane; p < nr / 2; p += 64) {
                  const float gt = rs[tp] * total(pa, 2 * p);
                  const float up = rs[tp] * total(pa, 2 * p + 1);
                  publish(o, t.row0 + r0 / 2 + p, gt / (1.0f + __expf(-gt)) * up, par);
                }
                break;
              case KIND_DOWN:
                for (int r = lane; r < nr; r += 64) {
                  const int j = t.row0 + r0 + r;
                  const float nx = xr[j] + total(pa, r);
                  publish(o, j, nx, par);
                  if (a.dbg_hidden) a.dbg_hidden[(srow * a.n_layers + layer) * H + j] = tag_clear(nx);
                }
                break;
              case KIND_LM:
                if constexpr (SMP) {
                  uint64_t cand[ROWS_PER_LANE];  // this lane's rows of the block, r = lane + 64 j
#pragma unroll
                  for (int j = 0; j < ROWS_PER_LANE; ++j) {
                    const int r = lane + 64 * j;
                    cand[j] = 0;
                    if (r < nr) {
                      const float v = rs[tp] * total(pa, r);
                      const int idx = t.row0 + r0 + r;
                      if (a.out_logits) __builtin_nontemporal_store(v, a.out_logits + srow * a.V + idx);
                      cand[j] = cand_key(v, idx);
                    }
                  }
                  topk_merge(lm_run, cand, a.top_k, lane);
                  break;
                }
                for (int r = lane; r < nr; r += 64) {
                  const float v = rs[tp] * total(pa, r);
                  const int idx = t.row0 + r0 + r;
                  if (a.out_logits) __builtin_nontemporal_store(v, a.out_logits + srow * a.V + idx);
                  if (v > lm_best[tp]) {  // each lane visits its rows in increasing order: first maximum kept
                    lm_best[tp] = v;
                    lm_idx[tp] = idx;
                  }
                }
                break;
            }
          }
          if (r0 + block_rows < rows) __syncthreads();  // C: partials consumed
        }
      } else if (t.kind == KIND_ATTN) {
        cw_attn_kv_write<HD, G, KV8, MT>(a, L, lane, layer, t.row0, t.nrows, t.aux0, L_att);
        // The KV row must be complete before this worker publishes anything later readers of
        // the row depend on (its split partial, below); the wait overlaps the compute waves.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (a.trace) t_preb = wall_clock64();
        __syncthreads();  // B: compute-wave states ready
        if (a.trace) {
          t_cmp = wall_clock64();
          for (int i = 0; i < TS_COUNT; ++i) cw[i] = cts[i];
          for (int w = 1; w < NWAVES; ++w) t_last = wds[w] > t_last ? wds[w] : t_last;
        }
        attn_merge_phase<HD, G, MT>(L, 0, lane);
        __syncthreads();  // E: merged partial ready
        cw_attn_publish<HD, G, MT>(a, L, out, lane, t.aux0, t.nrows, par);
      } else if (t.kind == KIND_COMBINE) {
        if (a.trace) t_cmp = wall_clock64();
#pragma unroll
        for (int tp = 0; tp < MT; ++tp)
          for (int d = lane; d < HD; d += 64) publish(out + tp * a.ll_tok, (int64_t)t.row0 * HD + d, L.vec[tp * VS + d], par);
      }
      if (SMP && wd.kind == KIND_LM) {
        // this worker's top_k candidates in decreasing order, lane i the i-th ((-inf, 0x7fffffff) where
        // the worker has fewer rows); the first one last, as the release of the worker's step
        uint64_t* dst = reinterpret_cast<uint64_t*>(a.lmpart) + (int64_t)bid * a.top_k;
        const float v = lm_run ? key_value(lm_run) : -INFINITY;
        const uint32_t ix = lm_run ? (uint32_t)key_index(lm_run) : 0x7fffffffu;
        const uint64_t word = (uint64_t)__float_as_uint(v) | ((uint64_t)(ix | (par << 31)) << 32);
        if (lane > 0 && lane < a.top_k) st_u64(dst + lane, word);
        if (lane == 0) st_u64_release(dst, word);
      } else if (wd.kind == KIND_LM) {
        // worker partial (max, lowest index); also published by workers without vocabulary rows
#pragma unroll
        for (int tp = 0; tp < MT; ++tp) {
          float best = lm_best[tp];
          int bi = lm_idx[tp];
          for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(best, off);
            const int oi = __shfl_xor(bi, off);
            if (ov > best || (ov == best && oi < bi)) {
              best = ov;
              bi = oi;
            }
          }
          if (lane == 0)
            st_u64_release(reinterpret_cast<uint64_t*>(a.lmpart) + (int64_t)tp * a.W + bid,
                           (uint64_t)__float_as_uint(best) | ((uint64_t)((uint32_t)bi | (par << 31)) << 32));
        }
      }
      if (a.trace && lane == 0) {
        const uint64_t t1 = wall_clock64();
        uint64_t* tr = a.trace + (((int64_t)step * a.n_waves + k) * a.W + bid) * TRACE_WORDS;
        tr[0] = t0;
        tr[1] = t_pro;
        tr[2] = t_cmp ? t_cmp : t_pro;
        tr[3] = t1;
        tr[7] = t_a;
        tr[4] = cw[TS_DONE];
        tr[5] = cw[TS_GATHERED];
        tr[6] = cw[TS_AFTER_A];
        tr[8] = cw[TS_FIRST];
        tr[9] = cw[TS_ENTRY];
        tr[10] = t_preb;
        tr[11] = t_last;
      }
    }
  }
  // the last step's token
  if (!stop && bid == 0) {
    int last = 0;
    if constexpr (SMP) {
      const float u = a.uniforms[a.n_steps - 1];
      if (!poll_candidates<WD>(a, L, lane, step_parity(a.n_steps - 1))) {
        last = draw_token(a, L, lane, u);
        if (lane == 0) a.out_tokens[a.n_steps - 1] = last;
      }
    } else {
      bool ab = false;
#pragma unroll
      for (int tp = 0; tp < MT; ++tp) {
        if (!ab) ab = gather_token<WD>(a, lane, step_parity(a.n_steps - 1), last, tp);
        if (!ab && lane == 0) a.out_tokens[(a.n_steps - 1) * MT + tp] = last;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// compute wave loop
// ---------------------------------------------------------------------------

// Register sets of the compute waves' stream ring (batches in flight per wave).  Two sets keep
// 8 KB per wave, 56 KB per compute unit in flight.  Four sets (112 KB per compute unit) were
// measured slower on the 1B-parameter Llama shape: the long streams (LM head, gate/up) did not
// speed up -- they already run near what the HBM delivers to a stream of 16-byte loads -- while
// the small tiles paid for padded ring passes and a longer in-order wait before each gather.
template <int HD, int G>
constexpr int stream_sets() {
  return 2;
}

template <int HD, int G, bool WD, bool Q8, bool SMP, bool KV8, int MT = 1>
__device__ __forceinline__ void compute_loop(const KernelArgs& a, const Lds& L, int bid, int wave, int lane,
                                             int block_rows) {
  constexpr int B = STREAM_BATCH;
  constexpr int NB = stream_sets<HD, G>();
  constexpr int NP = NB * B / 2;  // (K, V) register pairs of the attention ring
  const int c = wave - 1;
  // The abort word lives in LDS and is written and read only on either side of a barrier (which
  // orders them), so plain accesses: the compiler then emits LDS instructions.  A volatile access
  // through this generic pointer would be a FLAT access, whose wait also drains every outstanding
  // global load and store of the wavefront (its prefetch, its last publish).
  int* smi = reinterpret_cast<int*>(L.small);
  Stream<B, NB> st;
  {
    const Range r = next_gemv(L.segs, a.n_waves, -1, block_rows, c);
#pragma unroll
    for (int h = 0; h < NB; ++h) load_gemv_batch<B>(st.v + h * B, a.packed, r, h, lane);
    st.k = r.k;
    st.r0 = r.r0;
    st.sk = -1;
    st.ls = 0;
  }
  // this wave's staging area: LDS pointer (reads) and LDS byte address (direct-to-LDS loads)
  const float* stage_w = L.stage + c * (a.stage_batches * B * (CHUNK_BYTES / 4));
  const uint32_t stage_lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) float*)stage_w;
  int tok_unused = 0;
  bool stop = false;
  for (int step = 0; step < a.n_steps && !stop; ++step) {
    const uint32_t par = step_parity(step);
    const int pos = a.pos0 + step * MT;  // the step's first position
    const int64_t L_att = (int64_t)pos + MT;
    for (int k = 0; k < a.n_waves; ++k) {
      const TileDesc t = tile_of(L, k);
      const WaveDesc wd = wave_of(L, k);
      const int layer = wd.layer;
      uint64_t* ts = a.trace && c == 0 ? reinterpret_cast<uint64_t*>(L.small + SM_CTRACE) + (k & 1) * 8 : nullptr;
      if (ts && lane < TS_COUNT) ts[lane] = 0;
      uint64_t* wdone = a.trace ? reinterpret_cast<uint64_t*>(L.small + SM_WDONE) + (k & 1) * 8 + wave : nullptr;
      if (wdone && lane == 0) *wdone = 0;
      // The stream plan of the tile's first block -- its chunk range and what the registers
      // fetch once its last batches are in flight: the next block, the KV rows of this worker's
      // attention split when that is its next tile, or the next GEMV tile -- worked out before
      // the inputs arrive, so that streaming starts right after barrier A.
      const SegDesc sd = L.segs[k];
      const TileDesc tn = tile_of(L, k + 1 < a.n_waves ? k + 1 : 0);
      const bool next_attn = k + 1 < a.n_waves && tn.kind == KIND_ATTN;
      const Range ng0 = next_gemv(L.segs, a.n_waves, k, block_rows, c);
      const Range r_first0 = block_range(sd, k, 0, block_rows, c);
      const int rows = sc(sd.rows);
      const bool one_block = block_rows >= rows;
      const Range nr_first0 = !one_block ? block_range(sd, k, block_rows, block_rows, c) : next_attn ? no_range() : ng0;
      const bool kv_first0 = one_block && next_attn;
      KvOpen<NP> ko = kv_open<HD, NP, KV8, MT>(a, layer, tn.row0, tn.nrows, L_att, c, lane);
      Range ng = ng0, r_first = r_first0, nr_first = nr_first0;
      int kv_first = kv_first0;
      pin(ng);
      pin(r_first);
      pin(nr_first);
      pin(kv_first);
      pin(ko);
      // Batches 2 .. of a first block into the LDS area while this tile's inputs are outstanding
      // (range tails prefetch batches 0 and 1 into registers): a tile whose share streams beyond
      // its register prefetch stages its own; one whose share fits the registers stages the next
      // GEMV tile's, so that the staging lands during a wait that is already there (its own
      // inputs) instead of lengthening the next tile's.  Not issued with the tail prefetch: a
      // wavefront's outstanding loads are bounded, and the issue would stall the tile's end.
      // The next tile's batches are staged only in the wave right before it, by a GEMV tile that
      // fits the registers or by a worker without a tile in this wave (no input gather there: the
      // staging lands while the worker waits for the next tile's inputs).  The area holds one
      // tile's batches at a time (st.sk = -1 once they are consumed).
      if ((is_gemv(t.kind) || t.kind == KIND_NONE) && st.sk < 0) {
        const int own = is_gemv(t.kind) && r_first.i < r_first.ihi ? (r_first.ihi - r_first.i + B - 1) / B : 0;
        const Range& sr = own > NB ? r_first : ng;
        if (own > NB || (ng.k == k + 1 && ng.r0 == 0)) {
          // own staging lands during this tile's input wait and delays its end: one batch, which
          // arrives within that wait; the next tile's staging may take the whole area
          // (a plan without a staging area stages nothing: decode plans always have one, which the
          // plan validator checks, so only the multi-token instantiations test for it)
          const int own_limit = MT > 1 ? (a.stage_batches > 0 ? 1 : 0) : 1;
          st.ls = stage_range<B, NB>(a.packed, sr, own > NB ? own_limit : a.stage_batches, lane, stage_lds);
          st.sk = st.ls > 0 ? sr.k : -1;
        }
      }
      if (gather_inputs<HD, G, false, WD, Q8, SMP, KV8, MT>(a, L, bid, wave, lane, k, t, wd, step, par, tok_unused))
        smi[SM_ABORT] = 1;
      stamp(ts, TS_GATHERED, lane);
      __syncthreads();  // P
      if (smi[SM_ABORT]) {
        stop = true;
        break;
      }
      if (needs_barrier_a(a, t)) {
        lds_prologue<HD, G, Q8, KV8, MT>(a, L, wave, lane, t, layer, pos);
        __syncthreads();  // A
      }
      stamp(ts, TS_AFTER_A, lane);
      if (is_gemv(t.kind)) {
        for (int r0 = 0; r0 < rows; r0 += block_rows) {
          const bool last_block = r0 + block_rows >= rows;
          const Range r = r0 == 0 ? r_first : block_range(sd, k, r0, block_rows, c);
          if (r.i < r.ihi) {
            const Range nr = r0 == 0 ? nr_first
                             : !last_block ? block_range(sd, k, r0 + block_rows, block_rows, c)
                             : next_attn ? no_range()
                                         : ng;
            const bool kv_next = r0 == 0 ? kv_first : last_block && next_attn;
            stream_range<B, NB, Q8, MT>(
                L, a.packed, r, c, lane, st, st.k == k && st.r0 == r0,
                [&](int h) { return select_src<B>(kv_next, kv_half_src<B, NP>(ko, h), gemv_src<B>(a.packed, nr, h, lane)); },
                stage_w, r0 == 0 ? ts : nullptr, t.kind == KIND_O ? o_in_stride<MT>(a) : a.lds_vec_floats,
                block_rows * NCOMP);
            st.k = kv_next ? k + 1 : nr.k;
            st.r0 = kv_next ? 0 : nr.r0;
            if (r0 == 0) stamp(ts, TS_DONE, lane);
            if (r0 == 0 && wdone && lane == 0) *wdone = wall_clock64();
          }
          __syncthreads();                              // B
          if (r0 + block_rows < rows) __syncthreads();  // C
        }
      } else if (t.kind == KIND_ATTN) {
        compute_attention<HD, G, B, NB, KV8, MT>(a, L, k, c, lane, layer, t.row0, t.nrows, L_att, st, [&](int h) {
          load_gemv_batch<B>(st.v + h * B, a.packed, ng, h, lane);
        }, ts);
        st.k = ng.k;
        st.r0 = ng.r0;
        stamp(ts, TS_DONE, lane);
        if (wdone && lane == 0) *wdone = wall_clock64();
        __syncthreads();  // B
        attn_merge_phase<HD, G, MT>(L, wave, lane);
        __syncthreads();  // E
      }
    }
  }
  // the last range's tail prefetched (into registers and the LDS area) for a range that does not
  // come: let those loads land before the wavefront ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Q8: weight-only INT8 GEMV tiles (INT8 codes, per-row FP32 scales); else BF16 weights.
// SMP: sampled decoding (top-k / top-p draw from every worker's candidates); else greedy.
// KV8: INT8 KV cache (codes, per-position scales, smoothed keys); else BF16 rows.
// MT: positions per step (1 decode; 2 .. MAX_STEP_TOKENS: teacher-forced verify steps whose tiles
// run all MT positions, each weight stream serving them all).
template <int HD, int G, bool WD, bool Q8, bool SMP, bool KV8, int MT = 1>
__global__ void __launch_bounds__(BLOCK_THREADS, 1) tiles_worker(KernelArgs args) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  const KernelArgs& a = args;
  Lds L;
  L.stage = reinterpret_cast<float*>(lds_raw);
  L.vec = L.stage + a.lds_stage_floats;
  L.part = L.vec + MT * a.lds_vec_floats;  // (lds_vec_floats per position of the step)
  L.xres = L.part + a.lds_part_floats;
  L.scl = L.xres + (Q8 ? a.lds_xres_floats - MAX_BLOCK_ROWS : 0);  // (INT8 plans reserve a block's scales there)
  L.small = L.xres + a.lds_xres_floats;
  L.segs = reinterpret_cast<SegDesc*>(L.small + SMALL_FLOATS);
  L.tiles = reinterpret_cast<TileDesc*>(L.segs + a.n_waves);
  L.waves = reinterpret_cast<WaveDesc*>(L.tiles + a.n_waves);
  L.lsmall = reinterpret_cast<LayerSmall*>(L.waves + a.n_waves);
  const int tid = threadIdx.x, lane = tid & 63, bid = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int k = tid; k < a.n_waves; k += BLOCK_THREADS) {
    const TileDesc t = a.tiles[(int64_t)k * a.W + bid];
    SegDesc s;
    s.woff = t.woff;
    s.chunks_per_row = t.kpad / chunk_cols<Q8>();
    s.rows = is_gemv(t.kind) ? (t.kind == KIND_GU ? 2 * t.nrows : t.nrows) : 0;
    L.segs[k] = s;
    L.tiles[k] = t;
    L.waves[k] = a.waves[k];
  }
  for (int l = tid; l < a.n_layers; l += BLOCK_THREADS) L.lsmall[l] = a.small[l];
  if (tid == 0) reinterpret_cast<int*>(L.small)[SM_ABORT] = 0;
  __syncthreads();
  // The schedule as loaded (this worker's tiles, every wave descriptor, every layer's gain offsets:
  // one run of 32-bit words in LDS) must hash to what the host computed when it built the plan, and
  // the plan must carry this kernel's build id; otherwise every wavefront of this worker leaves before
  // using any of it, and the abort word makes the other workers leave at their next wait.
  if (wave == 0) {
    const uint32_t* words = reinterpret_cast<const uint32_t*>(L.tiles);
    const int nwords = a.n_waves * (int)((sizeof(TileDesc) + sizeof(WaveDesc)) / 4) + a.n_layers * (int)(sizeof(LayerSmall) / 4);
    uint64_t hs = 0;
    for (int i = lane; i < nwords; i += 64) hs += table_mix(((uint64_t)i << 32) | words[i]);
    for (int off = 32; off >= 1; off >>= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)hs, off), hi = __shfl_xor((uint32_t)(hs >> 32), off);
      hs += ((uint64_t)hi << 32) | lo;
    }
    const bool bad = hs != a.table_check[bid] || a.table_check[a.W] != (uint64_t)TILES_BUILD_ID;
    if (bad && lane == 0) {
      st_u32(a.sync + SYNC_STATUS_WORD, STATUS_TABLES);
      st_u32(a.sync + SYNC_ABORT_WORD, 1u);
      reinterpret_cast<int*>(L.small)[SM_ABORT] = 1;
    }
  }
  __syncthreads();
  if (reinterpret_cast<const int*>(L.small)[SM_ABORT]) return;
  // rows per GEMV block: the partial area's worth (MT > 1: per position, at most MAX_BLOCK_ROWS).  The
  // INT8 scale registers and the sampled candidates of a block hold MAX_BLOCK_ROWS rows: the plan
  // validator rejects INT8 and sampling plans with a longer tile where blocks may be longer.
  const int block_rows = MT > 1 ? min((a.lds_part_floats / (NCOMP * MT)) & ~1, MAX_BLOCK_ROWS)
                                : (a.lds_part_floats / NCOMP) & ~1;
  if (wave == 0) control_loop<HD, G, WD, Q8, SMP, KV8, MT>(a, L, bid, lane, block_rows);
  else compute_loop<HD, G, WD, Q8, SMP, KV8, MT>(a, L, bid, wave, lane, block_rows);
}

// ---------------------------------------------------------------------------
// stream-read ceiling: what HBM delivers to streams of the decode kernel's load form (16-byte
// non-temporal loads, one 1 KB chunk per wavefront instruction), each wavefront reading one
// contiguous share with STREAM_DEPTH chunks in flight; an XOR of everything read goes to `sink`
#ifndef TILES_WORKER_UNIT
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(BLOCK_THREADS) stream_read(const uint8_t* __restrict__ p, int64_t chunks_per_wave,
                                                            uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * NWAVES + (threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t r = rsrc(p + w * chunks_per_wave * CHUNK_BYTES);
  uint32_t x = 0;
  for (int64_t i = 0; i < chunks_per_wave; i += STREAM_DEPTH) {
    u32x4 v[STREAM_DEPTH];
#pragma unroll
    for (int u = 0; u < STREAM_DEPTH; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)lane * 16u, (uint32_t)(i + u) * CHUNK_BYTES, NT);
#pragma unroll
    for (int u = 0; u < STREAM_DEPTH; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off);
  if (lane == 0) atomicXor(sink, x);
}

hipError_t launch_stream_read(const uint8_t* p, int64_t bytes, int n_groups, uint32_t* sink, hipStream_t stream) {
  const int64_t per_wave = bytes / CHUNK_BYTES / ((int64_t)n_groups * NWAVES);
  hipLaunchKernelGGL(stream_read, dim3(n_groups), dim3(BLOCK_THREADS), 0, stream, p, per_wave, sink);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// edge latency floor: workgroup 0 and workgroup `peer` (one lane each) pass a counter back and
// forth through two words, with the decode kernel's publish (agent-scope store) and poll
// (device-coherent load) forms.  Every wait is bounded by `spin_limit` polls; a wait that gives
// up ends the exchange and sets out[1] (peer) or out[2] (workgroup 0).  The other workgroups of
// the grid leave at once.
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(64) edge_pingpong(uint32_t* words, int peer, int iters, uint32_t spin_limit,
                                                    uint64_t* __restrict__ out) {
  const int b = blockIdx.x;
  if ((b != 0 && b != peer) || threadIdx.x != 0) return;
  const __amdgpu_buffer_rsrc_t r = rsrc(words);
  // workgroup 0 writes word 0 and polls word 16 (a separate 64-byte line); the peer the reverse
  const uint32_t in_off = b == 0 ? 64u : 0u;
  uint32_t* mine = b == 0 ? words : words + 16;
  const uint64_t t0 = wall_clock64();
  bool gave_up = false;
  for (int i = 1; i <= iters && !gave_up; ++i) {
    if (b == 0) st_u32(mine, (uint32_t)i);
    uint32_t spins = 0;
    for (;;) {
      // the fence keeps every round's load: the compiler sees no writer of the word, and would
      // otherwise read it once and fold the wait into a single test
      COMPILER_FENCE();
      if (__builtin_amdgcn_raw_buffer_load_b32(r, in_off, 0, SC1) == (uint32_t)i) break;
      if (++spins >= spin_limit) {
        gave_up = true;
        break;
      }
    }
    if (b != 0 && !gave_up) st_u32(mine, (uint32_t)i);
  }
  const uint64_t t1 = wall_clock64();
  if (b == 0) {
    out[0] = t1 - t0;
    out[2] = gave_up;
  } else {
    out[1] = gave_up;
  }
}

hipError_t launch_edge_latency(uint32_t* words, int peer, int iters, uint32_t spin_limit, uint64_t* out,
                               hipStream_t stream) {
  hipLaunchKernelGGL(edge_pingpong, dim3(peer + 1), dim3(64), 0, stream, words, peer, iters, spin_limit, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// launch helpers: buffer fill (before every decode launch) and weight packing (plan creation)
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256) fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

hipError_t launch_fill(uint32_t* p, int64_t n, uint32_t v, hipStream_t stream) {
  const int64_t blocks = (n + 255) / 256;
  const int grid = blocks < 1024 ? (blocks > 0 ? (int)blocks : 1) : 1024;
  hipLaunchKernelGGL(fill_u32, dim3(grid), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

// `nblk` blocks of `count` 16-bit words, `stride` words apart (debug poison of KV rows).
__global__ void __launch_bounds__(256) fill_u16_blocks(uint16_t* __restrict__ p, int64_t stride, int64_t count, uint16_t v) {
  uint16_t* b = p + (int64_t)blockIdx.x * stride;
  for (int64_t i = threadIdx.x; i < count; i += 256) b[i] = v;
}

hipError_t launch_fill_blocks(uint16_t* p, int nblk, int64_t stride, int64_t count, uint16_t v, hipStream_t stream) {
  if (nblk < 1 || count < 1) return hipSuccess;
  hipLaunchKernelGGL(fill_u16_blocks, dim3(nblk), dim3(256), 0, stream, p, stride, count, v);
  return hipGetLastError();
}

// One launch copies every segment.  Rows whose byte counts and addresses are 16-byte multiples
// move with 16-byte accesses, others with 2-byte ones.
__global__ void __launch_bounds__(256) pack_weights(const PackSeg* __restrict__ segs, int nseg, uint8_t* __restrict__ dst) {
  for (int sidx = blockIdx.x; sidx < nseg; sidx += gridDim.x) {
    const PackSeg g = segs[sidx];
    const bool v16 = ((g.row_bytes | g.src_pitch | g.dst_pitch | g.dst_off | (int64_t)(uintptr_t)g.src) & 15) == 0;
    for (int64_t r = 0; r < g.rows; ++r) {
      const uint8_t* s = g.src + r * g.src_pitch;
      uint8_t* d = dst + g.dst_off + r * g.dst_pitch;
      if (v16) {
        for (int64_t b = (int64_t)threadIdx.x * 16; b < g.row_bytes; b += 256 * 16)
          *reinterpret_cast<u32x4*>(d + b) = *reinterpret_cast<const u32x4*>(s + b);
      } else {
        for (int64_t b = (int64_t)threadIdx.x * 2; b < g.row_bytes; b += 256 * 2)
          *reinterpret_cast<uint16_t*>(d + b) = *reinterpret_cast<const uint16_t*>(s + b);
      }
    }
  }
}

// INT8 KV cache conversion of a BF16 cache prefix ("History and roadmap" (TileInfer.jl), "M8 so
// far": INT8 KV cache with smoothed keys).  kv_sigma: the largest |K| of every (layer, KV head,
// channel) over positions [0, length), 1 for a channel that is zero there; one block per KV head.
__global__ void __launch_bounds__(256) kv_sigma(const uint16_t* __restrict__ k, int64_t cap, int64_t length, int hd,
                                                float* __restrict__ sigma) {
  __shared__ float red[256];
  const int64_t head = blockIdx.x;
  const int np = 256 / hd, c = threadIdx.x % hd, pl = threadIdx.x / hd;
  float m = 0.f;
  if (pl < np)
    for (int64_t p = pl; p < length; p += np) m = fmaxf(m, fabsf(bf16_to_f32(k[(head * cap + p) * hd + c])));
  red[threadIdx.x] = m;
  __syncthreads();
  if (pl == 0) {
    for (int j = 1; j < np; ++j) m = fmaxf(m, red[j * hd + c]);
    sigma[head * hd + c] = m > 0.f ? m : 1.f;
  }
}

// kv_quantize: every row (head, position < length) of a BF16 cache as symmetric INT8 codes and an
// FP32 scale, divided by sigma first when given (keys); one wavefront per row, head_dim <= 128.  The
// codes go to the interleaved INT8 cache (rows of 2 x head_dim bytes; per group of 8 dimensions the
// K codes, then the V codes): `vpart` is 0 for K, 8 for V.
__global__ void __launch_bounds__(256) kv_quantize(const uint16_t* __restrict__ src, int64_t cap, int64_t length,
                                                   int hd, int64_t nheads, const float* __restrict__ sigma,
                                                   int8_t* __restrict__ codes, int vpart, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t nrows = nheads * length;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < nrows; r += (int64_t)gridDim.x * 4) {
    const int64_t head = r / length, p = r - head * length;
    const int64_t row = head * cap + p;
    float x[2] = {0.f, 0.f}, am = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = lane + 64 * i;
      if (c < hd) {
        x[i] = bf16_to_f32(src[row * hd + c]);
        if (sigma) x[i] = __fdiv_rn(x[i], sigma[head * hd + c]);
        am = fmaxf(am, fabsf(x[i]));
      }
    }
    for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
    const float sc = __fdiv_rn(am, 127.f);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = lane + 64 * i;
      if (c < hd) codes[row * hd * 2 + (c >> 3) * 16 + vpart + (c & 7)] = (int8_t)(int)kv_code(x[i], sc);
    }
    if (lane == 0) scales[row] = sc;
  }
}

hipError_t launch_kv_convert(const uint16_t* k, const uint16_t* v, int64_t cap, int64_t length, int hd, int64_t nheads,
                             int8_t* codes, float* ks, float* vs, float* sigma, hipStream_t stream) {
  hipLaunchKernelGGL(kv_sigma, dim3((unsigned)nheads), dim3(256), 0, stream, k, cap, length, hd, sigma);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = nheads * length;
  const int64_t blocks = (rows + 3) / 4;
  const unsigned grid = (unsigned)(blocks < 1 ? 1 : blocks > 65536 ? 65536 : blocks);
  hipLaunchKernelGGL(kv_quantize, dim3(grid), dim3(256), 0, stream, k, cap, length, hd, nheads, sigma, codes, 0, ks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv_quantize, dim3(grid), dim3(256), 0, stream, v, cap, length, hd, nheads, nullptr, codes, 8, vs);
  return hipGetLastError();
}

hipError_t launch_pack(const PackSeg* segs, int nseg, uint8_t* dst, hipStream_t stream) {
  const int grid = nseg < 4096 ? (nseg > 0 ? nseg : 1) : 4096;
  hipLaunchKernelGGL(pack_weights, dim3(grid), dim3(256), 0, stream, segs, nseg, dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// scratch of the allocation-free decode entry point (tiles_decode_noalloc): the tagged-data
// buffers, the LM-head partials and the status words of a launch, in one file-scope array per
// GPU instead of plan-owned memory.  Host code never uses the array's name as an address (on the
// host it names a stand-in): the device address comes from hipGetSymbolAddress, once per device,
// with that device current.
// ---------------------------------------------------------------------------

static __device__ __align__(256) uint32_t scratch[NOALLOC_SCRATCH_BYTES / 4];

hipError_t noalloc_scratch(int device, uint32_t** out) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static uint32_t* ptr[MAX_DEVICES] = {};
  if (device < 0 || device >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[device] = static_cast<uint32_t*>(p);
  }
  *out = ptr[device];
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// host-visible handles of the instantiations
// ---------------------------------------------------------------------------

#endif  // TILES_WORKER_UNIT

#ifdef TILES_WORKER_UNIT
// The worker for a head size and query heads per attention tile, for one weight format, token
// selection and KV format (each worker unit instantiates one combination, so that the build
// compiles them in parallel).
template <bool Q8, bool SMP, bool KV8>
const void* worker_for(int head_dim, int group) {
  if (head_dim == 64) {
    switch (group) {
      case 1: return reinterpret_cast<const void*>(&tiles_worker<64, 1, false, Q8, SMP, KV8>);
      case 2: return reinterpret_cast<const void*>(&tiles_worker<64, 2, false, Q8, SMP, KV8>);
      case 3: return reinterpret_cast<const void*>(&tiles_worker<64, 3, false, Q8, SMP, KV8>);
      case 4: return reinterpret_cast<const void*>(&tiles_worker<64, 4, false, Q8, SMP, KV8>);
    }
  } else if (head_dim == 128) {
    switch (group) {
      case 1: return reinterpret_cast<const void*>(&tiles_worker<128, 1, false, Q8, SMP, KV8>);
      case 2: return reinterpret_cast<const void*>(&tiles_worker<128, 2, false, Q8, SMP, KV8>);
      case 3: return reinterpret_cast<const void*>(&tiles_worker<128, 3, false, Q8, SMP, KV8>);
      case 4: return reinterpret_cast<const void*>(&tiles_worker<128, 4, false, Q8, SMP, KV8>);
    }
  }
  return nullptr;
}
// The multi-token (verify-plan) worker for a head size, query heads per attention tile and positions
// per step, greedy, BF16 or INT8 cache: query rows (group x positions) at most MAX_GROUP.
template <bool Q8, bool KV8>
const void* worker_mt_for(int head_dim, int group, int mt) {
  if (head_dim == 64) {
    if (mt == 2 && group == 1) return reinterpret_cast<const void*>(&tiles_worker<64, 1, false, Q8, false, KV8, 2>);
    if (mt == 2 && group == 2) return reinterpret_cast<const void*>(&tiles_worker<64, 2, false, Q8, false, KV8, 2>);
    if (mt == 3 && group == 1) return reinterpret_cast<const void*>(&tiles_worker<64, 1, false, Q8, false, KV8, 3>);
    if (mt == 4 && group == 1) return reinterpret_cast<const void*>(&tiles_worker<64, 1, false, Q8, false, KV8, 4>);
  } else if (head_dim == 128) {
    if (mt == 2 && group == 1) return reinterpret_cast<const void*>(&tiles_worker<128, 1, false, Q8, false, KV8, 2>);
    if (mt == 2 && group == 2) return reinterpret_cast<const void*>(&tiles_worker<128, 2, false, Q8, false, KV8, 2>);
    if (mt == 3 && group == 1) return reinterpret_cast<const void*>(&tiles_worker<128, 1, false, Q8, false, KV8, 3>);
    if (mt == 4 && group == 1) return reinterpret_cast<const void*>(&tiles_worker<128, 1, false, Q8, false, KV8, 4>);
  }
  return nullptr;
}
#else
// (defined by the worker units; variant: INT8 weights * 4 + sampled * 2 + INT8 KV)
const void* worker_unit_0(int head_dim, int group);
const void* worker_unit_1(int head_dim, int group);
const void* worker_unit_2(int head_dim, int group);
const void* worker_unit_3(int head_dim, int group);
const void* worker_unit_4(int head_dim, int group);
const void* worker_unit_5(int head_dim, int group);
const void* worker_unit_6(int head_dim, int group);
const void* worker_unit_7(int head_dim, int group);
const void* worker_watchdog(int head_dim);
const void* worker_mt_unit_0(int head_dim, int group, int mt);  // BF16 weights, BF16 KV
const void* worker_mt_unit_1(int head_dim, int group, int mt);  // INT8 weights, BF16 KV
const void* worker_mt_unit_2(int head_dim, int group, int mt);  // BF16 weights, INT8 KV
const void* worker_mt_unit_3(int head_dim, int group, int mt);  // INT8 weights, INT8 KV

const void* worker_unit(int variant, int head_dim, int group) {
  switch (variant) {
    case 0: return worker_unit_0(head_dim, group);
    case 1: return worker_unit_1(head_dim, group);
    case 2: return worker_unit_2(head_dim, group);
    case 3: return worker_unit_3(head_dim, group);
    case 4: return worker_unit_4(head_dim, group);
    case 5: return worker_unit_5(head_dim, group);
    case 6: return worker_unit_6(head_dim, group);
    case 7: return worker_unit_7(head_dim, group);
  }
  return nullptr;
}

// The worker for a head size, query heads per attention tile, weight format, token selection, KV
// format and positions per step; `short_watchdog` selects the test instantiation whose waits check
// their watchdog every polling round (BF16 weights and KV, greedy, one query head per tile, one
// position per step only).
const void* worker_kernel(int head_dim, int group, bool short_watchdog, bool q8, bool sampled, bool kv8, int mt) {
  if (mt > 1) {
    if (short_watchdog || sampled) return nullptr;
    if (kv8) return q8 ? worker_mt_unit_3(head_dim, group, mt) : worker_mt_unit_2(head_dim, group, mt);
    return q8 ? worker_mt_unit_1(head_dim, group, mt) : worker_mt_unit_0(head_dim, group, mt);
  }
  if (short_watchdog) return group == 1 && !q8 && !sampled && !kv8 ? worker_watchdog(head_dim) : nullptr;
  return worker_unit((q8 ? 4 : 0) + (sampled ? 2 : 0) + (kv8 ? 1 : 0), head_dim, group);
}
#endif

}  // namespace tiles
