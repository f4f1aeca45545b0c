// The persistent tile worker for gfx950 (CDNA4).
//
// One workgroup per compute unit executes the static per-step schedule built by the
// host planner: for every decoded token, for every wave, run this worker's tile (if
// any), then wait at a grid barrier.  The kernel makes no scheduling decision of its
// own ("Tiles: Scheduling LLM Decoding as a Graph of Tiles", intro): tiles, workers,
// wave order and split boundaries are all fixed by the plan and the attended length.
//
// Workgroup organisation (512 threads = 8 wavefronts):
//   * wavefront 0 is the control wave: it stages each tile's input vector in LDS
//     (folding RMSNorm, the embedding lookup, the split merge, q/k norm, RoPE and the
//     KV write), runs the epilogues (residual add, SwiGLU, partial argmax), performs
//     every global store and takes part in the grid barrier;
//   * wavefronts 1..7 are compute waves.  Each streams its share of the worker's packed
//     weights through its own LDS ring with direct-to-LDS 16-byte loads
//     (global_load_lds_dwordx4).  The ring is refilled in consumption order across
//     wave boundaries, so while the workgroup waits at a grid barrier the weights of
//     the next tiles keep arriving: weights do not depend on activations, only the dot
//     products do (the Tiles page credits this prefetch idea to the megakernel it
//     builds on).
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
//   * LM head: logits and a (max, lowest index) partial per worker; after the last
//     barrier of a step every worker reduces all partials in worker order.
//
// Cross-worker data (activations, partials, barrier words, KV rows written in this
// launch) moves with device-coherent accesses (sc1 cache policy), so no L2 write-back
// or invalidate is needed; the control wave waits for its stores to complete before it
// signals the barrier.  Weights are read with plain loads into LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan_types.h"

namespace tiles {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int SC1 = 16;  // buffer-instruction cache policy bit: device-coherent access

// ---------------------------------------------------------------------------
// coherent memory helpers
// ---------------------------------------------------------------------------

__device__ inline uint32_t ld_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_f32(const float* p) {
  return __uint_as_float(ld_u32(reinterpret_cast<const uint32_t*>(p)));
}
__device__ inline void st_f32(float* p, float v) { st_u32(reinterpret_cast<uint32_t*>(p), __float_as_uint(v)); }
__device__ inline void st_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t ld_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Buffer descriptor over a scratch array (byte offsets < 4 GB).  Device-coherent buffer
// loads through it are plain (non-atomic) loads the compiler can issue back to back.
__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0xffffffffu, 0x00020000);
}
__device__ inline u32x4 cld4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, SC1);
}
__device__ inline f32x4 as_f32x4(u32x4 u) {
  return f32x4{__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)};
}
#define COMPILER_FENCE() asm volatile("" ::: "memory")

__device__ inline float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round-to-nearest-even FP32 -> BF16 (NaN kept quiet).
__device__ inline uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ inline float bf16_round(float f) { return __uint_as_float(f32_to_bf16_bits(f) << 16); }

// ---------------------------------------------------------------------------
// wavefront reductions (DPP butterflies; every lane ends with the same value)
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <-> 7-i within 8
constexpr int DPP_MIRROR = 0x140;       // lane i <-> 15-i within 16

__device__ inline float sum8(float v) {
  v += dpp<DPP_XOR1>(v);
  v += dpp<DPP_XOR2>(v);
  v += dpp<DPP_HALF_MIRROR>(v);
  return v;
}
__device__ inline float sum16(float v) {
  v = sum8(v);
  v += dpp<DPP_MIRROR>(v);
  return v;
}
__device__ inline float wave_sum(float v) {
  v = sum16(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// ---------------------------------------------------------------------------
// LDS layout (dynamic): vec | part | small | segs.
// small[] words written by the control wave before barrier A of every wave:
constexpr int SM_DONE = 0;   // int: no more waves (end of launch or abort)
constexpr int SM_KIND = 1;   // int: tile kind
constexpr int SM_ROW0 = 2;   // int
constexpr int SM_NROWS = 3;  // int
constexpr int SM_LAYER = 4;  // int
constexpr int SM_C = 5;      // int: chunks per GEMV row
constexpr int SM_POS = 6;    // int: position of the current step
// ---------------------------------------------------------------------------

struct Lds {
  float* vec;
  float* part;
  float* small;
  SegDesc* segs;
};

__device__ inline bool is_gemv(int kind) {
  return kind == KIND_QKV || kind == KIND_O || kind == KIND_GU || kind == KIND_DOWN || kind == KIND_LM;
}
// chunk range of compute wave c over n chunks
__device__ inline int chunk_lo(int n, int c) { return (int)(((int64_t)n * c) / NCOMP); }

// ---------------------------------------------------------------------------
// compute wave: weight streaming.  Each compute wave reads its share of a GEMV block (a
// contiguous chunk range) with 16-byte loads into registers, double-buffered in batches of
// STREAM_BATCH chunks.  Before a tile's last batch is consumed, the wave issues the loads of
// the first PREFETCH_CHUNKS chunks of its next GEMV tile, so those bytes arrive while the
// workgroup goes through the epilogue, the grid barrier and the next prologue.
// ---------------------------------------------------------------------------

constexpr int STREAM_BATCH = 4;
constexpr int PREFETCH_CHUNKS = 12;  // register budget: 8 are used when a KV head serves 3-4 query heads

__device__ inline float dot8(const u32x4 w, const float* v) {
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

// Chunk range [i, ihi) of compute wave c in block r0 of a GEMV segment.
struct Range {
  int k;         // schedule wave (-1: none)
  int C;         // chunks per row
  int i, ihi;
  int64_t base;  // byte offset of the block's first chunk
};

__device__ inline Range block_range(const SegDesc& s, int k, int r0, int block_rows, int c) {
  Range r;
  r.k = k;
  r.C = s.chunks_per_row;
  const int nr = min(block_rows, s.rows - r0);
  const int n = nr * s.chunks_per_row;
  r.i = chunk_lo(n, c);
  r.ihi = chunk_lo(n, c + 1);
  r.base = s.woff + (int64_t)r0 * s.chunks_per_row * CHUNK_BYTES;
  return r;
}

// First block of the next GEMV wave after `k` (wrapping into the next step) in which compute
// wave c has chunks; k = -1 when there is none.
__device__ inline Range next_gemv(const SegDesc* segs, int n_waves, int k, int block_rows, int c) {
  for (int d = 1; d <= n_waves; ++d) {
    const int kk = (k + d) % n_waves;
    if (segs[kk].rows == 0) continue;
    const Range r = block_range(segs[kk], kk, 0, block_rows, c);
    if (r.i < r.ihi) return r;
  }
  Range none;
  none.k = -1;
  none.C = 1;
  none.i = none.ihi = 0;
  none.base = 0;
  return none;
}

template <int PF>
struct Prefetch {
  u32x4 v[PF];
  int n;  // valid entries
  int k;  // schedule wave they belong to (-1: none)
};

template <int PF>
__device__ inline void issue_prefetch(Prefetch<PF>& pf, const Range& r, const uint8_t* packed, int lane) {
  pf.k = r.k;
  pf.n = r.k < 0 ? 0 : min(PF, r.ihi - r.i);
  const u32x4* g = reinterpret_cast<const u32x4*>(packed + r.base) + (int64_t)r.i * 64 + lane;
#pragma unroll
  for (int u = 0; u < PF; ++u)
    if (u < pf.n) pf.v[u] = __builtin_nontemporal_load(g + u * 64);
}

// Consume chunks [r.i, r.ihi): the first `npf` come from pf (when use_pf), the rest are streamed.
// Per-row partial sums go to part[row * NCOMP + c].  When `refill` is set, the loads of the next
// tile's prefetch are issued as early as the current tile allows.
template <int PF>
__device__ void stream_range(const Lds& L, const uint8_t* packed, const Range& r, int c, int lane, Prefetch<PF>& pf,
                             bool use_pf, bool refill, const Range& nxt) {
  const int C = r.C;
  int i = r.i;
  const int ihi = r.ihi;
  int row = i / C, seg = i - row * C;
  float acc = 0.f;
  const float* vlane = L.vec + lane * 8;
  const u32x4* g = reinterpret_cast<const u32x4*>(packed + r.base) + lane;
  const int npf = use_pf ? pf.n : 0;
  auto consume = [&](const u32x4& w) {
    acc += dot8(w, vlane + seg * CHUNK_COLS);
    if (++seg == C) {
      const float s = wave_sum(acc);
      if (lane == 0) L.part[row * NCOMP + c] = s;
      acc = 0.f;
      seg = 0;
      ++row;
    }
  };
  // first streamed batch is issued before the prefetched chunks are consumed
  u32x4 wa[STREAM_BATCH], wb[STREAM_BATCH];
  int j = i + npf;
  int na = min(STREAM_BATCH, ihi - j);
#pragma unroll
  for (int u = 0; u < STREAM_BATCH; ++u)
    if (u < na) wa[u] = __builtin_nontemporal_load(g + (int64_t)(j + u) * 64);
#pragma unroll
  for (int u = 0; u < PF; ++u)
    if (u < npf) consume(pf.v[u]);
  bool refilled = false;
  if (na <= 0) {
    if (refill) issue_prefetch(pf, nxt, packed, lane);
    refilled = true;
  }
  while (na > 0) {
    const int jn = j + na;
    const int nb = min(STREAM_BATCH, ihi - jn);
#pragma unroll
    for (int u = 0; u < STREAM_BATCH; ++u)
      if (u < nb) wb[u] = __builtin_nontemporal_load(g + (int64_t)(jn + u) * 64);
    if (nb <= 0 && !refilled) {  // last batch in flight: start the next tile's loads now
      if (refill) issue_prefetch(pf, nxt, packed, lane);
      refilled = true;
    }
#pragma unroll
    for (int u = 0; u < STREAM_BATCH; ++u)
      if (u < na) consume(wa[u]);
    j = jn;
    na = nb;
#pragma unroll
    for (int u = 0; u < STREAM_BATCH; ++u) wa[u] = wb[u];
  }
  if (seg != 0) {
    const float s = wave_sum(acc);
    if (lane == 0) L.part[row * NCOMP + c] = s;
  }
}

// total of row r of a block: partials of the compute waves whose ranges touch it, in order
__device__ inline float row_total(const Lds& L, int nr, int C, int r) {
  const int n = nr * C;
  const int first = r * C, last = r * C + C - 1;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCOMP; ++c) {
    const int lo = chunk_lo(n, c), hi = chunk_lo(n, c + 1);
    if (lo < hi && lo <= last && first < hi) s += L.part[r * NCOMP + c];
  }
  return s;
}

// ---------------------------------------------------------------------------
// control wave: prologues
// ---------------------------------------------------------------------------

// Coherent copy of n floats (n % 4 == 0) from a scratch vector into LDS, zero-padded to npad;
// loads are issued in batches of 16 per lane before any is consumed.
__device__ void cw_load_vec(float* dst, const float* src, int n, int npad, int lane) {
  constexpr int B = 16;
  const __amdgpu_buffer_rsrc_t r = rsrc(src);
  COMPILER_FENCE();
  for (int base = 0; base < npad; base += B * 256) {
    u32x4 v[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int i = base + u * 256 + lane * 4;
      v[u] = i < n ? cld4(r, (uint32_t)i * 4) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int i = base + u * 256 + lane * 4;
      if (i < npad) *reinterpret_cast<f32x4*>(dst + i) = as_f32x4(v[u]);
    }
  }
  COMPILER_FENCE();
}

// RMSNorm prologue with the scale folded out: vec[i] = src[i] * gain[i] (i < n), vec[n..npad) = 0,
// and the return value rs = 1 / sqrt(mean(src^2) + eps) multiplies the GEMV results instead
// (W (rs x * g) = rs W (x * g)).  src is an FP32 device-coherent vector or a BF16 embedding
// row; the source and gain loads of a batch are issued together.
__device__ float cw_norm(const Lds& L, int lane, const float* src_f32, const uint16_t* src_bf16, const uint16_t* gain,
                         int n, int npad, float eps) {
  constexpr int B = 8;
  const __amdgpu_buffer_rsrc_t r = rsrc(src_f32 ? (const void*)src_f32 : (const void*)src_bf16);
  float ss = 0.f;
  COMPILER_FENCE();
  for (int base = 0; base < npad; base += B * 256) {
    u32x4 xv[B];
    uint2 gv[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int i = base + u * 256 + lane * 4;
      xv[u] = u32x4{0u, 0u, 0u, 0u};
      gv[u] = uint2{0u, 0u};
      if (i < n) {
        if (src_f32) {
          xv[u] = cld4(r, (uint32_t)i * 4);
        } else {
          const uint2 e = *reinterpret_cast<const uint2*>(src_bf16 + i);
          xv[u] = u32x4{e.x << 16, e.x & 0xffff0000u, e.y << 16, e.y & 0xffff0000u};
        }
        gv[u] = *reinterpret_cast<const uint2*>(gain + i);
      }
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int i = base + u * 256 + lane * 4;
      const f32x4 x = as_f32x4(xv[u]);
      ss += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
      const f32x4 v = {x.x * bf16_lo(gv[u].x), x.y * bf16_hi(gv[u].x), x.z * bf16_lo(gv[u].y), x.w * bf16_hi(gv[u].y)};
      if (i < npad) *reinterpret_cast<f32x4*>(L.vec + i) = v;
    }
  }
  COMPILER_FENCE();
  const float tot = wave_sum(ss);
  return 1.0f / sqrtf(tot / (float)n + eps);
}

// merge the S splits of one query head (Ph -> [S][HD + 2]) for output dim d, fixed split order
__device__ inline float merge_splits(const float* Ph, int S, int HD, int d) {
  float mm = -INFINITY;
  for (int s = 0; s < S; ++s) mm = fmaxf(mm, Ph[s * (HD + 2)]);
  if (mm == -INFINITY) return 0.f;
  float ll = 0.f, aa = 0.f;
  for (int s = 0; s < S; ++s) {
    const float* st = Ph + s * (HD + 2);
    if (st[1] == 0.f) continue;
    const float f = __builtin_amdgcn_exp2f(st[0] - mm);
    ll += f * st[1];
    aa += f * st[2 + d];
  }
  return aa / ll;
}

// Attention tile LDS layout (inside `part`): q[G][HD] (normed, roped, scaled to the base-2
// domain) | kc[HD] (normed, roped, BF16-rounded) | vc[HD] (BF16-rounded) | compute-wave states
// [NCOMP][G][HD + 2] | merged partial [G][HD + 2].  The raw q/k/v are staged in `vec`.
template <int HD, int G>
__device__ inline float* attn_ws(const Lds& L) { return L.part + G * HD + 2 * HD; }
template <int HD, int G>
__device__ inline float* attn_merged(const Lds& L) { return L.part + G * HD + 2 * HD + NCOMP * G * (HD + 2); }

// control wave, before barrier P: raw q (G heads), k, v of KV group g into vec (one batch of loads)
template <int HD, int G>
__device__ void cw_attn_load(const KernelArgs& a, const Lds& L, int lane, int g) {
  constexpr int N = (G + 2) * HD;
  constexpr int B = (N + 255) / 256;
  const __amdgpu_buffer_rsrc_t r = rsrc(a.qkv);
  const int qbase = g * G * HD;
  const int kbase = a.n_heads * HD + g * HD;
  const int vbase = a.n_heads * HD + a.n_kv * HD + g * HD;
  COMPILER_FENCE();
  u32x4 v[B];
#pragma unroll
  for (int u = 0; u < B; ++u) {
    const int i = u * 256 + lane * 4;
    const int src = i < G * HD ? qbase + i : i < (G + 1) * HD ? kbase + (i - G * HD) : vbase + (i - (G + 1) * HD);
    v[u] = i < N ? cld4(r, (uint32_t)src * 4) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < B; ++u) {
    const int i = u * 256 + lane * 4;
    if (i < N) *reinterpret_cast<f32x4*>(L.vec + i) = as_f32x4(v[u]);
  }
  COMPILER_FENCE();
}

// all wavefronts, between barriers P and A: wave u < G normalises (optional) and rotates query
// head u, wave G the key; wave G + 1 rounds the value.  LDS only (plus read-only tables).
template <int HD, int G>
__device__ void attn_lds_prep(const KernelArgs& a, const Lds& L, int wave_index, int lane, int layer, int pos) {
  constexpr int HALF = HD / 2;
  float* q = L.part;
  float* kc = q + G * HD;
  float* vc = kc + HD;
  const float* raw = L.vec;
  if (wave_index <= G) {
    const int u = wave_index;
    float u0 = 0.f, u1 = 0.f;
    if (lane < HALF) {
      u0 = raw[u * HD + lane];
      u1 = raw[u * HD + lane + HALF];
    }
    if (a.small[layer].q_norm >= 0) {
      const float ss = wave_sum(u0 * u0 + u1 * u1);
      const float rs = 1.0f / sqrtf(ss / (float)HD + a.eps);
      const uint16_t* gn =
          reinterpret_cast<const uint16_t*>(a.packed + (u < G ? a.small[layer].q_norm : a.small[layer].k_norm));
      if (lane < HALF) {
        u0 = u0 * rs * bf16_to_f32(gn[lane]);
        u1 = u1 * rs * bf16_to_f32(gn[lane + HALF]);
      }
    }
    if (lane < HALF) {
      const float* cs = a.rope + ((int64_t)pos * HALF + lane) * 2;
      const float co = cs[0], si = cs[1];
      const float r0 = u0 * co - u1 * si;
      const float r1 = u1 * co + u0 * si;
      if (u < G) {
        q[u * HD + lane] = r0 * a.qscale;
        q[u * HD + lane + HALF] = r1 * a.qscale;
      } else {
        kc[lane] = bf16_round(r0);
        kc[lane + HALF] = bf16_round(r1);
      }
    }
  } else if (wave_index == G + 1) {
    for (int i = lane; i < HD; i += 64) vc[i] = bf16_round(raw[(G + 1) * HD + i]);
  }
}

// control wave, after barrier A: the split holding the current position writes its K/V row
template <int HD, int G>
__device__ void cw_attn_kv_write(const KernelArgs& a, const Lds& L, int lane, int layer, int g, int sp,
                                 int64_t L_att) {
  const float* kc = L.part + G * HD;
  const float* vc = kc + HD;
  const int64_t ch = (L_att + a.S - 1) / a.S;
  const int64_t lo = (int64_t)sp * ch;
  const int64_t hi = lo + ch < L_att ? lo + ch : L_att;
  const int64_t cur = L_att - 1;
  if (lo <= cur && cur < hi && lane < HD / 2) {
    const int64_t row = ((int64_t)layer * a.n_kv + g) * a.kv_cap + cur;
    const uint32_t kb = f32_to_bf16_bits(kc[2 * lane]) | (f32_to_bf16_bits(kc[2 * lane + 1]) << 16);
    const uint32_t vb = f32_to_bf16_bits(vc[2 * lane]) | (f32_to_bf16_bits(vc[2 * lane + 1]) << 16);
    st_u32(reinterpret_cast<uint32_t*>(a.kv_k + row * HD) + lane, kb);
    st_u32(reinterpret_cast<uint32_t*>(a.kv_v + row * HD) + lane, vb);
  }
}

// ---------------------------------------------------------------------------
// compute wave: one share of an attention split
// ---------------------------------------------------------------------------

template <int HD>
__device__ inline void unpack8(const u32x4 w, float* f) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

template <int HD, int G>
__device__ void compute_attention(const KernelArgs& a, const Lds& L, int c, int lane, int layer, int g, int sp,
                                  int64_t L_att) {
  const float* q = L.part;
  const float* kc = q + G * HD;
  const float* vc = kc + HD;
  float* ws = attn_ws<HD, G>(L);
  const int64_t ch = (L_att + a.S - 1) / a.S;
  int64_t lo = (int64_t)sp * ch;
  const int64_t hi = lo + ch < L_att ? lo + ch : L_att;
  if (lo > L_att) lo = L_att;
  const int64_t cur = L_att - 1;
  const int64_t kvrow0 = ((int64_t)layer * a.n_kv + g) * a.kv_cap;
  constexpr int LPP = HD / 8;  // lanes per position
  constexpr int P = 64 / LPP;  // positions per load
  constexpr int U = 2;         // position groups per batch (two batches in flight)
  const int64_t n = hi > lo ? hi - lo : 0;
  const int64_t wlo = lo + (n * c) / NCOMP, whi = lo + (n * (c + 1)) / NCOMP;
  const int pp = lane / LPP, dseg = lane % LPP;
  const float* qlane = q + dseg * 8;  // q values are re-read from LDS per use (register budget)
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  const u32x4* kbase_p = reinterpret_cast<const u32x4*>(a.kv_k + kvrow0 * HD);
  const u32x4* vbase_p = reinterpret_cast<const u32x4*>(a.kv_v + kvrow0 * HD);
  const __amdgpu_buffer_rsrc_t rk = rsrc(kbase_p), rv = rsrc(vbase_p);
  auto load = [&](int64_t jb, u32x4* kw, u32x4* vw) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = jb + u * P + pp;
      kw[u] = u32x4{0u, 0u, 0u, 0u};
      vw[u] = u32x4{0u, 0u, 0u, 0u};
      if (j < whi && j != cur) {
        if (j < a.pos0) {  // cached before this launch: streaming loads
          kw[u] = __builtin_nontemporal_load(kbase_p + j * LPP + dseg);
          vw[u] = __builtin_nontemporal_load(vbase_p + j * LPP + dseg);
        } else {           // written by another worker during this launch: device-coherent loads
          kw[u] = cld4(rk, (uint32_t)((j * LPP + dseg) * 16));
          vw[u] = cld4(rv, (uint32_t)((j * LPP + dseg) * 16));
        }
      }
    }
  };
  auto consume = [&](int64_t jb, const u32x4* kw, const u32x4* vw) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = jb + u * P + pp;
      const bool valid = j < whi;
      float kf[8], vf[8];
      if (j == cur) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kf[e] = kc[dseg * 8 + e];
          vf[e] = vc[dseg * 8 + e];
        }
      } else {
        unpack8<HD>(kw[u], kf);
        unpack8<HD>(vw[u], vf);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const f32x4 q0 = *reinterpret_cast<const f32x4*>(qlane + h * HD);
        const f32x4 q1 = *reinterpret_cast<const f32x4*>(qlane + h * HD + 4);
        float d0 = q0.x * kf[0], d1 = q0.y * kf[1];
        d0 = fmaf(q0.z, kf[2], d0);
        d1 = fmaf(q0.w, kf[3], d1);
        d0 = fmaf(q1.x, kf[4], d0);
        d1 = fmaf(q1.y, kf[5], d1);
        d0 = fmaf(q1.z, kf[6], d0);
        d1 = fmaf(q1.w, kf[7], d1);
        float s = d0 + d1;
        s = LPP == 8 ? sum8(s) : sum16(s);
        if (valid) {
          const float mn = fmaxf(m[h], s);
          const float al = __builtin_amdgcn_exp2f(m[h] - mn);
          const float p = __builtin_amdgcn_exp2f(s - mn);
          l[h] = l[h] * al + p;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(acc[h][e], al, p * vf[e]);
          m[h] = mn;
        }
      }
    }
  };
  if (wlo < whi) {
    u32x4 ka[U], va[U], kb[U], vb[U];
    load(wlo, ka, va);
    for (int64_t jb = wlo; jb < whi; jb += 2 * U * P) {
      const int64_t jn = jb + U * P;
      if (jn < whi) load(jn, kb, vb);
      consume(jb, ka, va);
      if (jn >= whi) break;
      const int64_t jnn = jn + U * P;
      if (jnn < whi) load(jnn, ka, va);
      consume(jn, kb, vb);
    }
  }
  // merge the P position groups of this wave (lanes differing by multiples of LPP)
#pragma unroll
  for (int off = LPP; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m2 = __shfl_xor(m[h], off);
      const float l2 = __shfl_xor(l[h], off);
      float a2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) a2[e] = __shfl_xor(acc[h][e], off);
      const float mn = fmaxf(m[h], m2);
      if (mn != -INFINITY) {
        const float f1 = __builtin_amdgcn_exp2f(m[h] - mn), f2 = __builtin_amdgcn_exp2f(m2 - mn);
        l[h] = l[h] * f1 + l2 * f2;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = acc[h][e] * f1 + a2[e] * f2;
        m[h] = mn;
      }
    }
  }
  if (pp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* st = ws + (c * G + h) * (HD + 2);
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
// the tile's partial (m, l, acc) per query head
template <int HD, int G>
__device__ void attn_merge_phase(const Lds& L, int wave_index, int lane) {
  const float* ws = attn_ws<HD, G>(L);
  float* mrg = attn_merged<HD, G>(L);
  for (int idx = wave_index * 64 + lane; idx < G * HD; idx += BLOCK_THREADS) {
    const int h = idx / HD, d = idx % HD;
    float mm = -INFINITY, ll = 0.f, aa = 0.f;
    for (int c = 0; c < NCOMP; ++c) {
      const float* st = ws + (c * G + h) * (HD + 2);
      const float m2 = st[0];
      const float mn = fmaxf(mm, m2);
      if (mn == -INFINITY) continue;
      const float f1 = __builtin_amdgcn_exp2f(mm - mn), f2 = __builtin_amdgcn_exp2f(m2 - mn);
      ll = ll * f1 + st[1] * f2;
      aa = aa * f1 + st[2 + d] * f2;
      mm = mn;
    }
    float* dst = mrg + h * (HD + 2);
    if (d == 0) {
      dst[0] = mm;
      dst[1] = ll;
    }
    dst[2 + d] = aa;
  }
}

// control wave, after barrier E: store the merged partials of query heads g*G .. g*G+G-1, split sp
template <int HD, int G>
__device__ void cw_attn_store(const KernelArgs& a, const Lds& L, int lane, int g, int sp) {
  const float* mrg = attn_merged<HD, G>(L);
  for (int idx = lane; idx < G * (HD + 2); idx += 64) {
    const int h = idx / (HD + 2), e = idx % (HD + 2);
    st_f32(a.part + ((int64_t)(g * G + h) * a.S + sp) * (HD + 2) + e, mrg[idx]);
  }
}

// LDS-only prologue work shared by all eight wavefronts between barriers P and A:
// merging the split partials into the o_proj input vector.  wave_index in [0, NWAVES).
template <int HD, int G>
__device__ inline void prologue_lds_phase(const KernelArgs& a, const Lds& L, int kind, int wave_index, int lane,
                                          int layer, int pos) {
  if (kind == KIND_ATTN) {
    attn_lds_prep<HD, G>(a, L, wave_index, lane, layer, pos);
  } else if (kind == KIND_O && a.combine_in_o) {
    const int nq = a.n_heads * HD;
    for (int i = wave_index * 64 + lane; i < nq; i += BLOCK_THREADS)
      L.vec[i] = merge_splits(L.part + (i / HD) * a.S * (HD + 2), a.S, HD, i % HD);
  }
}

// ---------------------------------------------------------------------------
// grid barrier (control wave): every worker publishes its generation on its own
// 64-byte line and polls all lines.  A watchdog bounds every wait.
// ---------------------------------------------------------------------------

// Spin until every lane's predicate holds; false = released, true = aborted (watchdog or peer abort).
template <typename Ready>
__device__ inline bool cw_spin(const KernelArgs& a, int lane, Ready ready) {
  uint32_t spins = 0;
  for (;;) {
    if (__all(ready())) return false;
    if ((++spins & 63) == 0) {
      if (ld_u32(a.sync + SYNC_ABORT_WORD) != 0) return true;
      if (spins > a.spin_limit) {
        if (lane == 0) {
          st_u32(a.sync + SYNC_STATUS_WORD, 1u);
          st_u32(a.sync + SYNC_ABORT_WORD, 1u);
        }
        return true;
      }
    }
  }
}

__device__ bool cw_grid_barrier(const KernelArgs& a, int bid, int lane, uint32_t gen) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are complete
  uint32_t* arrive = a.sync + SYNC_ARRIVE_BASE;
  uint32_t* release = arrive + (int64_t)a.W * SYNC_LINE_WORDS;
  if (lane == 0) st_u32(arrive + bid * SYNC_LINE_WORDS, gen);
  auto all_arrived = [&]() {
    bool ok = true;
    for (int w = lane; w < a.W; w += 64) ok &= (int32_t)(ld_u32(arrive + w * SYNC_LINE_WORDS) - gen) >= 0;
    return ok;
  };
  if (a.barrier_mode == 0) return cw_spin(a, lane, all_arrived);
  // gather/release: worker 0 waits for every arrival, then writes each worker's release line
  if (bid == 0) {
    if (cw_spin(a, lane, all_arrived)) return true;
    for (int w = lane; w < a.W; w += 64) st_u32(release + w * SYNC_LINE_WORDS, gen);
  }
  return cw_spin(a, lane, [&]() { return (int32_t)(ld_u32(release + bid * SYNC_LINE_WORDS) - gen) >= 0; });
}

// ---------------------------------------------------------------------------
// control wave main loop
// ---------------------------------------------------------------------------

template <int HD, int G>
__device__ void control_loop(const KernelArgs& a, const Lds& L, int bid, int lane, int block_rows) {
  int* smi = reinterpret_cast<int*>(L.small);
  uint32_t gen = 0;
  int tok = a.token0;
  bool aborted = false;
  const int H = a.H;
  for (int step = 0; step < a.n_steps && !aborted; ++step) {
    const int pos = a.pos0 + step;
    const int64_t L_att = (int64_t)pos + 1;
    const uint16_t* erow = reinterpret_cast<const uint16_t*>(a.packed + a.embed_off + (int64_t)tok * a.embed_stride);
    if (a.poison) {
      const float nan = __uint_as_float(0x7fc00000u);
      const int64_t gid = (int64_t)bid * 64 + lane, gsz = (int64_t)a.W * 64;
      for (int64_t i = gid; i < a.qkv_rows; i += gsz) st_f32(a.qkv + i, nan);
      for (int64_t i = gid; i < (int64_t)a.n_heads * a.S * (HD + 2); i += gsz) st_f32(a.part + i, nan);
      for (int64_t i = gid; i < (int64_t)a.n_heads * HD; i += gsz) st_f32(a.attn + i, nan);
      for (int64_t i = gid; i < a.F; i += gsz) st_f32(a.act + i, nan);
      aborted = cw_grid_barrier(a, bid, lane, ++gen);
      if (aborted) break;
    }
    float lm_best = -INFINITY;
    int lm_idx = 0x7fffffff;
    for (int wv = 0; wv < a.n_waves; ++wv) {
      const TileDesc t = a.tiles[(int64_t)wv * a.W + bid];
      const int layer = a.waves[wv].layer;
      uint64_t t0 = 0;
      if (a.trace) t0 = wall_clock64();
      // ---- prologue (global loads by the control wave) ----
      float rs = 1.0f;  // RMSNorm scale folded out of the input vector, applied to the GEMV results
      switch (t.kind) {
        case KIND_QKV:
          rs = cw_norm(L, lane, layer == 0 ? nullptr : a.x, layer == 0 ? erow : nullptr,
                       reinterpret_cast<const uint16_t*>(a.packed + a.small[layer].attn_norm), H, t.kpad, a.eps);
          break;
        case KIND_GU:
          rs = cw_norm(L, lane, a.x, nullptr, reinterpret_cast<const uint16_t*>(a.packed + a.small[layer].mlp_norm), H,
                       t.kpad, a.eps);
          break;
        case KIND_LM:
          rs = cw_norm(L, lane, a.x, nullptr, reinterpret_cast<const uint16_t*>(a.packed + a.final_norm_off), H, t.kpad,
                       a.eps);
          break;
        case KIND_O: {
          const int nq = a.n_heads * HD;
          if (a.combine_in_o) {
            // stage all split partials; all wavefronts merge them after barrier P
            const int np = a.n_heads * a.S * (HD + 2);  // even
            cw_load_vec(L.part, a.part, np & ~3, np & ~3, lane);
            for (int i = (np & ~3) + lane; i < np; i += 64) L.part[i] = ld_f32(a.part + i);
            for (int i = nq + lane; i < t.kpad; i += 64) L.vec[i] = 0.f;
          } else {
            cw_load_vec(L.vec, a.attn, nq, t.kpad, lane);
          }
          break;
        }
        case KIND_DOWN:
          cw_load_vec(L.vec, a.act, a.F, t.kpad, lane);
          break;
        case KIND_ATTN:
          cw_attn_load<HD, G>(a, L, lane, t.row0);
          break;
        default:
          break;
      }
      uint64_t t_pro = 0, t_cmp = 0;
      if (a.trace) t_pro = wall_clock64();
      if (lane == 0) {
        smi[SM_KIND] = t.kind;
        smi[SM_ROW0] = t.row0;
        smi[SM_NROWS] = t.nrows;
        smi[SM_LAYER] = layer;
        smi[SM_C] = t.kpad / CHUNK_COLS;
        smi[SM_POS] = pos;
      }
      __syncthreads();  // P: global inputs staged in LDS
      prologue_lds_phase<HD, G>(a, L, t.kind, 0, lane, layer, pos);
      __syncthreads();  // A: inputs ready
      if (t.kind == KIND_ATTN) cw_attn_kv_write<HD, G>(a, L, lane, layer, t.row0, t.nrows, L_att);
      // ---- compute waves run; epilogues ----
      if (is_gemv(t.kind)) {
        const int rows = t.kind == KIND_GU ? 2 * t.nrows : t.nrows;
        const int C = t.kpad / CHUNK_COLS;
        for (int r0 = 0; r0 < rows; r0 += block_rows) {
          const int nr = min(block_rows, rows - r0);
          __syncthreads();  // B: partials of this block ready
          if (a.trace && r0 == 0) t_cmp = wall_clock64();
          switch (t.kind) {
            case KIND_QKV:
              for (int r = lane; r < nr; r += 64) st_f32(a.qkv + t.row0 + r0 + r, rs * row_total(L, nr, C, r));
              break;
            case KIND_O:
              for (int r = lane; r < nr; r += 64) {
                const int j = t.row0 + r0 + r;
                const float old = layer == 0 ? bf16_to_f32(erow[j]) : ld_f32(a.x + j);
                st_f32(a.x + j, old + row_total(L, nr, C, r));
              }
              break;
            case KIND_GU:  // interleaved gate/up rows
              for (int p = lane; p < nr / 2; p += 64) {
                const float gt = rs * row_total(L, nr, C, 2 * p);
                const float up = rs * row_total(L, nr, C, 2 * p + 1);
                st_f32(a.act + t.row0 + r0 / 2 + p, gt / (1.0f + __expf(-gt)) * up);
              }
              break;
            case KIND_DOWN:
              for (int r = lane; r < nr; r += 64) {
                const int j = t.row0 + r0 + r;
                const float nx = ld_f32(a.x + j) + row_total(L, nr, C, r);
                st_f32(a.x + j, nx);
                if (a.dbg_hidden) a.dbg_hidden[((int64_t)step * a.n_layers + layer) * H + j] = nx;
              }
              break;
            case KIND_LM:
              for (int r = lane; r < nr; r += 64) {
                const float v = rs * row_total(L, nr, C, r);
                const int idx = t.row0 + r0 + r;
                if (a.out_logits) __builtin_nontemporal_store(v, a.out_logits + (int64_t)step * a.V + idx);
                if (v > lm_best) {  // each lane visits its rows in increasing order: first maximum kept
                  lm_best = v;
                  lm_idx = idx;
                }
              }
              break;
          }
          if (r0 + block_rows < rows) __syncthreads();  // C: partials consumed
        }
      } else {
        __syncthreads();  // B
        if (a.trace) t_cmp = wall_clock64();
        if (t.kind == KIND_ATTN) {
          attn_merge_phase<HD, G>(L, 0, lane);
          __syncthreads();  // E: merged partial ready
          cw_attn_store<HD, G>(a, L, lane, t.row0, t.nrows);
        } else if (t.kind == KIND_COMBINE) {
          float* P = L.part;
          const int np = a.S * (HD + 2);
          for (int i = lane; i < np; i += 64) P[i] = ld_f32(a.part + (int64_t)t.row0 * np + i);
          for (int d = lane; d < HD; d += 64) st_f32(a.attn + (int64_t)t.row0 * HD + d, merge_splits(P, a.S, HD, d));
        }
      }
      if (a.waves[wv].kind == KIND_LM) {
        // worker partial (max, lowest index); also written by workers without vocabulary rows
        for (int off = 32; off >= 1; off >>= 1) {
          const float ov = __shfl_xor(lm_best, off);
          const int oi = __shfl_xor(lm_idx, off);
          if (ov > lm_best || (ov == lm_best && oi < lm_idx)) {
            lm_best = ov;
            lm_idx = oi;
          }
        }
        if (lane == 0)
          st_u64(reinterpret_cast<uint64_t*>(a.lmpart) + bid,
                 (uint64_t)__float_as_uint(lm_best) | ((uint64_t)(uint32_t)lm_idx << 32));
      }
      uint64_t t1 = 0;
      if (a.trace) t1 = wall_clock64();
      aborted = cw_grid_barrier(a, bid, lane, ++gen);
      if (a.trace && lane == 0) {
        uint64_t* tr = a.trace + (((int64_t)step * a.n_waves + wv) * a.W + bid) * TRACE_WORDS;
        tr[0] = t0;
        tr[1] = t_pro;
        tr[2] = t_cmp;
        tr[3] = t1;
        tr[4] = wall_clock64();
      }
      if (aborted) break;
    }
    if (aborted) break;
    // next token: argmax over all workers' partials, in worker order
    float best = -INFINITY;
    int bidx = 0x7fffffff;
    {
      const __amdgpu_buffer_rsrc_t r = rsrc(a.lmpart);
      COMPILER_FENCE();
      for (int base = 0; base < a.W; base += 4 * 128) {  // 2 partials per 16-byte load, 4 loads in flight
        u32x4 pv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int w = base + u * 128 + lane * 2;
          pv[u] = w < a.W ? cld4(r, (uint32_t)w * 8) : u32x4{0xff800000u, 0x7fffffffu, 0xff800000u, 0x7fffffffu};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int w = base + u * 128 + lane * 2;
          for (int e = 0; e < 2; ++e) {
            const float v = __uint_as_float(e ? pv[u].z : pv[u].x);
            const int ix = (int)(e ? pv[u].w : pv[u].y);
            if (w + e < a.W && (v > best || (v == best && ix < bidx))) {
              best = v;
              bidx = ix;
            }
          }
        }
      }
      COMPILER_FENCE();
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
    if (bid == 0 && lane == 0) a.out_tokens[step] = bidx;
  }
  // release the compute waves: one more barrier (their P) with the done flag set
  if (lane == 0) smi[SM_DONE] = 1;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// compute wave main loop
// ---------------------------------------------------------------------------

template <int HD, int G>
__device__ void compute_loop(const KernelArgs& a, const Lds& L, int c, int lane, int block_rows) {
  const volatile int* smi = reinterpret_cast<const volatile int*>(L.small);
  Prefetch<(G >= 3 ? 8 : PREFETCH_CHUNKS)> pf;
  issue_prefetch(pf, next_gemv(L.segs, a.n_waves, -1, block_rows, c), a.packed, lane);
  int k = -1;  // schedule wave being executed
  for (;;) {   // one iteration per wave of every step, until the control wave raises the done flag
    __syncthreads();  // P
    if (smi[SM_DONE]) break;
    k = k + 1 == a.n_waves ? 0 : k + 1;
    prologue_lds_phase<HD, G>(a, L, smi[SM_KIND], c + 1, lane, smi[SM_LAYER], smi[SM_POS]);
    __syncthreads();  // A
    const int kind = smi[SM_KIND];
    const int row0 = smi[SM_ROW0];
    const int nrows = smi[SM_NROWS];
    const int layer = smi[SM_LAYER];
    const int pos = smi[SM_POS];
    if (is_gemv(kind)) {
      const SegDesc sd = L.segs[k];
      const int rows = sd.rows;
      for (int r0 = 0; r0 < rows; r0 += block_rows) {
        const Range r = block_range(sd, k, r0, block_rows, c);
        const bool last_block = r0 + block_rows >= rows;
        const Range nxt = last_block ? next_gemv(L.segs, a.n_waves, k, block_rows, c) : r;
        if (r.i < r.ihi) {
          stream_range(L, a.packed, r, c, lane, pf, r0 == 0 && pf.k == k, last_block, nxt);
        } else if (last_block) {
          issue_prefetch(pf, nxt, a.packed, lane);
        }
        __syncthreads();                              // B
        if (r0 + block_rows < rows) __syncthreads();  // C
      }
    } else {
      if (kind == KIND_ATTN) {
        compute_attention<HD, G>(a, L, c, lane, layer, row0, nrows, (int64_t)pos + 1);
        __syncthreads();  // B
        attn_merge_phase<HD, G>(L, c + 1, lane);
        __syncthreads();  // E
      } else {
        __syncthreads();  // B
      }
    }
  }
}

template <int HD, int G>
__global__ void __launch_bounds__(BLOCK_THREADS, 1) tiles_worker(KernelArgs args) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  const KernelArgs& a = args;
  Lds L;
  L.vec = reinterpret_cast<float*>(lds_raw);
  L.part = L.vec + a.lds_vec_floats;
  L.small = L.part + a.lds_part_floats;
  L.segs = reinterpret_cast<SegDesc*>(L.small + SMALL_FLOATS);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, bid = blockIdx.x;
  for (int k = tid; k < a.n_waves; k += BLOCK_THREADS) {
    const TileDesc t = a.tiles[(int64_t)k * a.W + bid];
    SegDesc s;
    s.woff = t.woff;
    s.chunks_per_row = t.kpad / CHUNK_COLS;
    s.rows = is_gemv(t.kind) ? (t.kind == KIND_GU ? 2 * t.nrows : t.nrows) : 0;
    L.segs[k] = s;
  }
  if (tid == 0) reinterpret_cast<int*>(L.small)[SM_DONE] = 0;
  __syncthreads();
  const int block_rows = (a.lds_part_floats / NCOMP) & ~1;
  if (wave == 0) control_loop<HD, G>(a, L, bid, lane, block_rows);
  else compute_loop<HD, G>(a, L, wave - 1, lane, block_rows);
}

// ---------------------------------------------------------------------------
// weight packing (plan creation): one launch copies every segment.  Rows whose byte counts
// and addresses are 16-byte multiples move with 16-byte accesses, others with 2-byte ones.
// ---------------------------------------------------------------------------

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

hipError_t launch_pack(const PackSeg* segs, int nseg, uint8_t* dst, hipStream_t stream) {
  const int grid = nseg < 4096 ? (nseg > 0 ? nseg : 1) : 4096;
  hipLaunchKernelGGL(pack_weights, dim3(grid), dim3(256), 0, stream, segs, nseg, dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// host-visible handles of the instantiations
// ---------------------------------------------------------------------------

const void* worker_kernel(int head_dim, int group) {
  if (head_dim == 64) {
    switch (group) {
      case 1: return reinterpret_cast<const void*>(&tiles_worker<64, 1>);
      case 2: return reinterpret_cast<const void*>(&tiles_worker<64, 2>);
      case 3: return reinterpret_cast<const void*>(&tiles_worker<64, 3>);
      case 4: return reinterpret_cast<const void*>(&tiles_worker<64, 4>);
    }
  } else if (head_dim == 128) {
    switch (group) {
      case 1: return reinterpret_cast<const void*>(&tiles_worker<128, 1>);
      case 2: return reinterpret_cast<const void*>(&tiles_worker<128, 2>);
      case 3: return reinterpret_cast<const void*>(&tiles_worker<128, 3>);
      case 4: return reinterpret_cast<const void*>(&tiles_worker<128, 4>);
    }
  }
  return nullptr;
}

}  // namespace tiles
