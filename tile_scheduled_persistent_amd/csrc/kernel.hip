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
// LDS layout (dynamic): ring [NCOMP][RING_SLOTS][1 KB] | vec | part | small | segs.
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
  unsigned char* ring;
  uint32_t ring_addr;  // LDS byte address of the ring
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
// weight prefetcher of one compute wave: walks the worker's GEMV chunks in the
// order the wave consumes them, across blocks, waves and steps.
// ---------------------------------------------------------------------------

struct Cursor {
  int k, r0, i, ihi;
  int64_t base;  // byte offset of the current block's first chunk
};

__device__ inline bool cursor_set(Cursor& cu, const SegDesc& s, int block_rows, int c) {
  const int nr = min(block_rows, s.rows - cu.r0);
  const int n = nr * s.chunks_per_row;
  cu.i = chunk_lo(n, c);
  cu.ihi = chunk_lo(n, c + 1);
  cu.base = s.woff + (int64_t)cu.r0 * s.chunks_per_row * CHUNK_BYTES;
  return cu.i < cu.ihi;
}

// Move to the next non-empty (wave, block) range; wraps to the next step.  A compute wave
// with no chunk in the whole step parks on a valid address (loads that are never consumed).
__device__ inline void cursor_next(Cursor& cu, const SegDesc* segs, int n_waves, int block_rows, int c) {
  if (cu.k == -2) {  // parked: keep re-reading the first chunk of the packed buffer
    cu.i = 0;
    cu.ihi = 1;
    return;
  }
  for (int guard = 0; guard < 4 * n_waves + 4; ++guard) {
    if (cu.k >= 0 && cu.r0 + block_rows < segs[cu.k].rows) {
      cu.r0 += block_rows;
    } else {
      cu.k = cu.k + 1 >= n_waves ? 0 : cu.k + 1;
      cu.r0 = 0;
      if (segs[cu.k].rows == 0) continue;
    }
    if (cursor_set(cu, segs[cu.k], block_rows, c)) return;
  }
  cu.k = -2;
  cu.r0 = 0;
  cu.base = 0;
  cu.i = 0;
  cu.ihi = 1;
}

// Direct-to-LDS 16-byte load of one chunk: lane l's 16 bytes land at lds_addr + 16 l.
// Issued through inline assembly so that the compiler neither reorders LDS reads of the
// ring around it nor adds waits for it: the ring protocol below does the waiting.
__device__ inline void dma_chunk(const void* gaddr, uint32_t lds_addr) {
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);  // wave-uniform by construction
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off\n\t" ::"v"(gaddr),
      "s"(lds_addr)
      : "memory", "m0");
}
// The chunk consumed next was issued RING_SLOTS-1 loads ago (one load is issued per
// consumed chunk, into the slot consumed one iteration earlier), so at most RING_SLOTS-2
// younger loads are in flight; vector-memory loads complete in issue order.  Any other
// load issued in between only makes this wait stricter.
__device__ inline void ring_wait() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(RING_SLOTS - 2) : "memory"); }
__device__ inline void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

struct Prefetcher {
  Cursor cu;
  int slot;       // ring slot of the next chunk to consume
  int free_slot;  // slot consumed in the previous iteration (refilled now)
  uint32_t ring_addr;
  const uint8_t* packed;
  int lane;

  __device__ inline void issue(const SegDesc* segs, int n_waves, int block_rows, int c, int into) {
    const u32x4* g = reinterpret_cast<const u32x4*>(packed + cu.base) + (int64_t)cu.i * 64 + lane;
    dma_chunk(g, ring_addr + (uint32_t)into * CHUNK_BYTES);
    if (++cu.i >= cu.ihi) cursor_next(cu, segs, n_waves, block_rows, c);
  }
};

// ---------------------------------------------------------------------------
// compute wave: GEMV block -> part[row * NCOMP + c]
// ---------------------------------------------------------------------------

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

__device__ void compute_gemv_block(Prefetcher& pf, const Lds& L, int n_waves, int block_rows, int c, int lane, int C,
                                   int nr) {
  const int n = nr * C;
  int i = chunk_lo(n, c);
  const int ihi = chunk_lo(n, c + 1);
  if (i >= ihi) return;
  int row = i / C, seg = i - row * C;
  float acc = 0.f;
  const unsigned char* ring_c = L.ring + (size_t)c * RING_SLOTS * CHUNK_BYTES + lane * 16;
  const float* vlane = L.vec + lane * 8;
  for (; i < ihi; ++i) {
    ring_wait();
    const u32x4 w = *reinterpret_cast<const u32x4*>(ring_c + pf.slot * CHUNK_BYTES);
    pf.issue(L.segs, n_waves, block_rows, c, pf.free_slot);
    pf.free_slot = pf.slot;
    pf.slot = pf.slot + 1 == RING_SLOTS ? 0 : pf.slot + 1;
    acc += dot8(w, vlane + seg * CHUNK_COLS);
    if (++seg == C) {
      const float s = wave_sum(acc);
      if (lane == 0) L.part[row * NCOMP + c] = s;
      acc = 0.f;
      seg = 0;
      ++row;
    }
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

// attention prologue: q (scaled to the base-2 domain), rounded k and v of the current
// position into LDS; the split holding the current position writes K/V to the cache.
template <int HD, int G>
__device__ void cw_attn_prologue(const KernelArgs& a, const Lds& L, int lane, int layer, int g, int sp, int pos,
                                 int64_t L_att) {
  float* q = L.part;
  float* kc = q + G * HD;
  float* vc = kc + HD;
  const int qbase = g * G * HD;
  const int kbase = a.n_heads * HD + g * HD;
  const int vbase = a.n_heads * HD + a.n_kv * HD + g * HD;
  constexpr int HALF = HD / 2;
  // raw q (G heads), k, v of this KV group: (G + 2) * HD floats, staged through LDS
  float* raw = L.vec;
  cw_load_vec(raw, a.qkv + qbase, G * HD, G * HD, lane);
  cw_load_vec(raw + G * HD, a.qkv + kbase, HD, HD, lane);
  cw_load_vec(raw + (G + 1) * HD, a.qkv + vbase, HD, HD, lane);
  const bool qkn = a.small[layer].q_norm >= 0;
  // G query heads and the key: optional RMSNorm over HD, then RoPE on pairs (i, i + HD/2)
  float co = 0.f, si = 0.f;
  if (lane < HALF) {
    const float* cs = a.rope + ((int64_t)pos * HALF + lane) * 2;
    co = cs[0];
    si = cs[1];
  }
  for (int u = 0; u <= G; ++u) {
    float u0 = 0.f, u1 = 0.f;
    if (lane < HALF) {
      u0 = raw[u * HD + lane];
      u1 = raw[u * HD + lane + HALF];
    }
    if (qkn) {
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
  }
  for (int i = lane; i < HD; i += 64) vc[i] = bf16_round(raw[(G + 1) * HD + i]);
  // KV write by the split that holds the current position
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
  float* ws = L.part + G * HD + 2 * HD;
  const int64_t ch = (L_att + a.S - 1) / a.S;
  int64_t lo = (int64_t)sp * ch;
  const int64_t hi = lo + ch < L_att ? lo + ch : L_att;
  if (lo > L_att) lo = L_att;
  const int64_t cur = L_att - 1;
  const int64_t kvrow0 = ((int64_t)layer * a.n_kv + g) * a.kv_cap;
  constexpr int LPP = HD / 8;  // lanes per position
  constexpr int P = 64 / LPP;  // positions per load
  constexpr int U = 4;         // loads in flight per operand
  const int64_t n = hi > lo ? hi - lo : 0;
  const int64_t wlo = lo + (n * c) / NCOMP, whi = lo + (n * (c + 1)) / NCOMP;
  const int pp = lane / LPP, dseg = lane % LPP;
  float qr[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[h][e] = q[h * HD + dseg * 8 + e];
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
  for (int64_t jb = wlo; jb < whi; jb += U * P) {
    // issue the loads of U position groups, then consume them
    u32x4 kw[U], vw[U];
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
        float d0 = qr[h][0] * kf[0], d1 = qr[h][1] * kf[1];
        d0 = fmaf(qr[h][2], kf[2], d0);
        d1 = fmaf(qr[h][3], kf[3], d1);
        d0 = fmaf(qr[h][4], kf[4], d0);
        d1 = fmaf(qr[h][5], kf[5], d1);
        d0 = fmaf(qr[h][6], kf[6], d0);
        d1 = fmaf(qr[h][7], kf[7], d1);
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

// control wave: merge the compute waves' states in order and store the split's partial
template <int HD, int G>
__device__ void cw_attn_merge(const KernelArgs& a, const Lds& L, int lane, int g, int sp) {
  const float* ws = L.part + G * HD + 2 * HD;
  for (int idx = lane; idx < G * HD; idx += 64) {
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
    float* dst = a.part + ((int64_t)(g * G + h) * a.S + sp) * (HD + 2);
    if (d == 0) {
      st_f32(dst, mm);
      st_f32(dst + 1, ll);
    }
    st_f32(dst + 2 + d, aa);
  }
}

// LDS-only prologue work shared by all eight wavefronts between barriers P and A:
// merging the split partials into the o_proj input vector.  wave_index in [0, NWAVES).
template <int HD>
__device__ inline void prologue_lds_phase(const KernelArgs& a, const Lds& L, int kind, int wave_index, int lane) {
  if (kind == KIND_O && a.combine_in_o) {
    const int nq = a.n_heads * HD;
    for (int i = wave_index * 64 + lane; i < nq; i += BLOCK_THREADS)
      L.vec[i] = merge_splits(L.part + (i / HD) * a.S * (HD + 2), a.S, HD, i % HD);
  }
}

// ---------------------------------------------------------------------------
// grid barrier (control wave): every worker publishes its generation on its own
// 64-byte line and polls all lines.  A watchdog bounds every wait.
// ---------------------------------------------------------------------------

__device__ bool cw_grid_barrier(const KernelArgs& a, int bid, int lane, uint32_t gen) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are complete
  uint32_t* arrive = a.sync + SYNC_ARRIVE_BASE;
  if (lane == 0) st_u32(arrive + bid * SYNC_LINE_WORDS, gen);
  uint32_t spins = 0;
  for (;;) {
    bool ok = true;
    for (int w = lane; w < a.W; w += 64) ok &= (int32_t)(ld_u32(arrive + w * SYNC_LINE_WORDS) - gen) >= 0;
    if (__all(ok)) return false;
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
          cw_attn_prologue<HD, G>(a, L, lane, layer, t.row0, t.nrows, pos, L_att);
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
      prologue_lds_phase<HD>(a, L, t.kind, 0, lane);
      __syncthreads();  // A: inputs ready
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
          cw_attn_merge<HD, G>(a, L, lane, t.row0, t.nrows);
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
  Prefetcher pf;
  pf.ring_addr = __builtin_amdgcn_readfirstlane(L.ring_addr + (uint32_t)(c * RING_SLOTS * CHUNK_BYTES));
  pf.packed = a.packed;
  pf.lane = lane;
  pf.cu.k = -1;
  pf.cu.r0 = 0;
  cursor_next(pf.cu, L.segs, a.n_waves, block_rows, c);
  for (int s = 0; s < RING_SLOTS - 1; ++s) pf.issue(L.segs, a.n_waves, block_rows, c, s);
  pf.slot = 0;
  pf.free_slot = RING_SLOTS - 1;
  for (;;) {  // one iteration per wave of every step, until the control wave raises the done flag
    __syncthreads();  // P
    if (smi[SM_DONE]) break;
    prologue_lds_phase<HD>(a, L, smi[SM_KIND], c + 1, lane);
    __syncthreads();  // A
    const int kind = smi[SM_KIND];
    const int row0 = smi[SM_ROW0];
    const int nrows = smi[SM_NROWS];
    const int layer = smi[SM_LAYER];
    const int C = smi[SM_C];
    const int pos = smi[SM_POS];
    if (is_gemv(kind)) {
      const int rows = kind == KIND_GU ? 2 * nrows : nrows;
      for (int r0 = 0; r0 < rows; r0 += block_rows) {
        const int nr = min(block_rows, rows - r0);
        compute_gemv_block(pf, L, a.n_waves, block_rows, c, lane, C, nr);
        __syncthreads();                              // B
        if (r0 + block_rows < rows) __syncthreads();  // C
      }
    } else {
      if (kind == KIND_ATTN) compute_attention<HD, G>(a, L, c, lane, layer, row0, nrows, (int64_t)pos + 1);
      __syncthreads();  // B
    }
  }
  vm_drain();
}

template <int HD, int G>
__global__ void __launch_bounds__(BLOCK_THREADS, 1) tiles_worker(KernelArgs args) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  const KernelArgs& a = args;
  Lds L;
  L.ring = lds_raw;
  L.ring_addr = (uint32_t)(uintptr_t)(LDS_AS unsigned char*)lds_raw;
  L.vec = reinterpret_cast<float*>(lds_raw + RING_BYTES);
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
