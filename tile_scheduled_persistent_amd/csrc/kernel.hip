// The persistent tile worker for gfx950 (CDNA4).
//
// One workgroup per compute unit executes the static per-step schedule built by the
// host planner: for every decoded token, for every wave, run this worker's tile (if
// any), then wait at a grid barrier.  The kernel makes no scheduling decision of its
// own ("Tiles: Scheduling LLM Decoding as a Graph of Tiles", intro): tiles, workers,
// wave order and split boundaries are all fixed by the plan and the attended length.
//
// Tile bodies:
//   * GEMV tiles stream their packed BF16 rows with 16-byte coalesced loads
//     (one "chunk" = 64 lanes x 16 B = 512 columns of a row), multiply by an FP32
//     input vector staged in LDS and reduce across the wavefront with DPP.
//     Prologues fold RMSNorm (and, at layer 0, the embedding lookup); epilogues fold
//     the residual add, SwiGLU and the greedy partial argmax ("History and roadmap",
//     TileInfer.jl, "M8 so far" table: residual add + RMSNorm, SwiGLU in the GEMV).
//   * Attention tiles apply q/k RMSNorm and RoPE, write the step's K/V (BF16) and run
//     one split of grouped-query attention with an online softmax whose per-wavefront
//     states are merged through LDS; splits are merged in the o_proj prologue or in a
//     wave of their own (roadmap "Milestones", M5: split-KV decode attention;
//     "Tried and not kept": combine kept out of the split kernel).
//   * The LM-head tile writes logits and a (max, lowest index) partial; after the
//     last barrier of a step every worker reduces all partials in worker order, so
//     all workers agree on the next token without another barrier.
//
// Cross-worker data (activations, partials, barrier words, the KV rows written this
// launch) moves with device-coherent accesses: stores and loads carry the sc1 cache
// policy, so they are performed at the device coherence point and need no L2
// write-back or invalidate; a worker waits for its own stores to complete before it
// signals the barrier.  Weights are read with non-temporal loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan_types.h"

namespace tiles {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int SC1 = 16;  // buffer-instruction cache policy: device-coherent

// ---------------------------------------------------------------------------
// coherent memory helpers
// ---------------------------------------------------------------------------

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
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

__device__ inline u32x4 ld_u32x4(const u32x4* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t lo = ld_u64(q), hi = ld_u64(q + 1);
  return u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}

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

// sum over groups of 8 consecutive lanes
__device__ inline float sum8(float v) {
  v += dpp<DPP_XOR1>(v);
  v += dpp<DPP_XOR2>(v);
  v += dpp<DPP_HALF_MIRROR>(v);
  return v;
}
// sum over groups of 16 consecutive lanes
__device__ inline float sum16(float v) {
  v = sum8(v);
  v += dpp<DPP_MIRROR>(v);
  return v;
}
// sum over the whole wavefront (result in every lane)
__device__ inline float wave_sum(float v) {
  v = sum16(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// ---------------------------------------------------------------------------
// kernel state
// ---------------------------------------------------------------------------

struct Ctx {
  const KernelArgs* a;
  float* vec;    // LDS input vector (lds_vec_floats)
  float* part;   // LDS partial area (lds_part_floats)
  float* small;  // LDS scratch (1024 floats)
  int bid, tid, wave, lane;
  int step, pos, L, tok;
  bool aborted;
};

// block-wide sum; all threads receive the result; deterministic order
__device__ inline float block_sum(Ctx& c, float v) {
  v = wave_sum(v);
  __syncthreads();
  if (c.lane == 0) c.small[c.wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) s += c.small[w];
  __syncthreads();
  return s;
}

// vec[i] = src[i] * rsqrt(mean(src^2) + eps) * gain[i] for i < n; vec[n..npad) = 0.
// src is either an FP32 device-coherent vector or a BF16 embedding row.
__device__ void norm_prologue(Ctx& c, const float* src_f32, const uint16_t* src_bf16, const uint16_t* gain, int n,
                              int npad) {
  float ss = 0.f;
  for (int i = c.tid; i < npad; i += BLOCK_THREADS) {
    float v = 0.f;
    if (i < n) v = src_bf16 ? bf16_to_f32(src_bf16[i]) : ld_f32(src_f32 + i);
    c.vec[i] = v;
    ss += v * v;
  }
  const float tot = block_sum(c, ss);
  const float rs = 1.0f / sqrtf(tot / (float)n + c.a->eps);
  for (int i = c.tid; i < n; i += BLOCK_THREADS) c.vec[i] = c.vec[i] * rs * bf16_to_f32(gain[i]);
  __syncthreads();
}

// ---------------------------------------------------------------------------
// GEMV tile: part[r * NWAVES + wave] = partial dot of packed row r with vec
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

// chunk range of wave w over n chunks
__device__ inline int chunk_lo(int n, int w) { return (int)(((int64_t)n * w) / NWAVES); }

constexpr int GEMV_BATCH = 8;

__device__ void gemv_tile(Ctx& c, int64_t woff, int kpad, int rows) {
  const int C = kpad / CHUNK_COLS;
  const int n = rows * C;
  const int c0 = chunk_lo(n, c.wave), c1 = chunk_lo(n, c.wave + 1);
  const u32x4* base = reinterpret_cast<const u32x4*>(c.a->packed + woff) + c.lane;
  const float* vlane = c.vec + c.lane * 8;
  if (c0 < c1) {
    int row = c0 / C, seg = c0 - row * C;
    float acc = 0.f;
    int i = c0;
    u32x4 wa[GEMV_BATCH], wb[GEMV_BATCH];
    int na = min(GEMV_BATCH, c1 - i);
#pragma unroll
    for (int u = 0; u < GEMV_BATCH; ++u)
      if (u < na) wa[u] = __builtin_nontemporal_load(base + (int64_t)(i + u) * 64);
    while (true) {
      const int inext = i + na;
      const int nb = min(GEMV_BATCH, c1 - inext);
#pragma unroll
      for (int u = 0; u < GEMV_BATCH; ++u)
        if (u < nb) wb[u] = __builtin_nontemporal_load(base + (int64_t)(inext + u) * 64);
#pragma unroll
      for (int u = 0; u < GEMV_BATCH; ++u) {
        if (u < na) {
          acc += dot8(wa[u], vlane + seg * CHUNK_COLS);
          if (++seg == C) {
            const float s = wave_sum(acc);
            if (c.lane == 0) c.part[row * NWAVES + c.wave] = s;
            acc = 0.f;
            seg = 0;
            ++row;
          }
        }
      }
      if (nb <= 0) break;
      i = inext;
      na = nb;
#pragma unroll
      for (int u = 0; u < GEMV_BATCH; ++u) wa[u] = wb[u];
    }
    if (seg != 0) {  // range ended inside a row
      const float s = wave_sum(acc);
      if (c.lane == 0) c.part[row * NWAVES + c.wave] = s;
    }
  }
  __syncthreads();
}

// total of row r: sum of the partials of the waves whose chunk ranges touch it, in wave order
__device__ inline float gemv_row_total(const Ctx& c, int rows, int C, int r) {
  const int n = rows * C;
  const int first = r * C, last = r * C + C - 1;
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) {
    const int lo = chunk_lo(n, w), hi = chunk_lo(n, w + 1);
    if (lo < hi && lo <= last && first < hi) s += c.part[r * NWAVES + w];
  }
  return s;
}

// Run a GEMV tile in row blocks that fit the LDS partial area; `epi(r0, nr, C)` consumes
// block [r0, r0 + nr) through gemv_row_total before the next block overwrites the partials.
template <typename Epi>
__device__ inline void gemv_rows(Ctx& c, const TileDesc& t, int rows, Epi&& epi) {
  const int block = (c.a->lds_part_floats / NWAVES) & ~1;
  const int C = t.kpad / CHUNK_COLS;
  for (int r0 = 0; r0 < rows; r0 += block) {
    const int nr = min(block, rows - r0);
    gemv_tile(c, t.woff + (int64_t)r0 * t.kpad * 2, t.kpad, nr);
    epi(r0, nr, C);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// attention: one (KV head, split) tile.  HD = head_dim, G = query heads per KV head.
// ---------------------------------------------------------------------------

template <int HD, int G>
__device__ void attention_tile(Ctx& c, const TileDesc& t, int layer) {
  const KernelArgs& a = *c.a;
  const int g = t.row0, sp = t.nrows;
  // LDS layout inside part: q[G][HD] | k[HD] | v[HD] | wave states [NWAVES][G][HD + 2]
  float* q = c.part;
  float* kc = q + G * HD;
  float* vc = kc + HD;
  float* ws = vc + HD;
  const float* qkv = a.qkv;
  const int qbase = g * G * HD;
  const int kbase = a.n_heads * HD + g * HD;
  const int vbase = a.n_heads * HD + a.n_kv * HD + g * HD;
  for (int i = c.tid; i < G * HD; i += BLOCK_THREADS) q[i] = ld_f32(qkv + qbase + i);
  for (int i = c.tid; i < HD; i += BLOCK_THREADS) {
    kc[i] = ld_f32(qkv + kbase + i);
    vc[i] = ld_f32(qkv + vbase + i);
  }
  __syncthreads();
  // q/k RMSNorm (optional) + RoPE: wave h < G handles query head h, wave G the key.
  if (c.wave <= G) {
    float* u = c.wave < G ? q + c.wave * HD : kc;
    constexpr int HALF = HD / 2;
    float u0 = 0.f, u1 = 0.f;
    if (c.lane < HALF) {
      u0 = u[c.lane];
      u1 = u[c.lane + HALF];
    }
    if (a.small[layer].q_norm >= 0) {
      const float ss = wave_sum(u0 * u0 + u1 * u1);
      const float rs = 1.0f / sqrtf(ss / (float)HD + a.eps);
      const uint16_t* gn =
          reinterpret_cast<const uint16_t*>(a.packed + (c.wave < G ? a.small[layer].q_norm : a.small[layer].k_norm));
      if (c.lane < HALF) {
        u0 = u0 * rs * bf16_to_f32(gn[c.lane]);
        u1 = u1 * rs * bf16_to_f32(gn[c.lane + HALF]);
      }
    }
    if (c.lane < HALF) {
      const float* cs = a.rope + ((int64_t)c.pos * HALF + c.lane) * 2;
      const float co = cs[0], si = cs[1];
      const float r0 = u0 * co - u1 * si;
      const float r1 = u1 * co + u0 * si;
      if (c.wave < G) {
        u[c.lane] = r0 * a.qscale;
        u[c.lane + HALF] = r1 * a.qscale;
      } else {
        u[c.lane] = bf16_round(r0);
        u[c.lane + HALF] = bf16_round(r1);
      }
    }
  } else if (c.wave == G + 1) {
    for (int i = c.lane; i < HD; i += 64) vc[i] = bf16_round(vc[i]);
  }
  __syncthreads();

  int64_t lo, hi;
  {
    const int64_t L = c.L;
    const int64_t ch = (L + a.S - 1) / a.S;
    lo = (int64_t)sp * ch;
    hi = lo + ch < L ? lo + ch : L;
    if (lo > L) lo = L;
  }
  const int64_t cur = c.L - 1;  // current position: taken from LDS, written to the cache by its split
  const int64_t kvrow0 = ((int64_t)layer * a.n_kv + g) * a.kv_cap;
  if (lo <= cur && cur < hi && c.tid < HD / 2) {
    const uint32_t kb = f32_to_bf16_bits(kc[2 * c.tid]) | (f32_to_bf16_bits(kc[2 * c.tid + 1]) << 16);
    const uint32_t vb = f32_to_bf16_bits(vc[2 * c.tid]) | (f32_to_bf16_bits(vc[2 * c.tid + 1]) << 16);
    st_u32(reinterpret_cast<uint32_t*>(a.kv_k + (kvrow0 + cur) * HD) + c.tid, kb);
    st_u32(reinterpret_cast<uint32_t*>(a.kv_v + (kvrow0 + cur) * HD) + c.tid, vb);
  }

  // per-wave sub-range
  constexpr int LPP = HD / 8;     // lanes per position
  constexpr int P = 64 / LPP;     // positions per load
  const int64_t n = hi - lo;
  const int64_t wlo = lo + (n * c.wave) / NWAVES, whi = lo + (n * (c.wave + 1)) / NWAVES;
  const int pp = c.lane / LPP, dseg = c.lane % LPP;
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
  for (int64_t j0 = wlo; j0 < whi; j0 += P) {
    const int64_t j = j0 + pp;
    const bool valid = j < whi;
    float kf[8], vf[8];
    if (valid && j != cur) {
      u32x4 kw, vw;
      if (j < a.pos0) {  // cached before this launch: streaming loads
        kw = __builtin_nontemporal_load(kbase_p + j * LPP + dseg);
        vw = __builtin_nontemporal_load(vbase_p + j * LPP + dseg);
      } else {           // written by another worker during this launch: device-coherent loads
        kw = ld_u32x4(kbase_p + j * LPP + dseg);
        vw = ld_u32x4(vbase_p + j * LPP + dseg);
      }
      kf[0] = bf16_lo(kw.x); kf[1] = bf16_hi(kw.x); kf[2] = bf16_lo(kw.y); kf[3] = bf16_hi(kw.y);
      kf[4] = bf16_lo(kw.z); kf[5] = bf16_hi(kw.z); kf[6] = bf16_lo(kw.w); kf[7] = bf16_hi(kw.w);
      vf[0] = bf16_lo(vw.x); vf[1] = bf16_hi(vw.x); vf[2] = bf16_lo(vw.y); vf[3] = bf16_hi(vw.y);
      vf[4] = bf16_lo(vw.z); vf[5] = bf16_hi(vw.z); vf[6] = bf16_lo(vw.w); vf[7] = bf16_hi(vw.w);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kf[e] = valid ? kc[dseg * 8 + e] : 0.f;
        vf[e] = valid ? vc[dseg * 8 + e] : 0.f;
      }
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
  // this wave's state -> LDS
  if (pp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* st = ws + (c.wave * G + h) * (HD + 2);
      if (dseg == 0) {
        st[0] = m[h];
        st[1] = l[h];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) st[2 + dseg * 8 + e] = acc[h][e];
    }
  }
  __syncthreads();
  // merge the waves in order; thread (h, d) produces the tile's partial
  if (c.tid < G * HD) {
    const int h = c.tid / HD, d = c.tid % HD;
    float mm = -INFINITY, ll = 0.f, aa = 0.f;
    for (int w = 0; w < NWAVES; ++w) {
      const float* st = ws + (w * G + h) * (HD + 2);
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

// ---------------------------------------------------------------------------
// grid barrier: every worker publishes its generation on its own 64-byte line and
// wavefront 0 of every worker polls all lines.  A watchdog bounds every wait.
// ---------------------------------------------------------------------------

__device__ void grid_barrier(Ctx& c, uint32_t gen) {
  const KernelArgs& a = *c.a;
  __builtin_amdgcn_s_waitcnt(0);  // this wavefront's stores are complete
  __syncthreads();
  __shared__ int s_abort;
  if (c.wave == 0) {
    uint32_t* arrive = a.sync + SYNC_ARRIVE_BASE;
    if (c.lane == 0) st_u32(arrive + c.bid * SYNC_LINE_WORDS, gen);
    uint32_t spins = 0;
    bool ab = false;
    for (;;) {
      bool ok = true;
      for (int w = c.lane; w < a.W; w += 64) ok &= (int32_t)(ld_u32(arrive + w * SYNC_LINE_WORDS) - gen) >= 0;
      if (__all(ok)) break;
      if ((++spins & 63) == 0) {
        if (ld_u32(a.sync + SYNC_ABORT_WORD) != 0) {
          ab = true;
          break;
        }
        if (spins > a.spin_limit) {
          if (c.lane == 0) {
            st_u32(a.sync + SYNC_STATUS_WORD, 1u);
            st_u32(a.sync + SYNC_ABORT_WORD, 1u);
          }
          ab = true;
          break;
        }
      }
    }
    if (c.lane == 0) s_abort = ab ? 1 : 0;
  }
  __syncthreads();
  c.aborted = s_abort != 0;
}

// ---------------------------------------------------------------------------
// the persistent kernel
// ---------------------------------------------------------------------------

template <int HD, int G>
__global__ void __launch_bounds__(BLOCK_THREADS, 1) tiles_worker(KernelArgs args) {
  extern __shared__ float lds[];
  Ctx c;
  c.a = &args;
  const KernelArgs& a = args;
  c.vec = lds;
  c.part = lds + a.lds_vec_floats;
  c.small = c.part + a.lds_part_floats;
  c.bid = blockIdx.x;
  c.tid = threadIdx.x;
  c.wave = c.tid >> 6;
  c.lane = c.tid & 63;
  c.aborted = false;
  c.tok = a.token0;
  uint32_t gen = 0;
  const int H = a.H;
  for (int step = 0; step < a.n_steps && !c.aborted; ++step) {
    c.step = step;
    c.pos = a.pos0 + step;
    c.L = c.pos + 1;
    const uint16_t* erow = reinterpret_cast<const uint16_t*>(a.packed + a.embed_off + (int64_t)c.tok * a.embed_stride);
    if (a.poison) {
      const float nan = __uint_as_float(0x7fc00000u);
      const int64_t gid = (int64_t)c.bid * BLOCK_THREADS + c.tid, gsz = (int64_t)a.W * BLOCK_THREADS;
      for (int64_t i = gid; i < a.qkv_rows; i += gsz) st_f32(a.qkv + i, nan);
      for (int64_t i = gid; i < (int64_t)a.n_heads * a.S * (a.head_dim + 2); i += gsz) st_f32(a.part + i, nan);
      for (int64_t i = gid; i < (int64_t)a.n_heads * a.head_dim; i += gsz) st_f32(a.attn + i, nan);
      for (int64_t i = gid; i < a.F; i += gsz) st_f32(a.act + i, nan);
      grid_barrier(c, ++gen);
      if (c.aborted) break;
    }
    for (int wv = 0; wv < a.n_waves; ++wv) {
      const WaveDesc wd = a.waves[wv];
      const TileDesc t = a.tiles[(int64_t)wv * a.W + c.bid];
      uint64_t t0 = 0, t1 = 0;
      if (a.trace && c.tid == 0) t0 = wall_clock64();
      const int layer = wd.layer;
      switch (t.kind) {
        case KIND_QKV: {
          const uint16_t* gain = reinterpret_cast<const uint16_t*>(a.packed + a.small[layer].attn_norm);
          norm_prologue(c, layer == 0 ? nullptr : a.x, layer == 0 ? erow : nullptr, gain, H, t.kpad);
          gemv_rows(c, t, t.nrows, [&](int r0, int nr, int C) {
            for (int r = c.tid; r < nr; r += BLOCK_THREADS) st_f32(a.qkv + t.row0 + r0 + r, gemv_row_total(c, nr, C, r));
          });
          break;
        }
        case KIND_ATTN:
          attention_tile<HD, G>(c, t, layer);
          break;
        case KIND_COMBINE: {
          if (c.tid < HD) {
            // read the S partials of head t.row0 through the coherent path into LDS, then merge
            float* P = c.part;
            for (int i = c.tid; i < a.S * (HD + 2); i += HD) P[i] = ld_f32(a.part + (int64_t)t.row0 * a.S * (HD + 2) + i);
          }
          __syncthreads();
          if (c.tid < HD) st_f32(a.attn + (int64_t)t.row0 * HD + c.tid, merge_splits(c.part, a.S, HD, c.tid));
          break;
        }
        case KIND_O: {
          const int nq = a.n_heads * HD;
          if (a.combine_in_o) {
            const int np = a.n_heads * a.S * (HD + 2);
            for (int i = c.tid; i < np; i += BLOCK_THREADS) c.part[i] = ld_f32(a.part + i);
            __syncthreads();
            for (int i = c.tid; i < nq; i += BLOCK_THREADS)
              c.vec[i] = merge_splits(c.part + (i / HD) * a.S * (HD + 2), a.S, HD, i % HD);
          } else {
            for (int i = c.tid; i < nq; i += BLOCK_THREADS) c.vec[i] = ld_f32(a.attn + i);
          }
          for (int i = nq + c.tid; i < t.kpad; i += BLOCK_THREADS) c.vec[i] = 0.f;
          __syncthreads();
          gemv_rows(c, t, t.nrows, [&](int r0, int nr, int C) {
            for (int r = c.tid; r < nr; r += BLOCK_THREADS) {
              const int j = t.row0 + r0 + r;
              const float old = layer == 0 ? bf16_to_f32(erow[j]) : ld_f32(a.x + j);
              st_f32(a.x + j, old + gemv_row_total(c, nr, C, r));
            }
          });
          break;
        }
        case KIND_GU: {
          const uint16_t* gain = reinterpret_cast<const uint16_t*>(a.packed + a.small[layer].mlp_norm);
          norm_prologue(c, a.x, nullptr, gain, H, t.kpad);
          // rows are interleaved gate/up pairs
          gemv_rows(c, t, 2 * t.nrows, [&](int r0, int nr, int C) {
            for (int p = c.tid; p < nr / 2; p += BLOCK_THREADS) {
              const float gt = gemv_row_total(c, nr, C, 2 * p);
              const float up = gemv_row_total(c, nr, C, 2 * p + 1);
              const float si = gt / (1.0f + __expf(-gt));
              st_f32(a.act + t.row0 + r0 / 2 + p, si * up);
            }
          });
          break;
        }
        case KIND_DOWN: {
          for (int i = c.tid; i < t.kpad; i += BLOCK_THREADS) c.vec[i] = i < a.F ? ld_f32(a.act + i) : 0.f;
          __syncthreads();
          gemv_rows(c, t, t.nrows, [&](int r0, int nr, int C) {
            for (int r = c.tid; r < nr; r += BLOCK_THREADS) {
              const int j = t.row0 + r0 + r;
              const float nx = ld_f32(a.x + j) + gemv_row_total(c, nr, C, r);
              st_f32(a.x + j, nx);
              if (a.dbg_hidden) a.dbg_hidden[((int64_t)c.step * a.n_layers + layer) * H + j] = nx;
            }
          });
          break;
        }
        case KIND_LM: {
          const uint16_t* gain = reinterpret_cast<const uint16_t*>(a.packed + a.final_norm_off);
          norm_prologue(c, a.x, nullptr, gain, H, t.kpad);
          float best = -INFINITY;
          int bidx = 0x7fffffff;
          gemv_rows(c, t, t.nrows, [&](int r0, int nr, int C) {
            for (int r = c.tid; r < nr; r += BLOCK_THREADS) {
              const float v = gemv_row_total(c, nr, C, r);
              const int idx = t.row0 + r0 + r;
              if (a.out_logits) __builtin_nontemporal_store(v, a.out_logits + (int64_t)c.step * a.V + idx);
              if (v > best) {  // each thread visits its rows in increasing order: first maximum kept
                best = v;
                bidx = idx;
              }
            }
          });
          // block argmax (greater value, then lower index)
          for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(best, off);
            const int oi = __shfl_xor(bidx, off);
            if (ov > best || (ov == best && oi < bidx)) {
              best = ov;
              bidx = oi;
            }
          }
          __syncthreads();
          if (c.lane == 0) {
            c.small[2 * c.wave] = best;
            reinterpret_cast<int*>(c.small)[2 * c.wave + 1] = bidx;
          }
          __syncthreads();
          if (c.tid == 0) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            for (int w = 0; w < NWAVES; ++w) {
              const float v = c.small[2 * w];
              const int ix = reinterpret_cast<int*>(c.small)[2 * w + 1];
              if (v > bv || (v == bv && ix < bi)) {
                bv = v;
                bi = ix;
              }
            }
            st_u64(reinterpret_cast<uint64_t*>(a.lmpart) + c.bid,
                   (uint64_t)__float_as_uint(bv) | ((uint64_t)(uint32_t)bi << 32));
          }
          break;
        }
        default:
          if (wd.kind == KIND_LM && c.tid == 0)
            st_u64(reinterpret_cast<uint64_t*>(a.lmpart) + c.bid,
                   (uint64_t)__float_as_uint(-INFINITY) | ((uint64_t)0x7fffffffu << 32));
          break;
      }
      if (a.trace && c.tid == 0) t1 = wall_clock64();
      grid_barrier(c, ++gen);
      if (a.trace && c.tid == 0) {
        uint64_t* tr = a.trace + (((int64_t)c.step * a.n_waves + wv) * a.W + c.bid) * 3;
        tr[0] = t0;
        tr[1] = t1;
        tr[2] = wall_clock64();
      }
      if (c.aborted) break;
    }
    if (c.aborted) break;
    // next token: argmax over all workers' partials, in worker order
    {
      float best = -INFINITY;
      int bidx = 0x7fffffff;
      for (int w = c.tid; w < a.W; w += BLOCK_THREADS) {
        const uint64_t pv = ld_u64(reinterpret_cast<const uint64_t*>(a.lmpart) + w);
        const float v = __uint_as_float((uint32_t)pv);
        const int ix = (int)(uint32_t)(pv >> 32);
        if (v > best || (v == best && ix < bidx)) {
          best = v;
          bidx = ix;
        }
      }
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(best, off);
        const int oi = __shfl_xor(bidx, off);
        if (ov > best || (ov == best && oi < bidx)) {
          best = ov;
          bidx = oi;
        }
      }
      __syncthreads();
      if (c.lane == 0) {
        c.small[2 * c.wave] = best;
        reinterpret_cast<int*>(c.small)[2 * c.wave + 1] = bidx;
      }
      __syncthreads();
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int w = 0; w < NWAVES; ++w) {
        const float v = c.small[2 * w];
        const int ix = reinterpret_cast<int*>(c.small)[2 * w + 1];
        if (v > bv || (v == bv && ix < bi)) {
          bv = v;
          bi = ix;
        }
      }
      __syncthreads();
      if (bi < 0 || bi >= a.V) bi = 0;  // only reachable with non-finite logits
      c.tok = bi;
      if (c.bid == 0 && c.tid == 0) a.out_tokens[step] = bi;
    }
  }
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
