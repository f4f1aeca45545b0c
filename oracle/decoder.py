"""Plain CPU definition of one batch-1 greedy decode step (test infrastructure only).

This is the oracle the GPU tile schedule is checked against.  It computes the
standard pre-norm Llama / Qwen3 decoder step with no blocking, splitting,
fusion or reordering: the tile graph on the GPU is an exact regrouping of the
same arithmetic (row tiles of each matrix-vector product, split-KV softmax),
so the only legitimate differences are FP32 summation order and the
exp/rsqrt/sin implementations.

Sources (the pages give the workload, not the formulas):

* Tiles page ("Tiles: Scheduling LLM Decoding as a Graph of Tiles"), intro and
  "What the code contains": Llama 3.2 1B, BF16, batch 1, greedy selection, a
  CPU reference checked against the Hugging Face model.
* TileInfer.jl roadmap ("History and roadmap"), "M8 so far" table: the fused
  decode ops are q/k norm + RoPE + KV write, residual add + RMSNorm, and
  SwiGLU; "Milestones" M2: the reference model computes in Float32.

Readings of points the pages leave open:

R1  RMSNorm is y = x / sqrt(mean(x^2) + eps) * g (plain gain), the mean taken
    over the whole vector (over head_dim for the per-head q/k norm).
R2  RoPE uses the "rotate-half" pairing (i, i + hd/2) with inverse frequency
    theta^(-2i/hd) and no frequency scaling.  The angle p * theta^(-2i/hd) is
    formed in FP64 and cos/sin are rounded to FP32 (FP64 mode keeps FP64).
R3  GQA: query head h reads KV head h // (n_heads / n_kv_heads).
R4  Attention scale 1/sqrt(hd); causal, including the current position; no
    biases, soft-caps or windows.
R5  K is cached after q/k norm and RoPE; K and V are rounded to BF16
    (round-to-nearest-even) when written, and the current step attends to the
    rounded values read back from the cache.
R6  Activations and the residual stream stay in FP32; only weights and the
    KV cache are BF16.
R7  SwiGLU: a = silu(W_gate h) * (W_up h), silu(z) = z * sigmoid(z).
R8  Greedy selection is argmax over the logits, lowest index on ties.
R9  The per-layer hidden state is the residual stream after the layer's MLP
    residual add.
R10 With tied embeddings the LM head is the embedding matrix.
Q1  Weight-only INT8 ("History and roadmap" (TileInfer.jl), "M8 so far" table: weight-only INT8
    linear layers; "Tried and not kept": group-wise quantization was not tried, so the scales are
    per output row): every linear layer -- Wq, Wk, Wv, Wo, W_gate, W_up, W_down and the LM head --
    is replaced by symmetric per-row INT8 codes and one FP32 scale per row, s = max|W_row| / 127 and
    q = round-half-even(W / s) clamped to [-127, 127], every operation in FP32 on the BF16 values; a
    row of zeros has s = 0 and q = 0.  The layer computes with the dequantized weights q * s.  The
    embedding lookup and the norm gains keep their BF16 values.
S1  Top-k / top-p sampling ("History and roadmap" (TileInfer.jl), "M8 so far" table: top-k/top-p
    sampling on the device, inside the graph, as fast as greedy; the pages give no order of the
    filters, no random number source and no precision).  A sampled step ranks the logits in decreasing order (equal
    logits by increasing token index, as for R8) and keeps the first top_k; weighs them by
    w_i = exp((z_i - z_0) / T) at temperature T (z_0 the largest); keeps the shortest prefix of that
    ranking whose cumulative weight reaches top_p times the kept total (at least one token); and
    draws one token of the prefix by inverse CDF: the first whose cumulative weight exceeds
    u * (prefix total), with one uniform u in [0, 1) per step, given as an input (the last token of
    the prefix if rounding leaves none).  The decision is an integer taken by floating point, so it
    is taken in FP32, the kernel's precision, with the sums accumulated in ranking order.
    Limits: T > 0, 0 < top_p <= 1, 1 <= top_k <= V.
K1  INT8 KV cache with smoothed keys ("History and roadmap" (TileInfer.jl), "M8 so far" table: INT8
    KV cache with smoothed keys, INT8 attention; "Tried and not kept": quantized queries undid the
    accuracy key smoothing gained, so queries stay FP32).  Each cached K row is divided by a
    per-(layer, KV head, channel) smoothing factor sigma_c > 0 and each K and V row is stored as
    symmetric INT8 codes with one FP32 scale per (layer, KV head, position), quantized as in Q1 but
    from FP32 values: s = max|r| / 127, q = round-half-even(r / s) clamped to [-127, 127] (s = 0,
    q = 0 for a row of zeros).  A step attends to the dequantized rows, K = (q * s) * sigma_c and
    V = q * s, each product in FP32; the current position's K and V are quantized from their FP32
    values (after q/k norm and RoPE) and the step attends to what was stored (as R5).
K2  sigma_c is the largest |K| of channel c over the positions cached when a BF16 cache is
    converted (1 for a channel that is zero there); positions decoded later keep those factors.
    Conversion: the BF16 values widened, divided by sigma, quantized per row.
V1  Greedy verify steps ("History and roadmap" (TileInfer.jl), "M8 so far" table: verify steps of
    up to 16 tokens on the split-KV decode kernels; "Milestones" M7: exact verification for greedy
    decoding).  A verify step of m tokens is m decode steps in which every position consumes the
    given token (the last accepted one, then the drafts); a draft is accepted while it equals the
    argmax after the position before it, and the step yields the accepted drafts followed by the
    argmax after the last of them.  The pages give no acceptance rule beyond "exact": this is the
    rule under which the accepted output equals what greedy decoding would have produced.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "bf16_round",
    "bf16_bits_to_float",
    "float_to_bf16_bits",
    "quantize_rows_int8",
    "dequantize_rows_int8",
    "sample_token",
    "quantize_rows_f32_int8",
    "convert_kv_int8",
    "dequantize_kv_rows",
    "LINEAR_WEIGHTS",
    "rmsnorm",
    "rope_cos_sin",
    "apply_rope",
    "attend",
    "silu",
    "OracleModel",
]

# ---------------------------------------------------------------------------
# BF16 (definition: IEEE-754 binary32 truncated to 8 significant bits, rounded
# to nearest, ties to even; exponent range of binary32).
# ---------------------------------------------------------------------------

_BF16_MIN_EXP = -126          # smallest normal exponent (as in binary32)
_BF16_SIG_BITS = 8            # significant bits including the implicit one


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest BF16 value, ties to even, returned as float64.

    Written from the definition of the format (8 significant bits, binary32
    exponent range, gradual underflow, overflow to +-inf) rather than by bit
    manipulation, so it is independent of any library conversion routine.
    Works for float32 and float64 inputs alike.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    finite = np.isfinite(x) & (x != 0.0)
    xf = x[finite]
    _, e = np.frexp(xf)                    # xf = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, _BF16_MIN_EXP + 1)   # gradual underflow below 2**-126
    ulp = np.ldexp(1.0, e - _BF16_SIG_BITS)
    r = np.round(xf / ulp) * ulp           # np.round: half to even; exact scaling
    with np.errstate(over="ignore"):
        r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
    out[finite] = r
    return out


def float_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) of round-to-nearest-even(x)."""
    r = bf16_round(x)
    with np.errstate(over="ignore", invalid="ignore"):
        f = r.astype(np.float32)           # exact: r has <= 8 significant bits
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    bits[np.isnan(r)] = 0x7FC0
    return bits


def bf16_bits_to_float(u: np.ndarray, dtype=np.float32) -> np.ndarray:
    """Exact widening of BF16 bit patterns (uint16) to float32 / float64."""
    u = np.asarray(u, dtype=np.uint16)
    f = (u.astype(np.uint32) << 16).view(np.float32)
    return f.astype(dtype, copy=False)


# ---------------------------------------------------------------------------
# Weight-only INT8 (reading Q1)
# ---------------------------------------------------------------------------

LINEAR_WEIGHTS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def quantize_rows_int8(w_bits: np.ndarray):
    """Q1: symmetric per-row INT8 codes and FP32 scales of a BF16 matrix (uint16 bits [R, C]).

    s_r = max_j |W_rj| / 127 and q_rj = round-half-even(W_rj / s_r), clamped to [-127, 127], each
    operation in FP32 (the division correctly rounded, as IEEE-754 prescribes); s_r = 0 and q = 0 for
    a row of zeros.  Returns (q int8 [R, C], s float32 [R])."""
    w = bf16_bits_to_float(np.atleast_2d(w_bits), np.float32)
    amax = np.max(np.abs(w), axis=-1)                      # exact
    s = (amax / np.float32(127.0)).astype(np.float32)      # FP32 division
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    r = (w / safe[:, None]).astype(np.float32)             # FP32 division
    q = np.clip(np.rint(r), -127, 127)                     # np.rint: half to even
    q = np.where(s[:, None] > 0, q, 0).astype(np.int8)
    return q, s


def dequantize_rows_int8(q: np.ndarray, s: np.ndarray, dtype=np.float32) -> np.ndarray:
    """Q1: the weights a quantized layer computes with, q * s per row (rounded to ``dtype``)."""
    return q.astype(dtype) * s.astype(dtype)[:, None]


def quantize_rows_f32_int8(x: np.ndarray):
    """K1: symmetric INT8 codes and FP32 scales of FP32 rows (last axis), as Q1: s = max|x| / 127,
    q = round-half-even(x / s) clamped to [-127, 127], FP32 divisions; s = 0, q = 0 for a zero row.
    Returns (q int8 [..., n], s float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    r = (x / safe[..., None]).astype(np.float32)
    q = np.clip(np.rint(r), -127, 127)
    q = np.where(s[..., None] > 0, q, 0).astype(np.int8)
    return q, s


def convert_kv_int8(kv_bits: dict, length: int) -> dict:
    """K1/K2: the INT8 cache of a BF16 cache (uint16 bits [layers, kv heads, capacity, hd]) whose
    first ``length`` positions are filled: sigma [layers, kv heads, hd] from those positions, codes
    and scales of those positions (later positions zero).  Returns a dict with ``kq``, ``vq`` (int8,
    the cache's shape), ``ks``, ``vs`` (float32 [layers, kv heads, capacity]) and ``sigma``."""
    k = bf16_bits_to_float(kv_bits["k"][:, :, :length], np.float32)
    v = bf16_bits_to_float(kv_bits["v"][:, :, :length], np.float32)
    sigma = np.max(np.abs(k), axis=2) if length > 0 else np.zeros(k.shape[:2] + k.shape[3:], np.float32)
    sigma = np.where(sigma > 0, sigma, np.float32(1.0)).astype(np.float32)
    shape = kv_bits["k"].shape
    out = {"kq": np.zeros(shape, np.int8), "vq": np.zeros(shape, np.int8),
           "ks": np.zeros(shape[:3], np.float32), "vs": np.zeros(shape[:3], np.float32), "sigma": sigma}
    out["kq"][:, :, :length], out["ks"][:, :, :length] = quantize_rows_f32_int8((k / sigma[:, :, None, :]).astype(np.float32))
    out["vq"][:, :, :length], out["vs"][:, :, :length] = quantize_rows_f32_int8(v)
    return out


def dequantize_kv_rows(q: np.ndarray, s: np.ndarray, sigma: Optional[np.ndarray] = None, dtype=np.float32):
    """K1: the rows a step attends to: (q * s) [* sigma], each product in FP32, then widened."""
    r = (q.astype(np.float32) * s.astype(np.float32)[..., None]).astype(np.float32)
    if sigma is not None:
        r = (r * sigma.astype(np.float32)).astype(np.float32)
    return r.astype(dtype)


# ---------------------------------------------------------------------------
# Layer pieces
# ---------------------------------------------------------------------------


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """R1: y = x / sqrt(mean(x^2) + eps) * g over the last axis."""
    dt = x.dtype
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return (x / np.sqrt(ms + dt.type(eps))) * g


def rope_cos_sin(pos: int, hd: int, theta: float, dtype=np.float32):
    """R2: cos/sin of p * theta^(-2i/hd), i < hd/2, angles in FP64."""
    i = np.arange(hd // 2, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * i / hd)
    phi = float(pos) * inv_freq
    return np.cos(phi).astype(dtype), np.sin(phi).astype(dtype)


def apply_rope(u: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """R2: rotate pairs (i, i + hd/2) of every row of u by the angles."""
    half = u.shape[-1] // 2
    a = u[..., :half]
    b = u[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """R4: softmax(K q / sqrt(hd)) V for one query head over L positions.

    q: [hd], K, V: [L, hd] (already widened).  Max-subtracted softmax.
    """
    dt = q.dtype
    s = (K @ q) * dt.type(1.0 / math.sqrt(q.shape[-1]))
    w = np.exp(s - s.max())
    w = w / w.sum()
    return w @ V


def silu(z: np.ndarray) -> np.ndarray:
    """R7: z * sigmoid(z)."""
    one = z.dtype.type(1.0)
    return z / (one + np.exp(-z))


def sample_token(logits: np.ndarray, temperature: float, top_k: int, top_p: float, u: float,
                 detail: bool = False):
    """S1: one token drawn from ``logits`` by top-k, then temperature softmax, then top-p, with the
    step's uniform ``u`` in [0, 1).  Every sum and comparison is FP32.  With ``detail`` also returns
    the ranking (token ids), the kept count, the FP32 cumulative weights and the drawn position."""
    z = np.asarray(logits, dtype=np.float32)
    if not (temperature > 0 and 0 < top_p <= 1 and 1 <= top_k <= z.shape[0] and 0 <= u < 1):
        raise ValueError("sampling parameters out of range")
    order = np.lexsort((np.arange(z.shape[0]), -z))[:top_k]   # decreasing logit, then increasing id
    zk = z[order]
    w = np.exp((zk - zk[0]) / np.float32(temperature)).astype(np.float32)
    cum = np.cumsum(w, dtype=np.float32)                       # sums in ranking order
    need = np.float32(top_p) * cum[-1]
    n = int(np.argmax(cum >= need)) + 1 if np.any(cum >= need) else top_k
    target = np.float32(u) * cum[n - 1]
    above = np.nonzero(cum[:n] > target)[0]
    i = int(above[0]) if above.size else n - 1
    tok = int(order[i])
    if detail:
        return tok, {"order": order, "n": n, "cum": cum, "pos": i, "target": target, "need": need}
    return tok


# ---------------------------------------------------------------------------
# Whole decode step
# ---------------------------------------------------------------------------


class OracleModel:
    """The decoder with BF16 weights given as uint16 bit arrays.

    ``cfg`` is any object with the attributes n_layers, hidden, n_heads,
    n_kv_heads, head_dim, ffn, vocab, rope_theta, rms_eps, qk_norm and
    tie_embeddings.  ``weights`` is a dict of uint16 arrays:
    ``embed`` [V, H], ``final_norm`` [H], optional ``lm_head`` [V, H] and
    ``layers``: a list of dicts with attn_norm [H], wq [n_q*hd, H],
    wk/wv [n_kv*hd, H], optional q_norm/k_norm [hd], wo [H, n_q*hd],
    mlp_norm [H], w_gate/w_up [F, H], w_down [H, F].

    The KV cache is a dict with uint16 arrays ``k`` and ``v`` of shape
    [n_layers, n_kv_heads, capacity, hd]; :meth:`step` writes position ``pos``.
    """

    def __init__(self, cfg, weights: dict, dtype=np.float32, widen_once: bool = True, weight_format: str = "bf16"):
        self.cfg = cfg
        self.dtype = np.dtype(dtype)
        self.w = weights
        self.widen_once = widen_once
        if weight_format not in ("bf16", "int8"):
            raise ValueError("weight_format must be 'bf16' or 'int8'")
        self.int8 = weight_format == "int8"                # Q1
        self._cache: dict = {}

    # widened weights -------------------------------------------------------
    def _get(self, layer: Optional[int], name: str, linear: bool = False) -> np.ndarray:
        """The weights a stage computes with: the BF16 values widened, or (INT8 model, a linear
        layer) its dequantized INT8 codes (Q1)."""
        key = (layer, name, linear)
        if key in self._cache:
            return self._cache[key]
        src = self.w[name] if layer is None else self.w["layers"][layer][name]
        if self.int8 and (linear or name in LINEAR_WEIGHTS):
            arr = dequantize_rows_int8(*quantize_rows_int8(src), self.dtype)
        else:
            arr = bf16_bits_to_float(src, self.dtype)
        if self.widen_once:
            self._cache[key] = arr
        return arr

    def _embed_row(self, token: int) -> np.ndarray:
        return bf16_bits_to_float(self.w["embed"][token], self.dtype).copy()

    def _lm_head(self) -> np.ndarray:
        # (INT8 model: the head is a linear layer, quantized like the others; the lookup of the
        # input token's embedding row stays BF16)
        if self.cfg.tie_embeddings or self.w.get("lm_head") is None:
            return self._get(None, "embed", linear=True)
        return self._get(None, "lm_head", linear=True)

    # one step ----------------------------------------------------------------
    def step(self, kv: dict, token: int, pos: int, kv_wide: Optional[dict] = None):
        """Run one decode step for ``token`` at position ``pos``.

        Returns (logits [V], hidden [n_layers, H]); writes K/V at ``pos``.
        ``kv_wide`` (optional) holds the cache already widened to this model's dtype
        (``k``/``v`` arrays shaped like the bit arrays, see :meth:`widen_kv`): attention then
        reads the widened rows instead of widening them again, and the row written at
        ``pos`` is written to both.  The values are the same either way.
        """
        c = self.cfg
        dt = self.dtype
        nq, nkv, hd = c.n_heads, c.n_kv_heads, c.head_dim
        group = nq // nkv
        eps = float(c.rms_eps)
        if not (0 <= token < c.vocab):
            raise ValueError("token out of range")
        int8_kv = "kq" in kv                                      # K1: an INT8 cache (convert_kv_int8)
        if pos >= (kv["kq"] if int8_kv else kv["k"]).shape[2]:
            raise ValueError("KV capacity exceeded")
        x = self._embed_row(token)
        hidden = np.empty((c.n_layers, c.hidden), dtype=dt)
        if dt == np.float64:
            cos, sin = rope_cos_sin(pos, hd, c.rope_theta, np.float64)
        else:
            cos, sin = rope_cos_sin(pos, hd, c.rope_theta, np.float32)
        for l in range(c.n_layers):
            h = rmsnorm(x, self._get(l, "attn_norm"), eps)
            q = (self._get(l, "wq") @ h).reshape(nq, hd)
            k = (self._get(l, "wk") @ h).reshape(nkv, hd)
            v = (self._get(l, "wv") @ h).reshape(nkv, hd)
            if c.qk_norm:
                q = rmsnorm(q, self._get(l, "q_norm"), eps)
                k = rmsnorm(k, self._get(l, "k_norm"), eps)
            q = apply_rope(q, cos, sin)
            k = apply_rope(k, cos, sin)
            if int8_kv:                                            # K1: quantized from FP32
                sg = kv["sigma"][l]
                kv["kq"][l, :, pos, :], kv["ks"][l, :, pos] = quantize_rows_f32_int8(
                    (k.astype(np.float32) / sg).astype(np.float32))
                kv["vq"][l, :, pos, :], kv["vs"][l, :, pos] = quantize_rows_f32_int8(v.astype(np.float32))
            else:
                kv["k"][l, :, pos, :] = float_to_bf16_bits(k)        # R5
                kv["v"][l, :, pos, :] = float_to_bf16_bits(v)
            if kv_wide is not None:
                if int8_kv:
                    kv_wide["k"][l, :, pos, :] = dequantize_kv_rows(kv["kq"][l, :, pos], kv["ks"][l, :, pos],
                                                                    kv["sigma"][l], dt)
                    kv_wide["v"][l, :, pos, :] = dequantize_kv_rows(kv["vq"][l, :, pos], kv["vs"][l, :, pos], None, dt)
                else:
                    kv_wide["k"][l, :, pos, :] = bf16_bits_to_float(kv["k"][l, :, pos, :], dt)
                    kv_wide["v"][l, :, pos, :] = bf16_bits_to_float(kv["v"][l, :, pos, :], dt)
            attn = np.empty((nq, hd), dtype=dt)
            for hh in range(nq):
                g = hh // group                                    # R3
                if kv_wide is not None:
                    Kc = kv_wide["k"][l, g, : pos + 1]
                    Vc = kv_wide["v"][l, g, : pos + 1]
                elif int8_kv:
                    Kc = dequantize_kv_rows(kv["kq"][l, g, : pos + 1], kv["ks"][l, g, : pos + 1], kv["sigma"][l, g], dt)
                    Vc = dequantize_kv_rows(kv["vq"][l, g, : pos + 1], kv["vs"][l, g, : pos + 1], None, dt)
                else:
                    Kc = bf16_bits_to_float(kv["k"][l, g, : pos + 1], dt)
                    Vc = bf16_bits_to_float(kv["v"][l, g, : pos + 1], dt)
                attn[hh] = attend(q[hh], Kc, Vc)
            x = x + self._get(l, "wo") @ attn.reshape(-1)
            h = rmsnorm(x, self._get(l, "mlp_norm"), eps)
            a = silu(self._get(l, "w_gate") @ h) * (self._get(l, "w_up") @ h)
            x = x + self._get(l, "w_down") @ a
            hidden[l] = x                                          # R9
        hf = rmsnorm(x, self._get(None, "final_norm"), eps)
        logits = self._lm_head() @ hf
        if not np.all(np.isfinite(logits)):
            raise FloatingPointError("non-finite logit")
        return logits, hidden

    # drivers -----------------------------------------------------------------
    def widen_kv(self, kv: dict) -> dict:
        """The whole cache widened (exactly) to this model's dtype, for :meth:`step`'s
        ``kv_wide``: long caches are then widened once instead of at every step (an INT8 cache:
        its dequantized rows, K1)."""
        if "kq" in kv:
            return {"k": dequantize_kv_rows(kv["kq"], kv["ks"], kv["sigma"][:, :, None, :], self.dtype),
                    "v": dequantize_kv_rows(kv["vq"], kv["vs"], None, self.dtype)}
        return {"k": bf16_bits_to_float(kv["k"], self.dtype).copy(),
                "v": bf16_bits_to_float(kv["v"], self.dtype).copy()}

    def verify(self, kv: dict, tokens: Sequence[int], pos0: int, widen_kv_once: bool = False):
        """V1: a greedy verify step of m = len(tokens) tokens [t_0, d_1, .., d_{m-1}]: the last
        accepted token at ``pos0`` and m - 1 draft tokens at the following positions.  Every
        position consumes its given token (teacher forcing), so a_i, the argmax after position
        pos0 + i, is the greedy token that follows t_0, d_1 .. d_i.  Draft d_{i+1} is accepted while
        a_i == d_{i+1}; the accepted count n is the length of that prefix, and the step yields
        d_1 .. d_n followed by a_n (the correction, or after n = m - 1 the bonus token).  The cache
        receives the rows of all m positions (those after pos0 + n are overwritten by later steps).
        Returns a dict with ``argmax`` [m], ``accepted`` n, ``tokens`` [n + 1] and ``logits`` [m, V].
        """
        tokens = [int(t) for t in tokens]
        m = len(tokens)
        res = self.decode(kv, tokens[0], pos0, m, teacher=tokens[1:], keep_hidden=False,
                          widen_kv_once=widen_kv_once)
        a = res["tokens"]
        n = 0
        while n < m - 1 and int(a[n]) == tokens[n + 1]:
            n += 1
        out = np.array(tokens[1:n + 1] + [int(a[n])], dtype=np.int64)
        return {"argmax": a, "accepted": n, "tokens": out, "logits": res["logits"]}

    def decode(self, kv: dict, token: int, pos0: int, n_steps: int,
               teacher: Optional[Sequence[int]] = None, keep_hidden: bool = True,
               widen_kv_once: bool = False, sampling: Optional[tuple] = None,
               uniforms: Optional[Sequence[float]] = None):
        """Decode ``n_steps`` steps starting with ``token`` at ``pos0``.

        Step i consumes ``token`` (i = 0), else the previous step's selected token
        (free-running) or ``teacher[i - 1]`` (teacher-forced).  The selected token is
        the argmax (R8), or with ``sampling`` = (temperature, top_k, top_p) the S1 draw
        with ``uniforms[i]``.  Returns a dict with ``tokens`` [n], ``logits`` [n, V] and
        ``hidden`` [n, n_layers, H] (or None).  ``widen_kv_once`` widens the cache
        once up front (see :meth:`widen_kv`); the results are the same.
        """
        toks = np.empty(n_steps, dtype=np.int64)
        logits_all = np.empty((n_steps, self.cfg.vocab), dtype=self.dtype)
        hidden_all = (np.empty((n_steps, self.cfg.n_layers, self.cfg.hidden), dtype=self.dtype)
                      if keep_hidden else None)
        t = int(token)
        kv_wide = self.widen_kv(kv) if widen_kv_once else None
        for i in range(n_steps):
            if i > 0:
                t = int(teacher[i - 1]) if teacher is not None else int(toks[i - 1])
            logits, hidden = self.step(kv, t, pos0 + i, kv_wide)
            if sampling is None:
                toks[i] = int(np.argmax(logits))                   # R8: first max
            else:
                toks[i] = sample_token(logits, *sampling, float(uniforms[i]))  # S1
            logits_all[i] = logits
            if keep_hidden:
                hidden_all[i] = hidden
        return {"tokens": toks, "logits": logits_all, "hidden": hidden_all}
