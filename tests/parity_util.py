"""Shared helpers of the GPU parity tests: seeded inputs on both sides, the
oracle, and the comparison bars.

Bars (from the decode contract of this library): per-layer hidden states
within relative L2 1e-2 of the oracle, logits within max-abs 5e-2, greedy
tokens identical wherever the oracle's top-2 logit margin exceeds 0.1, and
bit-identical results across repeated GPU runs.
"""

from __future__ import annotations

import os

import numpy as np
import torch

from oracle import OracleModel, convert_kv_int8, dequantize_kv_rows
from tile_scheduled_persistent_amd import synth, tiles

# plan flags added to every plan the parity tests create (e.g. TILES_TEST_EXTRA_FLAGS=0x8 runs the
# suite with the attention scores on the matrix cores)
EXTRA_FLAGS = int(os.environ.get("TILES_TEST_EXTRA_FLAGS", "0"), 0)
HIDDEN_REL_L2 = 1e-2
LOGIT_MAX_ABS = 5e-2
MARGIN = 0.1
FLIP_FRACTION = 0.05  # cached BF16 entries that may differ (see kv_rows_close)


def top2_margin(logits: np.ndarray) -> float:
    part = np.partition(logits.astype(np.float64), -2)
    return float(part[-1] - part[-2])


class Setup:
    """Seeded weights and KV cache for a model, resident on the GPU, plus host bit
    views for the oracle.  `gen_device` is where the generators run."""

    def __init__(self, m, capacity: int, n_cached: int, key_scale: bool = False, gen_device: str = "cpu",
                 widen_once: bool = True, weights: str = "bf16", kv: str = "bf16"):
        self.m = m
        self.weights = weights  # "int8": weight-only INT8 linear layers on both sides
        self.kv = kv            # "int8": INT8 KV cache with smoothed keys on both sides
        self.capacity = capacity
        self.n_cached = n_cached
        w = synth.make_weights(m, device=gen_device)
        k, v = synth.make_kv(m, capacity, n_cached, key_scale=key_scale, device=gen_device)
        self.w_bits = synth.weights_as_bits(w)
        self.kv_bits = {"k": synth.bits(k), "v": synth.bits(v)}
        if gen_device == "cpu":
            w = {"embed": w["embed"].cuda(), "final_norm": w["final_norm"].cuda(),
                 "layers": [{kk: vv.cuda() for kk, vv in d.items()} for d in w["layers"]],
                 **({"lm_head": w["lm_head"].cuda()} if "lm_head" in w else {})}
            k, v = k.cuda(), v.cuda()
        self.w_dev = w
        self.k0, self.v0 = k, v
        self.widen_once = widen_once
        self._oracle = None

    def fresh_kv(self, plan: "tiles.Plan" = None) -> tiles.KVCache:
        """A fresh device cache (INT8 KV: converted from the BF16 one by the library, with `plan`)."""
        if self.kv == "int8":
            kv = tiles.KVCache.convert_int8(plan, self.k0, self.v0, self.n_cached)
            torch.cuda.synchronize()
            return kv
        return tiles.KVCache(self.k0.clone(), self.v0.clone(), self.n_cached)

    def oracle(self) -> OracleModel:
        if self._oracle is None:
            self._oracle = OracleModel(self.m, self.w_bits, np.float32, widen_once=self.widen_once,
                                       weight_format=self.weights)
        return self._oracle

    def oracle_kv(self):
        if self.kv == "int8":
            return convert_kv_int8(self.kv_bits, self.n_cached)
        return {"k": self.kv_bits["k"].copy(), "v": self.kv_bits["v"].copy()}

    def plan(self, flags=tiles.TILES_DEBUG_HIDDEN, **kw) -> tiles.Plan:
        flags |= EXTRA_FLAGS
        kw.setdefault("kv_format", self.kv)
        return tiles.Plan(self.m, self.w_dev, self.capacity, flags=flags, weight_format=self.weights, **kw)


def run_gpu(plan: tiles.Plan, kv: tiles.KVCache, token: int, n: int, want_hidden=True):
    """One launch of n steps; returns (tokens [n], logits [n, V], hidden [n, L, H] or None)."""
    out_t = torch.zeros(n, dtype=torch.int32, device="cuda")
    out_l = torch.zeros((n, plan.model.vocab), dtype=torch.float32, device="cuda")
    plan.decode(kv, token, n, out_t, out_l)
    assert plan.status() == tiles.TILES_OK, tiles.last_error()
    torch.cuda.synchronize()
    hid = plan.read_debug(hidden=True)[0] if want_hidden else None
    return out_t.cpu().numpy().astype(np.int64), out_l.cpu().numpy(), hid


def check_step(tag: str, g_logits, g_hidden, o_logits, o_hidden, g_tok: int, o_tok: int):
    """Assert the bars for one step.  Returns the oracle margin."""
    if g_hidden is not None:
        num = np.linalg.norm((g_hidden - o_hidden).astype(np.float64), axis=-1)
        den = np.linalg.norm(o_hidden.astype(np.float64), axis=-1)
        rel = num / den
        assert rel.max() <= HIDDEN_REL_L2, f"{tag}: hidden rel L2 {rel.max():.3e} (layer {int(rel.argmax())})"
    err = np.abs(g_logits.astype(np.float64) - o_logits.astype(np.float64)).max()
    assert err <= LOGIT_MAX_ABS, f"{tag}: logits max abs err {err:.3e}"
    margin = top2_margin(o_logits)
    if margin > MARGIN:
        assert g_tok == o_tok, f"{tag}: token {g_tok} != oracle {o_tok} at margin {margin:.3f}"
    return margin


def compare_teacher_forced(tag, g_tokens, g_logits, g_hidden, o_res):
    """Compare every step of a GPU launch with an oracle teacher-forced on the GPU's own inputs
    (step i of both consumed the same token).  Asserts the bars at every step and returns the
    observed errors: max per-layer hidden relative L2, max logit abs error, the number of steps
    whose token was checked (oracle top-2 margin > MARGIN) and the smallest oracle margin."""
    n = len(g_tokens)
    assert o_res["logits"].shape[0] == n
    worst_h, worst_l, checked, min_margin = 0.0, 0.0, 0, float("inf")
    for i in range(n):
        margin = check_step(f"{tag} step {i}", g_logits[i], None if g_hidden is None else g_hidden[i],
                            o_res["logits"][i], o_res["hidden"][i], int(g_tokens[i]), int(o_res["tokens"][i]))
        if g_hidden is not None:
            num = np.linalg.norm((g_hidden[i] - o_res["hidden"][i]).astype(np.float64), axis=-1)
            den = np.linalg.norm(o_res["hidden"][i].astype(np.float64), axis=-1)
            worst_h = max(worst_h, float((num / den).max()))
        worst_l = max(worst_l, float(np.abs(g_logits[i].astype(np.float64) - o_res["logits"][i]).max()))
        checked += margin > MARGIN
        min_margin = min(min_margin, margin)
    return {"steps": n, "hidden_rel_l2_max": worst_h, "logit_abs_max": worst_l, "tokens_checked": checked,
            "min_margin": min_margin}


def kv_rows_close(tag, g_cache, o_bits, pos: int, n: int):
    """The K or V rows a launch wrote (positions pos .. pos + n - 1) against the oracle's: the same
    relative-L2 bar per (layer, head, position) row as the hidden states.  Both sides round the same
    FP32 values to BF16, which differ only by summation order; an entry flips to the neighbouring BF16
    value with a probability of about its relative FP32 difference times 2^8 (about 1 % at the 4e-5
    the residual stream reaches after 28 layers), while a rounding-mode mistake (truncation) would
    flip about half of them: at most FLIP_FRACTION of the entries may differ."""
    gb = synth.bits(g_cache)[:, :, pos:pos + n]
    ob = o_bits[:, :, pos:pos + n]
    gf = (gb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    of = (ob.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rel = np.linalg.norm(gf - of, axis=-1) / np.linalg.norm(of, axis=-1)
    assert rel.max() <= HIDDEN_REL_L2, f"{tag}: cached rows rel L2 {rel.max():.3e}"
    frac = float(np.mean(gb != ob))
    assert frac < FLIP_FRACTION, f"{tag}: {frac:.3%} of cached entries differ"
    return float(rel.max()), frac


def compare_free_running(tag, g_tokens, g_logits, g_hidden, o_res, n_check: int):
    """Compare a free-running GPU launch with a free-running oracle for the first
    n_check steps while both consumed the same input token.  Returns the number
    of steps compared."""
    compared = 0
    for i in range(n_check):
        check_step(f"{tag} step {i}", g_logits[i], None if g_hidden is None else g_hidden[i], o_res["logits"][i],
                   o_res["hidden"][i], int(g_tokens[i]), int(o_res["tokens"][i]))
        compared += 1
        if int(g_tokens[i]) != int(o_res["tokens"][i]):
            break  # inputs of later steps differ; allowed only at a low-margin step (checked above)
    return compared


# Sampled decoding: both sides draw in FP32 from logits that differ by summation order (max-abs
# about 1e-4 on the shapes tested), so a draw is compared exactly unless the oracle's sits near a
# decision boundary: the K-th and (K+1)-th largest logits within SAMPLE_DELTA_Z, or a cumulative
# weight within SAMPLE_DELTA_REL (relative) of the top-p threshold or of the draw's target.  A logit
# error e moves a weight by about e / T relative: at T >= 0.3 and e <= 2e-4 that is 7e-4, under the
# 2e-3 band.  Near a boundary the GPU's token must be one of the oracle's top_k + 1 candidates.
SAMPLE_DELTA_Z = 1e-3
SAMPLE_DELTA_REL = 2e-3


def check_sampled_token(tag: str, g_tok: int, o_logits: np.ndarray, sampling, u: float) -> bool:
    """Assert the GPU's sampled token against the oracle's S1 draw from the oracle's logits with
    the same uniform.  Returns True when the draw was compared exactly."""
    from oracle import sample_token

    T, K, P = sampling
    tok, d = sample_token(o_logits, T, K, P, float(u), detail=True)
    z = np.asarray(o_logits, np.float32)
    rank = np.lexsort((np.arange(len(z)), -z))
    cum = d["cum"].astype(np.float64)
    n, total = d["n"], float(cum[-1])
    near = K < len(z) and float(z[rank[K - 1]]) - float(z[rank[K]]) < SAMPLE_DELTA_Z
    # (the last candidate's sum is the total: whether it reaches the threshold never changes the prefix)
    near = near or bool(np.any(np.abs(cum[:-1] - float(d["need"])) < SAMPLE_DELTA_REL * total))
    near = near or bool(np.any(np.abs(cum[:n] - float(d["target"])) < SAMPLE_DELTA_REL * float(cum[n - 1])))
    if not near:
        assert g_tok == tok, f"{tag}: sampled token {g_tok} != oracle {tok} (u = {u})"
        return True
    assert g_tok in set(int(x) for x in rank[:K + 1]), f"{tag}: sampled token {g_tok} not among the top {K + 1}"
    return False


def run_gpu_sampled(plan: tiles.Plan, kv: tiles.KVCache, token: int, n: int, uniforms: np.ndarray, want_hidden=True):
    """One sampled launch of n steps with the given uniforms: (tokens [n], logits [n, V], hidden)."""
    out_t = torch.zeros(n, dtype=torch.int32, device="cuda")
    out_l = torch.zeros((n, plan.model.vocab), dtype=torch.float32, device="cuda")
    u = torch.from_numpy(np.ascontiguousarray(uniforms[:n], dtype=np.float32)).cuda()
    plan.decode(kv, token, n, out_t, out_l, uniforms=u)
    assert plan.status() == tiles.TILES_OK, tiles.last_error()
    torch.cuda.synchronize()
    hid = plan.read_debug(hidden=True)[0] if want_hidden else None
    return out_t.cpu().numpy().astype(np.int64), out_l.cpu().numpy(), hid


def compare_sampled_teacher_forced(tag, g_tokens, g_logits, g_hidden, o_res, sampling, uniforms):
    """Every step of a sampled GPU launch against an oracle teacher-forced on the GPU's tokens
    (same uniforms): hidden and logit bars as for greedy steps, and check_sampled_token.
    Returns the observed errors and the number of exactly compared draws."""
    n = len(g_tokens)
    assert o_res["logits"].shape[0] == n
    worst_h, worst_l, exact = 0.0, 0.0, 0
    for i in range(n):
        if g_hidden is not None:
            num = np.linalg.norm((g_hidden[i] - o_res["hidden"][i]).astype(np.float64), axis=-1)
            den = np.linalg.norm(o_res["hidden"][i].astype(np.float64), axis=-1)
            h = float((num / den).max())
            assert h <= HIDDEN_REL_L2, f"{tag} step {i}: hidden rel L2 {h:.3e}"  # (fails on NaN too)
            worst_h = max(worst_h, h)
        err = float(np.abs(g_logits[i].astype(np.float64) - o_res["logits"][i]).max())
        assert err <= LOGIT_MAX_ABS, f"{tag} step {i}: logits max abs err {err:.3e}"
        worst_l = max(worst_l, err)
        exact += check_sampled_token(f"{tag} step {i}", int(g_tokens[i]), o_res["logits"][i], sampling, uniforms[i])
    return {"steps": n, "hidden_rel_l2_max": worst_h, "logit_abs_max": worst_l, "draws_exact": exact}


def split_int8_cache(kv: tiles.KVCache):
    """The device INT8 cache as host arrays in the oracle's form: K codes, V codes (de-interleaved:
    per group of 8 dimensions the K codes come first), K and V scales, smoothing factors."""
    codes = kv.k.cpu().numpy()
    L, H, cap, hd2 = codes.shape
    g = codes.reshape(L, H, cap, hd2 // 16, 2, 8)
    kq = np.ascontiguousarray(g[:, :, :, :, 0, :]).reshape(L, H, cap, hd2 // 2)
    vq = np.ascontiguousarray(g[:, :, :, :, 1, :]).reshape(L, H, cap, hd2 // 2)
    return kq, vq, kv.k_scale.cpu().numpy(), kv.v_scale.cpu().numpy(), kv.k_smooth.cpu().numpy()


def kv8_rows_close(tag, kv: tiles.KVCache, okv: dict, pos: int, n: int):
    """The INT8 rows a launch wrote (positions pos .. pos + n - 1) against the oracle's.  Both sides
    quantize FP32 rows x (K: divided by the smoothing factors) that differ by summation order, within
    the hidden-state bar: ||dx||_2 <= HIDDEN_REL_L2 ||x||_2.  A scale is max|x| / 127, and a maximum
    moves by at most ||dx||_inf <= ||dx||_2, so |ds| <= HIDDEN_REL_L2 ||x||_2 / 127 (||x||_2 taken from
    the oracle's codes times its scale).  A code may land one step away, rarely (at most FLIP_FRACTION
    of them).  Returned per K / V: the largest dequantized-row relative L2 difference, the fraction of
    differing codes and the largest relative scale difference (for the report; a flip in an outlier
    channel of a smoothed key is worth about 1/127 of the row on its own, so no fixed row bar fits)."""
    kq, vq, ks, vs, sg = split_int8_cache(kv)
    assert np.array_equal(sg, okv["sigma"]), f"{tag}: smoothing factors changed"
    out = {}
    for name, gq, gs, oq, os_, sig in (("K", kq, ks, okv["kq"], okv["ks"], okv["sigma"]),
                                      ("V", vq, vs, okv["vq"], okv["vs"], None)):
        gq, oq = gq[:, :, pos:pos + n].astype(np.int32), oq[:, :, pos:pos + n].astype(np.int32)
        gs, os_ = gs[:, :, pos:pos + n].astype(np.float64), os_[:, :, pos:pos + n].astype(np.float64)
        assert np.abs(gq - oq).max() <= 1, f"{tag} {name}: a code off by more than one step"
        frac = float(np.mean(gq != oq))
        assert frac < FLIP_FRACTION, f"{tag} {name}: {frac:.3%} of codes differ"
        xnorm = np.linalg.norm(oq * os_[..., None], axis=-1)  # ||x||_2 of the oracle's row (smoothed units)
        assert np.all(np.abs(gs - os_) <= HIDDEN_REL_L2 * xnorm / 127.0 + 1e-30), f"{tag} {name}: scale beyond bound"
        rs = np.abs(gs - os_) / np.maximum(os_, 1e-30)
        s4 = None if sig is None else sig[:, :, None, :]
        gd = dequantize_kv_rows(gq.astype(np.int8), gs, s4, np.float64)
        od = dequantize_kv_rows(oq.astype(np.int8), os_, s4, np.float64)
        rel = np.linalg.norm(gd - od, axis=-1) / np.maximum(np.linalg.norm(od, axis=-1), 1e-30)
        out[name] = (float(rel.max()), frac, float(rs.max()))
    return out
