"""Pins of the CPU oracle against facts that do not come from the oracle itself:
library conversions, closed forms, invariants, hand-worked examples and brute
force on tiny inputs.  Each test names the plausible mistake it would catch.
"""

import math

import numpy as np
import pytest
import torch

from oracle import (OracleModel, apply_rope, attend, bf16_bits_to_float, bf16_round, float_to_bf16_bits, rmsnorm,
                    rope_cos_sin, silu)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------------------
# BF16 rounding: pinned to torch's float32 -> bfloat16 conversion (RNE).
# Catches: truncation instead of rounding, ties-away, wrong overflow/underflow.
# ---------------------------------------------------------------------------

def _torch_bits(x32):
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_round_matches_torch_random_and_ties():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 200_000),
        rng.standard_normal(1000).astype(np.float32),
    ]).astype(np.float32)
    # exact ties: low 16 bits = 0x8000 with both parities of bit 16
    u = rng.integers(0x00800000, 0x7F000000, 20_000, dtype=np.uint32)
    u = (u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    ties = u.view(np.float32)
    x = np.concatenate([x, ties, -ties])
    assert np.array_equal(float_to_bf16_bits(x), _torch_bits(x))


def test_bf16_round_special_values():
    f32 = np.finfo(np.float32)
    x = np.array([0.0, -0.0, np.inf, -np.inf, f32.max, -f32.max, f32.tiny, f32.tiny / 3, 1e-45, -1e-45,
                  3.3895314e38, 3.3961e38, 3.39e38, 1.0, 1.00390625, 1.005859375, 65504.0], dtype=np.float32)
    assert np.array_equal(float_to_bf16_bits(x), _torch_bits(x))
    nan_bits = float_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(bf16_bits_to_float(nan_bits))[0]


def test_bf16_round_float64_input_is_correctly_rounded():
    # fp64 input exactly halfway between two bf16 values in fp64 but not in fp32 must still round correctly:
    # 1 + 2^-8 (a tie -> 1.0), 1 + 2^-8 + 2^-40 (above the tie -> 1 + 2^-7).
    x = np.array([1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, 1 + 3 * 2.0 ** -8], dtype=np.float64)
    assert list(bf16_round(x)) == [1.0, 1 + 2.0 ** -7, 1 + 4 * 2.0 ** -8]


def test_bf16_widening_is_exact_for_every_pattern():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_float(allbits)
    t = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    finite = np.isfinite(t)
    assert np.array_equal(f[finite], t[finite])
    back = float_to_bf16_bits(f[finite])
    assert np.array_equal(back, allbits[finite])


# ---------------------------------------------------------------------------
# RMSNorm.  Catches: mean vs sum, missing sqrt, eps outside the sqrt, (1+g).
# ---------------------------------------------------------------------------

def test_rmsnorm_unit_rms_before_gain():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 2048)).astype(np.float32) * 3
    g = (1 + 0.01 * rng.standard_normal(2048)).astype(np.float32)
    y = rmsnorm(x, g, 0.0)
    rms = np.sqrt(np.mean((y / g).astype(np.float64) ** 2, axis=-1))
    assert np.allclose(rms, 1.0, atol=1e-6)


def test_rmsnorm_constant_vector_closed_form():
    for c in [0.5, 3.0, -2.0, 1e-3]:
        for eps in [1e-5, 1e-6, 0.25]:
            x = np.full(64, c, dtype=np.float64)
            y = rmsnorm(x, np.ones(64), eps)
            assert np.allclose(y, c / math.sqrt(c * c + eps), rtol=1e-14)


# ---------------------------------------------------------------------------
# RoPE.  Catches: interleaved vs rotate-half pairing, wrong frequency exponent,
# sign of the rotation, angle in FP32.
# ---------------------------------------------------------------------------

def test_rope_hand_worked_example():
    # hd = 4, theta = 100: inverse frequencies 100^0 = 1 and 100^(-1/2) = 0.1; pairs (0,2), (1,3).
    cos, sin = rope_cos_sin(1, 4, 100.0, np.float64)
    u = np.array([1.0, 2.0, 3.0, 4.0])
    got = apply_rope(u, cos, sin)
    want = [1 * math.cos(1) - 3 * math.sin(1),
            2 * math.cos(0.1) - 4 * math.sin(0.1),
            3 * math.cos(1) + 1 * math.sin(1),
            4 * math.cos(0.1) + 2 * math.sin(0.1)]
    assert np.allclose(got, want, rtol=0, atol=1e-15)


def test_rope_hd2_is_plane_rotation_by_p_radians():
    for p in [0, 1, 7, 1023, 32790]:
        cos, sin = rope_cos_sin(p, 2, 5e5, np.float64)
        got = apply_rope(np.array([1.0, 0.0]), cos, sin)
        assert np.allclose(got, [math.cos(p), math.sin(p)], atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(2)
    hd, theta = 128, 1e6
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)
    c0, s0 = rope_cos_sin(0, hd, theta, np.float64)
    assert np.array_equal(apply_rope(q, c0, s0), q)
    for p in [1, 100, 32767]:
        c, s = rope_cos_sin(p, hd, theta, np.float64)
        assert np.isclose(np.linalg.norm(apply_rope(q, c, s)), np.linalg.norm(q), rtol=1e-13)
    # <R_m q, R_n k> depends only on m - n
    def dot(m, n):
        cm, sm = rope_cos_sin(m, hd, theta, np.float64)
        cn, sn = rope_cos_sin(n, hd, theta, np.float64)
        return apply_rope(q, cm, sm) @ apply_rope(k, cn, sn)
    assert np.isclose(dot(10, 3), dot(1007, 1000), rtol=1e-9)
    assert np.isclose(dot(5, 5), q @ k, rtol=1e-12)


def test_rope_angle_formed_in_fp64():
    # at p = 32790 an FP32 angle p*inv_freq would be off by up to ~1e-3 rad; the FP64 angle rounded once is not.
    hd, theta, p = 128, 1e6, 32790
    c, s = rope_cos_sin(p, hd, theta, np.float32)
    i = np.arange(hd // 2)
    phi = p * theta ** (-2.0 * i / hd)
    assert np.array_equal(c, np.cos(phi).astype(np.float32))
    assert np.array_equal(s, np.sin(phi).astype(np.float32))


# ---------------------------------------------------------------------------
# Attention.  Catches: missing 1/sqrt(hd), softmax over the wrong axis,
# missing max subtraction overflow, wrong weighting of V.
# ---------------------------------------------------------------------------

def _attend_bruteforce(q, K, V):
    L, hd = K.shape
    s = []
    for j in range(L):
        acc = 0.0
        for d in range(hd):
            acc += float(q[d]) * float(K[j, d])
        s.append(acc / math.sqrt(hd))
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = sum(e)
    out = []
    for d in range(hd):
        out.append(sum(e[j] / z * float(V[j, d]) for j in range(L)))
    return np.array(out)


def test_attend_bruteforce_tiny():
    rng = np.random.default_rng(3)
    for L in [1, 2, 5, 8]:
        for hd in [2, 4, 8]:
            q = rng.standard_normal(hd)
            K = rng.standard_normal((L, hd)) * 2
            V = rng.standard_normal((L, hd))
            assert np.allclose(attend(q, K, V), _attend_bruteforce(q, K, V), rtol=1e-12, atol=1e-13)


def test_attend_weights_sum_to_one_and_scale():
    rng = np.random.default_rng(4)
    L = 16
    q = rng.standard_normal(L)
    K = rng.standard_normal((L, L)) * 3
    w = attend(q, K, np.eye(L))           # V = I returns the softmax weights
    assert np.isclose(w.sum(), 1.0, rtol=1e-14)
    assert np.all(w > 0)
    # two keys along e0: weights are a logistic of (a - b) q0 / sqrt(hd)
    hd = 16
    q = np.zeros(hd); q[0] = 2.0
    K = np.zeros((2, hd)); K[0, 0] = 1.5; K[1, 0] = -0.5
    w = attend(q, K, np.eye(2, hd))[:2]
    p0 = 1.0 / (1.0 + math.exp(-(2.0 * 1.5 - 2.0 * -0.5) / math.sqrt(hd)))
    assert np.allclose(w, [p0, 1 - p0], rtol=1e-14)


def test_attend_single_position_returns_v_exactly():
    rng = np.random.default_rng(5)
    for dt in [np.float32, np.float64]:
        q = rng.standard_normal(64).astype(dt) * 100
        K = rng.standard_normal((1, 64)).astype(dt)
        V = rng.standard_normal((1, 64)).astype(dt)
        assert np.array_equal(attend(q, K, V), V[0])


def test_attend_equal_keys_is_mean_of_v():
    rng = np.random.default_rng(6)
    q = rng.standard_normal(8)
    K = np.tile(rng.standard_normal(8), (10, 1))
    V = rng.standard_normal((10, 8))
    assert np.allclose(attend(q, K, V), V.mean(axis=0), rtol=1e-13)


def test_attend_large_scores_do_not_overflow():
    q = np.full(64, 50.0, dtype=np.float32)
    K = np.full((3, 64), 40.0, dtype=np.float32)
    K[1] = 41.0
    V = np.eye(3, 64, dtype=np.float32)
    w = attend(q, K, V)[:3]
    assert np.all(np.isfinite(w)) and np.isclose(w.sum(), 1.0, rtol=1e-6)


# ---------------------------------------------------------------------------
# SiLU.  Catches: sigmoid instead of silu, sign errors.
# ---------------------------------------------------------------------------

def test_silu_values():
    z = np.array([0.0, 1.0, -1.0, 30.0, -30.0])
    s = silu(z)
    assert s[0] == 0.0
    assert np.isclose(s[1], 0.7310585786300049, rtol=1e-15)        # 1 / (1 + e^-1)
    assert np.isclose(s[2], -0.2689414213699951, rtol=1e-15)       # -1 / (1 + e)
    assert np.isclose(s[3], 30.0, rtol=1e-12)
    assert abs(s[4]) < 1e-11


# ---------------------------------------------------------------------------
# FP32 matrix-vector products stay within the classical error bound.
# ---------------------------------------------------------------------------

def test_fp32_matvec_within_error_bound():
    rng = np.random.default_rng(7)
    for K in [256, 2048, 9728]:
        W = (rng.standard_normal((64, K)) * 0.02).astype(np.float32)
        x = rng.standard_normal(K).astype(np.float32)
        y32 = (W @ x).astype(np.float64)
        y64 = W.astype(np.float64) @ x.astype(np.float64)
        bound = K * 2.0 ** -24 * (np.abs(W).astype(np.float64) @ np.abs(x).astype(np.float64))
        assert np.all(np.abs(y32 - y64) <= bound)


# ---------------------------------------------------------------------------
# Whole decode step: closed forms on hand-built models.
# ---------------------------------------------------------------------------

class Cfg:
    def __init__(self, **kw):
        self.n_layers = 2
        self.hidden = 8
        self.n_heads = 2
        self.n_kv_heads = 1
        self.head_dim = 4
        self.ffn = 8
        self.vocab = 16
        self.rope_theta = 10000.0
        self.rms_eps = 1e-5
        self.qk_norm = False
        self.tie_embeddings = True
        self.__dict__.update(kw)


def _b(a):
    return float_to_bf16_bits(np.asarray(a, dtype=np.float64))


def _zero_model(c, rng):
    H, F, hd = c.hidden, c.ffn, c.head_dim
    qr, kr = c.n_heads * hd, c.n_kv_heads * hd
    layers = []
    for _ in range(c.n_layers):
        d = dict(attn_norm=_b(np.ones(H)), wq=_b(np.zeros((qr, H))), wk=_b(np.zeros((kr, H))),
                 wv=_b(np.zeros((kr, H))), wo=_b(np.zeros((H, qr))), mlp_norm=_b(np.ones(H)),
                 w_gate=_b(np.zeros((F, H))), w_up=_b(np.zeros((F, H))), w_down=_b(np.zeros((H, F))))
        if c.qk_norm:
            d["q_norm"] = _b(np.ones(hd))
            d["k_norm"] = _b(np.ones(hd))
        layers.append(d)
    return {"embed": _b(rng.standard_normal((c.vocab, H)) * 0.5), "final_norm": _b(np.ones(H)), "layers": layers}


def _kv(c, cap):
    shape = (c.n_layers, c.n_kv_heads, cap, c.head_dim)
    return {"k": np.zeros(shape, np.uint16), "v": np.zeros(shape, np.uint16)}


def test_step_residual_identity_and_head_closed_form():
    """W_o = W_down = 0: the residual stream stays E[t]; with E[t] = c*1 the final
    norm is c/sqrt(c^2+eps) and logits[r] = that times the row sum of E[r].
    Catches: residual not carried, head applied to un-normed x, wrong final gain."""
    c = Cfg()
    rng = np.random.default_rng(8)
    w = _zero_model(c, rng)
    w["embed"][3] = _b(np.full(c.hidden, 0.75))
    m = OracleModel(c, w, np.float64)
    logits, hidden = m.step(_kv(c, 4), 3, 0)
    assert np.array_equal(hidden[0], np.full(c.hidden, 0.75)) and np.array_equal(hidden[1], hidden[0])
    E = bf16_bits_to_float(w["embed"], np.float64)
    s = 0.75 / math.sqrt(0.75 ** 2 + c.rms_eps)
    assert np.allclose(logits, s * E.sum(axis=1), rtol=1e-13)


def test_step_uniform_attention_is_mean_of_cached_v_including_current():
    """W_q = 0 makes every score 0, so each head returns the mean of V over
    positions 0..p, where V[p] is this step's bf16-rounded v.  With W_o = I
    and no MLP, x1 = x0 + concat_h mean_j V[g(h)][j].
    Catches: current position excluded, v not rounded, GQA map, residual order."""
    c = Cfg(n_layers=1, n_heads=2, n_kv_heads=1, head_dim=4, hidden=8)
    rng = np.random.default_rng(9)
    w = _zero_model(c, rng)
    w["embed"][5] = _b(np.full(8, 0.5))
    wv = np.zeros((4, 8)); wv[0, 0] = 0.3; wv[1, 1] = -1.7; wv[2, :] = 0.125; wv[3, 7] = 2.0
    w["layers"][0]["wv"] = _b(wv)
    w["layers"][0]["wo"] = _b(np.eye(8))
    kv = _kv(c, 8)
    p = 3
    cached = rng.standard_normal((p, 4))
    kv["v"][0, 0, :p] = _b(cached)
    m = OracleModel(c, w, np.float64)
    _, hidden = m.step(kv, 5, p)
    s = 0.5 / math.sqrt(0.25 + c.rms_eps)                     # rmsnorm of 0.5*1
    v_now = (torch.tensor(bf16_bits_to_float(w["layers"][0]["wv"], np.float64) @ np.full(8, s))
             .to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy())
    allv = np.vstack([bf16_bits_to_float(_b(cached), np.float64), v_now])
    mean_v = allv.mean(axis=0)
    want = 0.5 + np.concatenate([mean_v, mean_v])           # both q heads read KV head 0
    assert np.allclose(hidden[0], want, rtol=1e-13)
    assert np.array_equal(kv["v"][0, 0, p], _torch_bits(v_now.astype(np.float32)))


def test_step_gqa_mapping_consecutive_heads_share_kv():
    """n_heads = 4, n_kv_heads = 2: heads 0, 1 read KV head 0 and heads 2, 3 read
    KV head 1 (h // 2), not h % 2.  Catches a wrong GQA map."""
    c = Cfg(n_layers=1, n_heads=4, n_kv_heads=2, head_dim=2, hidden=8)
    rng = np.random.default_rng(10)
    w = _zero_model(c, rng)
    w["layers"][0]["wo"] = _b(np.eye(8))
    kv = _kv(c, 4)
    p = 2
    kv["v"][0, 0, :p] = _b(np.full((p, 2), 1.0))
    kv["v"][0, 1, :p] = _b(np.full((p, 2), 4.0))
    m = OracleModel(c, w, np.float64)
    x0 = bf16_bits_to_float(w["embed"][1], np.float64)
    _, hidden = m.step(kv, 1, p)
    a, b = 1.0 * p / (p + 1), 4.0 * p / (p + 1)             # current v = 0 (W_v = 0)
    assert np.allclose(hidden[0] - x0, [a, a, a, a, b, b, b, b], rtol=1e-13)


def test_step_mlp_closed_form():
    """Attention off; W_gate = W_up = W_down = I (H = F = 2), x = [a, b]:
    x_out = x + silu(h) * h with h = x / rms(x).  Catches gate/up swap in the
    product, silu on the wrong branch, missing MLP norm."""
    c = Cfg(n_layers=1, hidden=2, ffn=2, n_heads=1, n_kv_heads=1, head_dim=2, vocab=4)
    rng = np.random.default_rng(11)
    w = _zero_model(c, rng)
    w["embed"][2] = _b([0.5, -1.25])
    w["layers"][0]["w_gate"] = _b(np.eye(2) * 2.0)
    w["layers"][0]["w_up"] = _b(np.eye(2))
    w["layers"][0]["w_down"] = _b(np.eye(2))
    m = OracleModel(c, w, np.float64)
    _, hidden = m.step(_kv(c, 2), 2, 0)
    x = np.array([0.5, -1.25])
    h = x / math.sqrt((0.25 + 1.5625) / 2 + c.rms_eps)
    sig = 1.0 / (1.0 + np.exp(-2.0 * h))
    want = x + (2.0 * h * sig) * h
    assert np.allclose(hidden[0], want, rtol=1e-13)


def test_step_qk_norm_makes_scores_scale_invariant():
    """With q/k RMSNorm, scaling W_q and W_k by 8 changes nothing (up to eps);
    without it the output changes.  Catches a q/k norm that is skipped."""
    rng = np.random.default_rng(12)
    outs = {}
    for qk in [True, False]:
        c = Cfg(n_layers=1, n_heads=2, n_kv_heads=1, head_dim=4, hidden=8, qk_norm=qk, rms_eps=1e-12)
        base = _zero_model(c, rng)
        wq = rng.standard_normal((8, 8)); wk = rng.standard_normal((4, 8)); wv = rng.standard_normal((4, 8))
        res = []
        for scale in [1.0, 8.0]:
            w = {**base, "layers": [dict(base["layers"][0])]}
            w["layers"][0]["wq"] = _b(wq * scale)
            w["layers"][0]["wk"] = _b(wk * scale)
            w["layers"][0]["wv"] = _b(wv)
            w["layers"][0]["wo"] = _b(np.eye(8))
            kv = _kv(c, 4)
            kv["k"][0, 0, :2] = _b(rng.standard_normal((2, 4)) * 0 + np.array([[1, 2, 3, 4], [-2, 1, 0.5, 3]]))
            kv["v"][0, 0, :2] = _b(np.array([[1, 0, 0, 0], [0, 1, 0, 0]]))
            _, hid = OracleModel(c, w, np.float64).step(kv, 0, 2)
            res.append(hid[0])
        outs[qk] = res
    assert np.allclose(outs[True][0], outs[True][1], rtol=1e-9)
    assert not np.allclose(outs[False][0], outs[False][1], rtol=1e-3)


def test_step_untied_head_equal_to_embedding_matches_tied():
    c = Cfg()
    rng = np.random.default_rng(13)
    w = _zero_model(c, rng)
    w["layers"][0]["wv"] = _b(rng.standard_normal((4, 8)) * 0.3)
    w["layers"][0]["wo"] = _b(rng.standard_normal((8, 8)) * 0.3)
    l1, _ = OracleModel(c, w, np.float64).step(_kv(c, 2), 1, 0)
    c2 = Cfg(tie_embeddings=False)
    w2 = dict(w, lm_head=w["embed"].copy())
    l2, _ = OracleModel(c2, w2, np.float64).step(_kv(c2, 2), 1, 0)
    assert np.array_equal(l1, l2)
    w3 = dict(w, lm_head=_b(rng.standard_normal((c.vocab, c.hidden))))
    l3, _ = OracleModel(c2, w3, np.float64).step(_kv(c2, 2), 1, 0)
    assert not np.allclose(l1, l3)


def test_step_kv_written_after_rope_at_position():
    """k is cached after RoPE at position p: with hd = 2 and W_k giving k = [r, 0],
    the cached key is bf16([r cos p, r sin p]).  Catches caching the unrotated key."""
    c = Cfg(n_layers=1, n_heads=1, n_kv_heads=1, head_dim=2, hidden=2, ffn=2, vocab=4)
    rng = np.random.default_rng(14)
    w = _zero_model(c, rng)
    w["embed"][1] = _b([1.0, 1.0])
    wk = np.array([[0.75, 0.0], [0.0, 0.0]])
    w["layers"][0]["wk"] = _b(wk)
    kv = _kv(c, 8)
    p = 5
    OracleModel(c, w, np.float64).step(kv, 1, p)
    s = 1.0 / math.sqrt(1.0 + c.rms_eps)
    r = 0.75 * s
    want = torch.tensor([r * math.cos(p), r * math.sin(p)], dtype=torch.float64).to(torch.float32)
    assert np.array_equal(kv["k"][0, 0, p], _torch_bits(want.numpy()))


def test_decode_teacher_forced_on_own_tokens_equals_free_running():
    c = Cfg(vocab=32)
    rng = np.random.default_rng(15)
    w = _zero_model(c, rng)
    for d in w["layers"]:
        for k in ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"]:
            d[k] = _b(rng.standard_normal(bf16_bits_to_float(d[k]).shape) * 0.3)
    w["embed"] = _b(rng.standard_normal((32, 8)))
    m = OracleModel(c, w, np.float32)
    free = m.decode(_kv(c, 12), 7, 0, 10)
    forced = m.decode(_kv(c, 12), 7, 0, 10, teacher=list(free["tokens"][:-1]))
    assert np.array_equal(free["tokens"], forced["tokens"])
    assert np.array_equal(free["logits"], forced["logits"])


def _verify_model(c, seed):
    rng = np.random.default_rng(seed)
    w = _zero_model(c, rng)
    for d in w["layers"]:
        for k in ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"]:
            d[k] = _b(rng.standard_normal(bf16_bits_to_float(d[k]).shape) * 0.3)
    w["embed"] = _b(rng.standard_normal((c.vocab, 8)))
    return OracleModel(c, w, np.float32)


def test_verify_accepts_the_greedy_continuation_whole():
    """V1: drafts equal to free-running greedy decoding are all accepted, and the step yields that
    continuation one token further (the bonus token), with the greedy tokens as its argmaxes."""
    c = Cfg(vocab=32)
    m = _verify_model(c, 21)
    free = m.decode(_kv(c, 12), 7, 0, 9)
    g = [int(t) for t in free["tokens"]]
    r = m.verify(_kv(c, 12), [7] + g[:7], 0)
    assert r["accepted"] == 7
    assert list(r["tokens"]) == g[:8]
    assert list(r["argmax"]) == g[:8]


def test_verify_stops_at_the_first_wrong_draft():
    """V1: a wrong draft at position j (1-based) ends acceptance at j - 1 drafts and the step yields
    the greedy token there instead; drafts after it do not matter."""
    c = Cfg(vocab=32)
    m = _verify_model(c, 22)
    g = [int(t) for t in m.decode(_kv(c, 12), 3, 0, 8)["tokens"]]
    for j in (1, 3, 6):
        drafts = list(g[:7])
        drafts[j - 1] = (g[j - 1] + 5) % 32
        for k in range(j, 7):  # later drafts: anything, even the greedy ones
            drafts[k] = (g[k] + 11) % 32 if k % 2 else g[k]
        r = m.verify(_kv(c, 12), [3] + drafts, 0)
        assert r["accepted"] == j - 1, j
        assert list(r["tokens"]) == g[:j], j


def test_verify_of_one_token_is_one_greedy_step():
    c = Cfg(vocab=32)
    m = _verify_model(c, 23)
    g = int(m.decode(_kv(c, 12), 5, 2, 1)["tokens"][0])
    r = m.verify(_kv(c, 12), [5], 2)
    assert r["accepted"] == 0 and list(r["tokens"]) == [g] and list(r["argmax"]) == [g]


def test_fp32_oracle_close_to_fp64_on_tiny_synthetic_model():
    from tile_scheduled_persistent_amd import synth
    from tile_scheduled_persistent_amd.configs import TINY
    w = synth.weights_as_bits(synth.make_weights(TINY))
    k, v = synth.make_kv(TINY, 24, 10)
    kv32 = {"k": synth.bits(k), "v": synth.bits(v)}
    kv64 = {"k": kv32["k"].copy(), "v": kv32["v"].copy()}
    toks = synth.make_tokens(TINY, 4)
    r32 = OracleModel(TINY, w, np.float32).decode(kv32, toks[0], 10, 4, teacher=toks[1:])
    r64 = OracleModel(TINY, w, np.float64).decode(kv64, toks[0], 10, 4, teacher=toks[1:])
    rel = np.linalg.norm(r32["hidden"] - r64["hidden"], axis=-1) / np.linalg.norm(r64["hidden"], axis=-1)
    assert rel.max() < 1e-5
    assert np.abs(r32["logits"] - r64["logits"]).max() < 1e-4


# ---------------------------------------------------------------------------
# Plumbing of the whole step: which weights and which gain each stage reads.
# Every layer and every norm gets its own, non-unit gain, so that a stage
# reading another stage's (or another layer's) tensors changes the result.
# ---------------------------------------------------------------------------

def test_step_layers_and_norm_gains_closed_form():
    """Two layers with distinct weights and distinct, non-unit gains.  Layer 0 passes x through
    (W_o = W_down = 0); layer 1 has attention off and an MLP W_gate = 2I, W_up = I, W_down = I.
    Then hidden[0] = x0, hidden[1] = x0 + silu(2h) * h with h = x0 / rms(x0) * g_mlp[1], and
    logits = E (x1 / rms(x1) * g_final).
    Catches: a layer reading another layer's weights or gains, the MLP norm taking the attention
    gain, the final-norm gain dropped."""
    c = Cfg(n_layers=2, hidden=4, ffn=4, n_heads=1, n_kv_heads=1, head_dim=4, vocab=8)
    rng = np.random.default_rng(16)
    w = _zero_model(c, rng)
    ga = [np.array([1.25, 0.75, 1.5, 0.5]), np.array([0.625, 1.75, 1.125, 0.875])]
    gm = [np.array([0.5, 1.5, 0.75, 1.25]), np.array([1.375, 0.625, 0.25, 2.0])]
    gf = np.array([0.75, 1.25, 2.0, 0.5])
    for l in range(2):
        w["layers"][l]["attn_norm"] = _b(ga[l])
        w["layers"][l]["mlp_norm"] = _b(gm[l])
    # layer 0's MLP is live up to W_down = 0, so reading its gate/up instead of layer 1's is not enough
    w["layers"][0]["w_gate"] = _b(np.eye(4) * -3.0)
    w["layers"][0]["w_up"] = _b(np.eye(4) * 0.5)
    w["layers"][1]["w_gate"] = _b(np.eye(4) * 2.0)
    w["layers"][1]["w_up"] = _b(np.eye(4))
    w["layers"][1]["w_down"] = _b(np.eye(4))
    w["final_norm"] = _b(gf)
    x0 = np.array([0.5, -1.25, 0.75, 2.0])
    w["embed"][3] = _b(x0)
    logits, hidden = OracleModel(c, w, np.float64).step(_kv(c, 2), 3, 0)
    assert np.array_equal(hidden[0], x0)
    h = x0 / math.sqrt(np.mean(x0 * x0) + c.rms_eps) * gm[1]
    x1 = x0 + (2.0 * h / (1.0 + np.exp(-2.0 * h))) * h
    assert np.allclose(hidden[1], x1, rtol=1e-13, atol=0)
    E = bf16_bits_to_float(w["embed"], np.float64)
    hf = x1 / math.sqrt(np.mean(x1 * x1) + c.rms_eps) * gf
    assert np.allclose(logits, E @ hf, rtol=1e-12, atol=1e-15)


def test_step_qk_norm_before_rope_with_own_gains():
    """Per-head q/k RMSNorm with distinct non-unit gains, then RoPE, on head_dim 2 (one frequency,
    angle = position).  W_q, W_k pick the first normed input coordinate, so q_raw = [a, 0] and
    k_raw = [b, 0]; normed: [g_q0 a / sqrt(a^2/2 + eps), 0] and [g_k0 b / sqrt(b^2/2 + eps), 0];
    rotated by p.  The cached key is that vector rounded to BF16; the attention output over
    (cached position 0, current position 1) is w0 V0 + w1 v1 with softmax weights of q.K / sqrt(2).
    Catches: q/k norm after RoPE, the k norm taking the q gain (or the reverse)."""
    c = Cfg(n_layers=1, hidden=2, ffn=2, n_heads=1, n_kv_heads=1, head_dim=2, vocab=4, qk_norm=True,
            rms_eps=1e-6)
    rng = np.random.default_rng(17)
    w = _zero_model(c, rng)
    ga = np.array([1.5, 0.5])
    gq = np.array([0.25, 3.0])
    gk = np.array([2.0, 0.5])
    L0 = w["layers"][0]
    L0["attn_norm"] = _b(ga)
    L0["mlp_norm"] = _b([0.875, 1.625])
    L0["q_norm"] = _b(gq)
    L0["k_norm"] = _b(gk)
    L0["wq"] = _b([[1.0, 0.0], [0.0, 0.0]])
    L0["wk"] = _b([[0.75, 0.0], [0.0, 0.0]])
    L0["wv"] = _b([[0.0, 0.0], [0.0, 1.0]])
    L0["wo"] = _b(np.eye(2))
    w["embed"][1] = _b([1.0, 1.0])
    kv = _kv(c, 4)
    kv["k"][0, 0, 0] = _b([1.0, 2.0])
    kv["v"][0, 0, 0] = _b([1.0, 0.0])
    p, eps = 1, c.rms_eps
    _, hidden = OracleModel(c, w, np.float64).step(kv, 1, p)
    h = np.array([1.0, 1.0]) / math.sqrt(1.0 + eps) * ga
    a, b = h[0], 0.75 * h[0]
    qa = gq[0] * a / math.sqrt(a * a / 2 + eps)
    ka = gk[0] * b / math.sqrt(b * b / 2 + eps)
    q = np.array([qa * math.cos(p), qa * math.sin(p)])
    k_now = np.array([ka * math.cos(p), ka * math.sin(p)])
    cached = bf16_bits_to_float(kv["k"][0, 0, p], np.float64)
    assert np.allclose(cached, k_now, rtol=2.0 ** -8, atol=0)           # rounded to BF16 (half an ulp)
    s0 = q @ np.array([1.0, 2.0]) / math.sqrt(2.0)
    s1 = q @ cached / math.sqrt(2.0)
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    v1 = bf16_bits_to_float(kv["v"][0, 0, p], np.float64)
    assert np.allclose(v1, [0.0, h[1]], rtol=2.0 ** -8, atol=0)
    want = np.array([1.0, 1.0]) + (1.0 - w1) * np.array([1.0, 0.0]) + w1 * v1
    assert np.allclose(hidden[0], want, rtol=1e-12, atol=0)


def test_decode_argmax_ties_take_the_lowest_index():
    """Two identical embedding rows (tied head) give exactly equal logits; with them dominant the
    greedy token is the lower of the two indices, whatever the input.  Catches an argmax that
    keeps the last maximum."""
    c = Cfg(vocab=16)
    rng = np.random.default_rng(18)
    w = _zero_model(c, rng)
    row = np.full(c.hidden, 2.0)
    w["embed"][5] = _b(row)
    w["embed"][11] = _b(row)
    w["embed"][2] = _b(np.full(c.hidden, 0.5))
    res = OracleModel(c, w, np.float64).decode(_kv(c, 4), 2, 0, 3)
    assert res["logits"][0][5] == res["logits"][0][11] == res["logits"][0].max()
    assert list(res["tokens"]) == [5, 5, 5]


def test_widened_cache_path_equals_the_plain_path():
    """The optional FP32 shadow of the cache (widened once, updated on every write) gives
    exactly the plain path's tokens, logits, hidden states and cache bits."""
    from tile_scheduled_persistent_amd import synth
    from tile_scheduled_persistent_amd.configs import TINY
    w = synth.weights_as_bits(synth.make_weights(TINY))
    k, v = synth.make_kv(TINY, 24, 10)
    kva = {"k": synth.bits(k), "v": synth.bits(v)}
    kvb = {"k": kva["k"].copy(), "v": kva["v"].copy()}
    toks = synth.make_tokens(TINY, 6)
    m = OracleModel(TINY, w, np.float32)
    a = m.decode(kva, toks[0], 10, 6, teacher=toks[1:])
    b = m.decode(kvb, toks[0], 10, 6, teacher=toks[1:], widen_kv_once=True)
    for key in ("tokens", "logits", "hidden"):
        assert np.array_equal(a[key], b[key])
    assert np.array_equal(kva["k"], kvb["k"]) and np.array_equal(kva["v"], kvb["v"])


# ---------------------------------------------------------------------------
# Weight-only INT8 (per-row symmetric codes, FP32 scales).  Catches: truncation
# instead of round-half-even, a scale of max/128, a dropped scale, the LM head
# left in BF16, the embedding lookup quantized.
# ---------------------------------------------------------------------------

from oracle import dequantize_rows_int8, quantize_rows_int8  # noqa: E402


def test_int8_quantizer_hand_worked_ties_and_zero_row():
    # max |W| = 127/128, so s = 2^-7 exactly; W / s = 127, 2.5, 3.5, -2.5, 0 -> ties go to the even code
    w = _b([[127 / 128, 2.5 * 2 ** -7, 3.5 * 2 ** -7, -2.5 * 2 ** -7, 0.0], [0.0, 0.0, 0.0, 0.0, 0.0]])
    q, s = quantize_rows_int8(w)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert q.tolist() == [[127, 2, 4, -2, 0], [0, 0, 0, 0, 0]]
    assert s.tolist() == [2 ** -7, 0.0]
    assert np.array_equal(dequantize_rows_int8(q, s, np.float64)[1], np.zeros(5))


def test_int8_quantizer_bounds_on_random_rows():
    rng = np.random.default_rng(19)
    mags = 10.0 ** rng.integers(-6, 4, 300)
    w = _b(rng.standard_normal((300, 257)) * mags[:, None])
    q, s = quantize_rows_int8(w)
    W = bf16_bits_to_float(w, np.float64)
    amax = np.abs(W).max(axis=1)
    assert np.array_equal(s, (amax.astype(np.float32) / np.float32(127.0)).astype(np.float32))
    assert np.abs(q.astype(np.int32)).max() <= 127
    # the largest entry of each row takes the code +-127
    assert np.all(np.abs(q.astype(np.int32)).max(axis=1) == 127)
    # every entry within half a step (plus the FP32 division's rounding) of its dequantized value
    err = np.abs(W - q.astype(np.float64) * s.astype(np.float64)[:, None])
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 128 * 2.0 ** -23))


def test_int8_step_computes_with_the_dequantized_codes():
    """One layer, attention off, an MLP whose down projection has rows [1, 0.3] and [0.6, -1]: in the
    INT8 model the output is x + (q * s) a with the hand-computed codes (127, 38) / 127 and
    (64, -127) / 127, not the BF16 product; the embedding row is looked up unquantized and the tied
    head is quantized (its rows E[r] give codes of their own).  Catches: INT8 ignored, the scale
    dropped, the head left in BF16, the lookup quantized."""
    c = Cfg(n_layers=1, hidden=2, ffn=2, n_heads=1, n_kv_heads=1, head_dim=2, vocab=4)
    rng = np.random.default_rng(20)
    w = _zero_model(c, rng)
    w["embed"] = _b([[0.5, -1.25], [1.0, 0.3], [0.75, 0.5], [-0.25, 0.125]])
    w["layers"][0]["w_gate"] = _b(np.eye(2) * 2.0)
    w["layers"][0]["w_up"] = _b(np.eye(2))
    w["layers"][0]["w_down"] = _b([[1.0, 0.3], [0.6, -1.0]])
    m = OracleModel(c, w, np.float64, weight_format="int8")
    logits, hidden = m.step(_kv(c, 2), 0, 0)
    x = np.array([0.5, -1.25])                                   # BF16 lookup, exact
    h = x / math.sqrt(np.mean(x * x) + c.rms_eps)
    # gate 2I and up I quantize exactly (codes 127 with scales 2/127 and 1/127)
    s_g, s_u = np.float32(2.0) / np.float32(127.0), np.float32(1.0) / np.float32(127.0)
    gate = 127 * float(s_g) * h
    up = 127 * float(s_u) * h
    a = gate / (1.0 + np.exp(-gate)) * up
    sd = float(s_u)
    w_down = np.array([[127, 38], [round(0.6015625 * 127), -127]]) * sd  # 0.6 is 0.6015625 in BF16: code 76
    assert round(0.6015625 * 127) == 76
    x1 = x + w_down @ a
    assert np.allclose(hidden[0], x1, rtol=1e-12, atol=0)
    E = bf16_bits_to_float(w["embed"], np.float64)
    qE, sE = quantize_rows_int8(w["embed"])
    hf = x1 / math.sqrt(np.mean(x1 * x1) + c.rms_eps)
    assert np.allclose(logits, (qE.astype(np.float64) * sE.astype(np.float64)[:, None]) @ hf, rtol=1e-12)
    assert not np.allclose(logits, E @ hf, rtol=1e-6)            # the head really is quantized


# ---------------------------------------------------------------------------
# Sampling (S1): hand-worked draws, closed-form frequencies over a grid of uniforms, support of
# the top-k and top-p filters, the tie order, and the per-step uniform in decode.
# ---------------------------------------------------------------------------
from oracle import sample_token  # noqa: E402


def _grid_frequencies(z, temperature, top_k, top_p, n=20000):
    counts = np.zeros(len(z))
    for j in range(n):
        counts[sample_token(z, temperature, top_k, top_p, (j + 0.5) / n)] += 1
    return counts / n


def test_sampling_hand_worked_example():
    """Logits 2, 1, 0, -1 on token ids 3, 0, 2, 1 at T = 1: weights 1, 1/e, 1/e^2 for the three kept
    (top_k = 3); cumulative 1, 1 + 1/e = 1.368, 1.503.  top_p = 0.8 needs 0.8 * 1.503 = 1.203, so the
    prefix is ids (3, 0) with total 1.368: u = 0.5 -> 0.684 < 1 -> id 3; u = 0.75 -> 1.026 > 1 -> id 0.
    top_p = 1: u = 0.95 -> 1.428 > 1.368 -> id 2.  Catches: ids not carried with their logits, the
    temperature or the top-p threshold misapplied, the draw scaled by the wrong total."""
    z = np.zeros(4, np.float32)
    z[[3, 0, 2, 1]] = [2, 1, 0, -1]
    e1, e2 = math.exp(-1), math.exp(-2)
    assert 0.8 * (1 + e1 + e2) > 1 and 0.8 * (1 + e1 + e2) < 1 + e1
    assert sample_token(z, 1.0, 3, 0.8, 0.5) == 3
    assert sample_token(z, 1.0, 3, 0.8, 0.75) == 0
    assert sample_token(z, 1.0, 3, 0.8, 0.999) == 0
    assert sample_token(z, 1.0, 3, 1.0, 0.95) == 2
    assert sample_token(z, 1.0, 3, 1.0, 0.0) == 3
    assert 0.95 * (1 + e1 + e2) > 1 + e1
    # T = 0.5 doubles the gaps: weights 1, e^-2, e^-4; u = 0.9 of 1.154 = 1.039 > 1 -> id 0
    assert 0.9 * (1 + e2 + math.exp(-4)) > 1
    assert sample_token(z, 0.5, 3, 1.0, 0.9) == 0
    # at T = 2 the gaps halve: weights 1, e^-0.5, e^-1 (total 1.974); u = 0.6 -> 1.185 < 1.607 -> id 0,
    # u = 0.9 -> 1.777 > 1.607 -> id 2
    assert 1 < 0.6 * (1 + math.exp(-0.5) + e1) < 1 + math.exp(-0.5) < 0.9 * (1 + math.exp(-0.5) + e1)
    assert sample_token(z, 2.0, 3, 1.0, 0.6) == 0
    assert sample_token(z, 2.0, 3, 1.0, 0.9) == 2


def test_sampling_top1_and_tiny_top_p_are_the_argmax():
    """top_k = 1, or top_p below the largest probability, leaves only the argmax (lowest id on
    ties) whatever u is.  Catches: a filter that keeps too much, ties broken by the higher id."""
    rng = np.random.default_rng(41)
    for trial in range(20):
        z = rng.standard_normal(50).astype(np.float32)
        z[[7, 31]] = z.max() + 1.0  # a tie for the maximum: id 7 wins
        for u in (0.0, 0.3, 0.999):
            assert sample_token(z, 0.8, 1, 1.0, u) == 7
            assert sample_token(z, 0.8, 10, 1e-6, u) == 7


def test_sampling_frequencies_are_the_softmax():
    """With every token kept, the fraction of a fine grid of uniforms that draws each token is
    its softmax probability at temperature T (closed form, FP64).  Catches: temperature applied
    as a product, a missing or doubled exponent, an offset draw."""
    z = np.array([0.3, -1.2, 2.0, 0.7, -0.1, 1.1], np.float32)
    for T in (0.7, 1.5):
        p = np.exp(z.astype(np.float64) / T)
        p /= p.sum()
        f = _grid_frequencies(z, T, len(z), 1.0)
        assert np.abs(f - p).max() < 2e-4, (T, f, p)


def test_sampling_top_k_and_top_p_supports():
    """top_k keeps the k largest logits and renormalises over them; top_p keeps the shortest
    prefix reaching p of that total.  Frequencies equal the renormalised closed form and no other
    token is ever drawn.  Catches: top-p taken over all V logits, the prefix one short or long,
    no renormalisation."""
    z = np.array([0.5, 2.5, -0.3, 1.9, 0.1, 2.2, -2.0, 1.0, 0.0, 1.4], np.float32)
    T = 0.9
    rank = np.argsort(-z, kind="stable")
    for k, p in ((4, 1.0), (4, 0.6), (10, 0.9), (6, 0.5)):
        w = np.exp((z[rank[:k]].astype(np.float64) - z[rank[0]]) / T)
        c = np.cumsum(w) / w.sum()
        n = int(np.argmax(c >= p)) + 1
        expect = np.zeros(len(z))
        expect[rank[:n]] = w[:n] / w[:n].sum()
        f = _grid_frequencies(z, T, k, p)
        assert np.abs(f - expect).max() < 2e-4, (k, p, f, expect)


def test_sampling_equal_logits_take_increasing_ids():
    """Equal logits rank by increasing token id: with logits 0, 3, 3, 3, 1 and top_k = 2 only ids 1
    and 2 are ever drawn, half the time each.  Catches: ties by decreasing id, a top-p prefix
    that must exceed p rather than reach it."""
    z = np.array([0, 3, 3, 3, 1], np.float32)
    f = _grid_frequencies(z, 1.0, 2, 1.0, n=4000)
    assert np.allclose(f, [0, 0.5, 0.5, 0, 0])
    # a prefix that reaches top_p exactly is long enough: four equal weights, top_p = 1/2 needs
    # exactly 2 of 4 (exact in FP32), so only ids 0 and 1 are drawn
    z = np.array([3, 3, 3, 3, 0], np.float32)
    f = _grid_frequencies(z, 1.0, 4, 0.5, n=4000)
    assert np.allclose(f, [0.5, 0.5, 0, 0, 0])


def test_decode_sampling_uses_each_steps_uniform():
    """A model whose logits are all exactly equal (identical embedding rows, tied head): with
    top_k = 4 and T = 1 the weights are 1, 1, 1, 1 and the draw at step i is id floor(4 u_i), the
    strict inequality putting u = 0.25 at id 1.  Catches: the uniform of another step, a
    non-strict draw, decode not sampling."""
    c = Cfg(vocab=16)
    w = _zero_model(c, np.random.default_rng(19))
    w["embed"] = _b(np.full((c.vocab, c.hidden), 0.25))
    u = [0.1, 0.25, 0.6, 0.99, 0.5]
    res = OracleModel(c, w, np.float32).decode(_kv(c, 8), 3, 0, 5, sampling=(1.0, 4, 1.0), uniforms=u)
    assert np.all(res["logits"] == res["logits"][0][0])
    assert list(res["tokens"]) == [0, 1, 2, 3, 2]


# ---------------------------------------------------------------------------
# INT8 KV cache with smoothed keys (K1, K2): a hand-worked conversion, bounds per channel that only
# hold with smoothing, zero channels, and a step whose attention is the mean of the stored V.
# ---------------------------------------------------------------------------
from oracle import convert_kv_int8, dequantize_kv_rows, quantize_rows_f32_int8  # noqa: E402


def test_kv_int8_conversion_hand_worked():
    """K rows (1, 100) and (-2, 50): sigma = (2, 100); smoothed rows (0.5, 1) and (-1, 0.5), scale
    1/127 each; codes (64, 127) (63.5 rounds half to even) and (-127, 64); dequantized (64/127 * 2,
    100) and (-2, 64/127 * 100).  V rows (0.5, -0.25) and (1, 2): no smoothing; scales 0.5/127 and
    2/127; codes (127, -64) (-63.5 to even) and (64, 127).  Catches: no smoothing, smoothing of V,
    scale over 128, truncated codes, sigma left out of the dequantized K."""
    k = np.array([[1, 100], [-2, 50]], np.float32)[None, None]
    v = np.array([[0.5, -0.25], [1, 2]], np.float32)[None, None]
    c = convert_kv_int8({"k": float_to_bf16_bits(k), "v": float_to_bf16_bits(v)}, 2)
    assert np.array_equal(c["sigma"][0, 0], np.array([2, 100], np.float32))
    assert np.array_equal(c["kq"][0, 0], np.array([[64, 127], [-127, 64]], np.int8))
    assert np.array_equal(c["ks"][0, 0], np.full(2, np.float32(1) / np.float32(127), np.float32))
    assert np.array_equal(c["vq"][0, 0], np.array([[127, -64], [64, 127]], np.int8))
    assert np.array_equal(c["vs"][0, 0], np.array([np.float32(0.5) / np.float32(127), np.float32(2) / np.float32(127)]))
    kd = dequantize_kv_rows(c["kq"], c["ks"], c["sigma"][:, :, None, :], np.float64)[0, 0]
    assert np.allclose(kd, [[64 / 127 * 2, 100], [-2, 64 / 127 * 100]], rtol=1e-6)
    vd = dequantize_kv_rows(c["vq"], c["vs"], None, np.float64)[0, 0]
    assert np.allclose(vd, [[0.5, -0.5 * 64 / 127], [2 * 64 / 127, 2]], rtol=1e-6)


def test_kv_int8_errors_are_bounded_per_channel_by_smoothing():
    """Keys with per-channel scales U(0.5, 4) and one outlier channel (x100): sigma is each channel's
    largest |K| over the cached positions (computed here independently), and every dequantized entry
    is within sigma_c / 254 (half a code of the smoothed row, whose largest entry is at most 1) of
    the true key -- without smoothing the outlier's scale would swamp the small channels.  V entries
    are within half a code of their row's scale."""
    rng = np.random.default_rng(77)
    L, G, P, hd = 2, 3, 40, 16
    scale = rng.uniform(0.5, 4.0, size=(L, G, 1, hd))
    scale[:, :, :, 5] *= 100.0
    k = (rng.standard_normal((L, G, P, hd)) * scale).astype(np.float32)
    v = rng.standard_normal((L, G, P, hd)).astype(np.float32)
    kb, vb = float_to_bf16_bits(k), float_to_bf16_bits(v)
    c = convert_kv_int8({"k": kb, "v": vb}, P)
    kw = bf16_bits_to_float(kb, np.float64)
    vw = bf16_bits_to_float(vb, np.float64)
    assert np.array_equal(c["sigma"], np.abs(kw).max(axis=2).astype(np.float32))
    kd = dequantize_kv_rows(c["kq"], c["ks"], c["sigma"][:, :, None, :], np.float64)
    err = np.abs(kd - kw)
    assert np.all(err <= c["sigma"][:, :, None, :].astype(np.float64) / 254 * (1 + 1e-5) + 1e-30)
    vd = dequantize_kv_rows(c["vq"], c["vs"], None, np.float64)
    assert np.all(np.abs(vd - vw) <= c["vs"][..., None].astype(np.float64) / 2 * (1 + 1e-5))
    # the smoothing is what makes the small channels precise
    small = err[..., :5].max() / np.abs(kw[..., :5]).max()
    assert small < 1 / 200


def test_kv_int8_zero_channel_zero_row_and_unfilled_positions():
    k = np.zeros((1, 1, 4, 4), np.float32)
    k[0, 0, 0] = [1, 0, -3, 0]
    k[0, 0, 1] = [0.5, 0, 0, 0]
    v = np.zeros((1, 1, 4, 4), np.float32)
    c = convert_kv_int8({"k": float_to_bf16_bits(k), "v": float_to_bf16_bits(v)}, 2)
    assert np.array_equal(c["sigma"][0, 0], np.array([1, 1, 3, 1], np.float32))  # zero channels: 1
    assert np.all(c["vq"] == 0) and np.all(c["vs"] == 0)                          # zero rows: s = 0, q = 0
    assert np.all(c["kq"][0, 0, 2:] == 0) and np.all(c["ks"][0, 0, 2:] == 0)     # not filled
    assert np.array_equal(c["kq"][0, 0, 1], np.array([127, 0, 0, 0], np.int8))


def test_kv_int8_step_attends_the_stored_rows():
    """Zero W_q makes every score 0, so each head's attention output is the plain mean of the V rows
    it attends, the current one included, as stored (dequantized); with W_o the identity the layer's
    residual gains exactly that mean.  The current position's stored K and V are within half a code
    of their FP32 values (K as smoothed by the cache's sigma).  Catches: attending FP32 rows of the
    current position, V rows not dequantized with their own scale, the current row not written."""
    c = Cfg(n_layers=1)
    rng = np.random.default_rng(31)
    w = _zero_model(c, rng)
    H, nq, hd = c.hidden, c.n_heads, c.head_dim
    assert nq * hd == H
    w["layers"][0]["wo"] = _b(np.eye(H))
    wk = rng.standard_normal((c.n_kv_heads * hd, H)) * 0.05
    wv = rng.standard_normal((c.n_kv_heads * hd, H)) * 0.05
    w["layers"][0]["wk"] = _b(wk)
    w["layers"][0]["wv"] = _b(wv)
    cap, pos = 8, 5
    kvb = {"k": float_to_bf16_bits(rng.standard_normal((1, c.n_kv_heads, cap, hd)).astype(np.float32)),
           "v": float_to_bf16_bits(rng.standard_normal((1, c.n_kv_heads, cap, hd)).astype(np.float32))}
    kv8 = convert_kv_int8(kvb, pos)
    o = OracleModel(c, w, np.float64)
    tok = 3
    _, hidden = o.step(kv8, tok, pos)
    x = bf16_bits_to_float(w["embed"][tok], np.float64)
    attn = hidden[0] - x
    group = nq // c.n_kv_heads
    for hh in range(nq):
        g = hh // group
        vd = dequantize_kv_rows(kv8["vq"][0, g, :pos + 1], kv8["vs"][0, g, :pos + 1], None, np.float64)
        assert np.allclose(attn[hh * hd:(hh + 1) * hd], vd.mean(axis=0), rtol=1e-9, atol=1e-12)
    # the current row: FP32 k and v of this step (position 0 of RoPE is not used: pos = 5, so k is
    # rotated; compare V, which is not rotated, and K's stored scale against its definition)
    h = x / np.sqrt(np.mean(x * x) + c.rms_eps) * bf16_bits_to_float(w["layers"][0]["attn_norm"], np.float64)
    v_true = (bf16_bits_to_float(w["layers"][0]["wv"], np.float64) @ h).reshape(c.n_kv_heads, hd)
    vd = dequantize_kv_rows(kv8["vq"][0, :, pos], kv8["vs"][0, :, pos], None, np.float64)
    assert np.all(np.abs(vd - v_true) <= kv8["vs"][0, :, pos, None] / 2 * (1 + 1e-4) + 1e-7)
    assert np.all(kv8["ks"][0, :, pos] > 0) and np.any(kv8["kq"][0, :, pos] != 0)
