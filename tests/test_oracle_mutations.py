"""Mutation check of the oracle pins: each plausible mistake below, planted in a copy of
``oracle/decoder.py`` (on the CPU, in memory), must make at least one pin in
``test_oracle_pins.py`` fail.  A pin set that a planted mistake survives does not pin
that part of the oracle.

The mistakes cover the readings the oracle rests on (RoPE pairing, frequency and sign,
GQA map, attention scale and causal range, RMSNorm form, BF16 rounding, SwiGLU branch,
residual source), the plumbing of the step (which layer's weights and which gain
each stage reads, q/k norm before RoPE, the argmax tie rule), the INT8 weight codes, the INT8
KV cache (smoothing, scales, codes, dequantization) and the sampling draw (tie order, temperature, top-k and top-p supports, the draw's scale and
strictness, the per-step uniform) and the verify step's acceptance rule.
"""

import importlib.util
import os
import sys
import types

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DECODER = os.path.join(ROOT, "oracle", "decoder.py")
PINS = os.path.join(HERE, "test_oracle_pins.py")

# (name, text in decoder.py, replacement, replace every occurrence)
MUTATIONS = [
    ("verify compares the wrong draft", "int(a[n]) == tokens[n + 1]", "int(a[n]) == tokens[n]", False),
    ("verify yields the argmax after the next position", "[int(a[n])]", "[int(a[min(n + 1, m - 1)])]", False),
    ("verify without the correction token", "out = np.array(tokens[1:n + 1] + [int(a[n])], dtype=np.int64)",
     "out = np.array(tokens[1:n + 1], dtype=np.int64)", False),
    ("interleaved RoPE pairs", "a = u[..., :half]\n    b = u[..., half:]", "a = u[..., 0::2]\n    b = u[..., 1::2]", False),
    ("RoPE rotation sign", "a * cos - b * sin, b * cos + a * sin", "a * cos + b * sin, b * cos - a * sin", False),
    ("RoPE frequency exponent", "float(theta) ** (-2.0 * i / hd)", "float(theta) ** (-1.0 * i / hd)", False),
    ("GQA map h % n_kv", "g = hh // group", "g = hh % nkv", False),
    ("attention scale missing", "dt.type(1.0 / math.sqrt(q.shape[-1]))", "dt.type(1.0)", False),
    ("current position excluded", ": pos + 1]", ": max(pos, 1)]", True),
    ("current V not rounded",
     'Vc = bf16_bits_to_float(kv["v"][l, g, : pos + 1], dt)',
     'Vc = np.vstack([bf16_bits_to_float(kv["v"][l, g, :pos], dt), v[g][None]])', False),
    ("eps outside the sqrt", "(x / np.sqrt(ms + dt.type(eps))) * g", "(x / (np.sqrt(ms) + dt.type(eps))) * g", False),
    ("(1 + g) gain", "(x / np.sqrt(ms + dt.type(eps))) * g", "(x / np.sqrt(ms + dt.type(eps))) * (1 + g)", False),
    ("truncating BF16", "r = np.round(xf / ulp) * ulp", "r = np.trunc(xf / ulp) * ulp", False),
    ("SiLU on the up branch",
     'silu(self._get(l, "w_gate") @ h) * (self._get(l, "w_up") @ h)',
     '(self._get(l, "w_gate") @ h) * silu(self._get(l, "w_up") @ h)', False),
    ("q/k norm skipped", "if c.qk_norm:", "if False:", False),
    ("residual from the normed x", 'x = x + self._get(l, "wo")', 'x = h + self._get(l, "wo")', False),
    ("q/k norm after RoPE",
     '            if c.qk_norm:\n'
     '                q = rmsnorm(q, self._get(l, "q_norm"), eps)\n'
     '                k = rmsnorm(k, self._get(l, "k_norm"), eps)\n'
     '            q = apply_rope(q, cos, sin)\n'
     '            k = apply_rope(k, cos, sin)\n',
     '            q = apply_rope(q, cos, sin)\n'
     '            k = apply_rope(k, cos, sin)\n'
     '            if c.qk_norm:\n'
     '                q = rmsnorm(q, self._get(l, "q_norm"), eps)\n'
     '                k = rmsnorm(k, self._get(l, "k_norm"), eps)\n', False),
    ("every layer reads layer 0's tensors", "self._get(l, ", "self._get(0, ", True),
    ("final-norm gain dropped", 'rmsnorm(x, self._get(None, "final_norm"), eps)', "rmsnorm(x, np.ones_like(x), eps)", False),
    ("k norm takes the q gain", 'rmsnorm(k, self._get(l, "k_norm"), eps)', 'rmsnorm(k, self._get(l, "q_norm"), eps)', False),
    ("q norm takes the k gain", 'rmsnorm(q, self._get(l, "q_norm"), eps)', 'rmsnorm(q, self._get(l, "k_norm"), eps)', False),
    ("MLP norm takes the attention gain", 'rmsnorm(x, self._get(l, "mlp_norm"), eps)',
     'rmsnorm(x, self._get(l, "attn_norm"), eps)', False),
    ("widened cache row written unrounded", 'kv_wide["v"][l, :, pos, :] = bf16_bits_to_float(kv["v"][l, :, pos, :], dt)',
     'kv_wide["v"][l, :, pos, :] = v', False),
    ("INT8 codes truncated", "q = np.clip(np.rint(r), -127, 127)                     # np.rint",
     "q = np.clip(np.trunc(r), -127, 127)                     # np.rint", False),
    ("INT8 scale over 128", "s = (amax / np.float32(127.0)).astype(np.float32)      # FP32 division",
     "s = (amax / np.float32(128.0)).astype(np.float32)      # FP32 division", False),
    ("INT8 scale dropped", "return q.astype(dtype) * s.astype(dtype)[:, None]", "return q.astype(dtype) / np.float32(127.0) + 0 * s[:, None]", False),
    ("INT8 LM head left in BF16", 'return self._get(None, "embed", linear=True)', 'return self._get(None, "embed")', False),
    ("INT8 embedding lookup quantized", "return bf16_bits_to_float(self.w[\"embed\"][token], self.dtype).copy()",
     "return self._get(None, \"embed\", linear=True)[token].copy()", False),
    ("sampling ranks equal logits by decreasing id", "np.lexsort((np.arange(z.shape[0]), -z))",
     "np.lexsort((-np.arange(z.shape[0]), -z))", False),
    ("sampling temperature applied as a product", "(zk - zk[0]) / np.float32(temperature)",
     "(zk - zk[0]) * np.float32(temperature)", False),
    ("top-p prefix needs more than p", "cum >= need", "cum > need", True),
    ("top-p threshold over the unfiltered total", "need = np.float32(top_p) * cum[-1]",
     "need = np.float32(top_p) * np.float32(np.exp((z - zk[0]) / np.float32(temperature)).sum())", False),
    ("draw scaled by the kept total, not the prefix's", "target = np.float32(u) * cum[n - 1]",
     "target = np.float32(u) * cum[-1]", False),
    ("draw non-strict", "np.nonzero(cum[:n] > target)", "np.nonzero(cum[:n] >= target)", False),
    ("top-k keeps one more", ")[:top_k]   # decreasing", ")[:top_k + 1]   # decreasing", False),
    ("decode samples with the previous step's uniform", "float(uniforms[i])", "float(uniforms[i - 1])", False),
    ("INT8 KV without smoothing", "sigma = np.where(sigma > 0, sigma, np.float32(1.0)).astype(np.float32)",
     "sigma = np.ones_like(sigma, dtype=np.float32)", False),
    ("INT8 KV smooths V too", "quantize_rows_f32_int8(v)\n", "quantize_rows_f32_int8((v / sigma[:, :, None, :]).astype(np.float32))\n", False),
    ("INT8 KV scale over 128", "s = (amax / np.float32(127.0)).astype(np.float32)\n    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)\n    r = (x /",
     "s = (amax / np.float32(128.0)).astype(np.float32)\n    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)\n    r = (x /", False),
    ("INT8 KV codes truncated", "q = np.clip(np.rint(r), -127, 127)\n    q = np.where(s[..., None]", "q = np.clip(np.trunc(r), -127, 127)\n    q = np.where(s[..., None]", False),
    ("INT8 KV keys dequantized without sigma", "    if sigma is not None:\n        r = (r * sigma", "    if False:\n        r = (r * sigma", False),
    ("INT8 KV current V row stored unquantized", "kv[\"vq\"][l, :, pos, :], kv[\"vs\"][l, :, pos] = quantize_rows_f32_int8(v.astype(np.float32))",
     "kv[\"vq\"][l, :, pos, :], kv[\"vs\"][l, :, pos] = quantize_rows_f32_int8(v.astype(np.float32)); kv[\"vs\"][l, :, pos] *= 1.01", False),
    ("argmax keeps the last maximum", "toks[i] = int(np.argmax(logits))",
     "toks[i] = int(len(logits) - 1 - np.argmax(logits[::-1]))", False),
]


def _mutated_oracle(src: str) -> types.ModuleType:
    mod = types.ModuleType("oracle")
    mod.__file__ = DECODER
    exec(compile(src, DECODER + " (mutated)", "exec"), mod.__dict__)
    return mod


def _failing_pins(oracle_mod: types.ModuleType):
    """Run every zero-argument test of the pin module with `oracle` bound to oracle_mod;
    return the names of the tests that fail."""
    saved = sys.modules.get("oracle")
    sys.modules["oracle"] = oracle_mod
    try:
        spec = importlib.util.spec_from_file_location("_pins_under_mutation", PINS)
        pins = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(pins)
        failed = []
        for name in sorted(n for n in dir(pins) if n.startswith("test_")):
            try:
                getattr(pins, name)()
            except Exception:  # an assertion, or the mutated oracle raising: either way the pin caught it
                failed.append(name)
        return failed
    finally:
        if saved is not None:
            sys.modules["oracle"] = saved
        else:
            sys.modules.pop("oracle", None)


def test_unmutated_oracle_passes_every_pin():
    with open(DECODER) as f:
        src = f.read()
    assert _failing_pins(_mutated_oracle(src)) == []


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name,old,new,every", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, every):
    with open(DECODER) as f:
        src = f.read()
    n = src.count(old)
    assert n >= 1 and (every or n == 1), f"mutation site of '{name}' not found exactly once ({n})"
    mutated = src.replace(old, new) if every else src.replace(old, new, 1)
    failed = _failing_pins(_mutated_oracle(mutated))
    assert failed, f"no pin catches the planted mistake: {name}"
