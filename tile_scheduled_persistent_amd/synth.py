"""Seeded synthetic inputs (weights, KV cache, tokens) shared by the GPU path,
the tests and the CPU oracle.

This module holds no arithmetic of the decoder: it only draws numbers.  The
pages run trained checkpoints (Tiles page, "What the code contains": a pinned
Hugging Face checkpoint); none are available, so every tensor is random with
the shapes of the decoders in :mod:`configs`:

* linear weights and the embedding ~ N(0, 0.02), rounded to BF16;
* every RMSNorm gain ~ 1 + N(0, 0.01), rounded to BF16;
* the KV cache ~ N(0, 1), rounded to BF16, optionally with keys multiplied by
  a per-(layer, KV head, channel) scale ~ U(0.5, 4) before rounding;
* tokens ~ U[0, vocab);
* the uniforms of sampled decoding ~ U[0, 1), one per step, FP32.

Each tensor has its own torch generator seeded from (seed, model, tensor
index), in the canonical order embed, then per layer attn_norm, wq, wk, wv,
[q_norm, k_norm], wo, mlp_norm, w_gate, w_up, w_down, then final_norm.
Values depend on the device the generator runs on; a test uses one device for
both sides, and the oracle always receives the very bytes the GPU receives.
"""

from __future__ import annotations

import zlib
from typing import Dict, List

import numpy as np
import torch

from .configs import ModelConfig

SEED_WEIGHTS = 0
SEED_KV = 1
SEED_TOKENS = 2
SEED_KEY_SCALE = 3
SEED_UNIFORMS = 4

WEIGHT_STD = 0.02
GAIN_STD = 0.01


def _seed(seed: int, cfg: ModelConfig, index: int) -> int:
    h = zlib.crc32(cfg.name.encode())
    return (seed * 1_000_003 + h * 7919 + index * 104_729) % (2 ** 62)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std: float, mean: float, device, seed: int) -> torch.Tensor:
    g = _gen(device, seed)
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(mean=mean, std=std, generator=g)
    return t.to(torch.bfloat16)


def weight_names(cfg: ModelConfig) -> List[str]:
    names = ["attn_norm", "wq", "wk", "wv"]
    if cfg.qk_norm:
        names += ["q_norm", "k_norm"]
    names += ["wo", "mlp_norm", "w_gate", "w_up", "w_down"]
    return names


def weight_shape(cfg: ModelConfig, name: str):
    H, F = cfg.hidden, cfg.ffn
    return {
        "attn_norm": (H,), "mlp_norm": (H,),
        "q_norm": (cfg.head_dim,), "k_norm": (cfg.head_dim,),
        "wq": (cfg.q_rows, H), "wk": (cfg.kv_rows, H), "wv": (cfg.kv_rows, H),
        "wo": (H, cfg.q_rows), "w_gate": (F, H), "w_up": (F, H), "w_down": (H, F),
    }[name]


def make_weights(cfg: ModelConfig, seed: int = SEED_WEIGHTS, device="cpu") -> Dict:
    """BF16 weights as torch tensors on ``device``: ``embed`` [V, H],
    ``final_norm`` [H], optional ``lm_head`` (untied only) and ``layers``
    (list of dicts keyed by :func:`weight_names`)."""
    idx = 0
    out: Dict = {}
    out["embed"] = _normal((cfg.vocab, cfg.hidden), WEIGHT_STD, 0.0, device, _seed(seed, cfg, idx))
    idx += 1
    layers = []
    for _ in range(cfg.n_layers):
        d = {}
        for name in weight_names(cfg):
            shape = weight_shape(cfg, name)
            if name.endswith("norm"):
                d[name] = _normal(shape, GAIN_STD, 1.0, device, _seed(seed, cfg, idx))
            else:
                d[name] = _normal(shape, WEIGHT_STD, 0.0, device, _seed(seed, cfg, idx))
            idx += 1
        layers.append(d)
    out["layers"] = layers
    out["final_norm"] = _normal((cfg.hidden,), GAIN_STD, 1.0, device, _seed(seed, cfg, idx))
    idx += 1
    if not cfg.tie_embeddings:
        out["lm_head"] = _normal((cfg.vocab, cfg.hidden), WEIGHT_STD, 0.0, device, _seed(seed, cfg, idx))
    return out


def make_kv(cfg: ModelConfig, capacity: int, n_cached: int, seed: int = SEED_KV, key_scale: bool = False,
            device="cpu"):
    """BF16 K and V caches [n_layers, n_kv_heads, capacity, head_dim].

    Positions < ``n_cached`` ~ N(0, 1) (keys times a per-channel scale
    ~ U(0.5, 4) when ``key_scale``); later positions are zero."""
    shape = (cfg.n_layers, cfg.n_kv_heads, capacity, cfg.head_dim)
    k = torch.zeros(shape, dtype=torch.bfloat16, device=device)
    v = torch.zeros(shape, dtype=torch.bfloat16, device=device)
    if n_cached > 0:
        for l in range(cfg.n_layers):
            gk = _gen(device, _seed(seed, cfg, 2 * l))
            gv = _gen(device, _seed(seed, cfg, 2 * l + 1))
            kk = torch.empty((cfg.n_kv_heads, n_cached, cfg.head_dim), dtype=torch.float32, device=device)
            kk.normal_(0.0, 1.0, generator=gk)
            if key_scale:
                gs = _gen(device, _seed(SEED_KEY_SCALE, cfg, l))
                s = torch.empty((cfg.n_kv_heads, 1, cfg.head_dim), dtype=torch.float32, device=device)
                s.uniform_(0.5, 4.0, generator=gs)
                kk.mul_(s)
            k[l, :, :n_cached] = kk.to(torch.bfloat16)
            del kk
            vv = torch.empty((cfg.n_kv_heads, n_cached, cfg.head_dim), dtype=torch.float32, device=device)
            vv.normal_(0.0, 1.0, generator=gv)
            v[l, :, :n_cached] = vv.to(torch.bfloat16)
            del vv
    return k, v


def make_tokens(cfg: ModelConfig, n: int, seed: int = SEED_TOKENS) -> List[int]:
    """``n`` tokens ~ U[0, vocab) (CPU generator: identical on every machine)."""
    g = _gen("cpu", _seed(seed, cfg, 0))
    return [int(t) for t in torch.randint(0, cfg.vocab, (n,), generator=g)]


def make_uniforms(cfg: ModelConfig, n: int, seed: int = SEED_UNIFORMS) -> np.ndarray:
    """``n`` FP32 uniforms in [0, 1), one per sampled step (CPU generator: identical on every machine)."""
    g = _gen("cpu", _seed(seed, cfg, 0))
    u = torch.rand(n, generator=g, dtype=torch.float32).numpy()
    return np.minimum(u, np.float32(1.0) - np.float32(2.0 ** -24))  # strictly below 1


# --------------------------------------------------------------------------
# views for the CPU oracle (bit patterns, no arithmetic)
# --------------------------------------------------------------------------

def bits(t: torch.Tensor) -> np.ndarray:
    """The BF16 bit patterns of ``t`` as a host uint16 array."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def weights_as_bits(w: Dict) -> Dict:
    out = {"embed": bits(w["embed"]), "final_norm": bits(w["final_norm"]),
           "layers": [{k: bits(v) for k, v in d.items()} for d in w["layers"]]}
    if "lm_head" in w:
        out["lm_head"] = bits(w["lm_head"])
    return out
