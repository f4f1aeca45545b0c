"""Model shapes and decode workloads.

The shapes are the decoders the pages run: Llama 3.2 1B (Tiles page, intro:
"Llama 3.2 1B in BF16 at batch size one"), Qwen3-0.6B and Qwen3-4B
(TileInfer.jl roadmap, "Where it stands" table: decode "after 1,023 cached
positions"), plus a tiny decoder that a CPU oracle finishes in well under a
second and a long-context Qwen3-4B workload whose attention carries a large
share of the bytes (the roadmap's "M8 so far" table measures 4B decode at 32k
positions).  Weights are random (no checkpoints are used); see ``synth``.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rope_theta: float
    rms_eps: float
    qk_norm: bool
    tie_embeddings: bool = True

    @property
    def q_rows(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_rows(self) -> int:
        return self.n_kv_heads * self.head_dim

    def param_count(self) -> int:
        """Parameters read once per token: every linear layer, every norm
        gain, the LM head (the embedding matrix when tied) and one embedding
        row."""
        H, F, V = self.hidden, self.ffn, self.vocab
        per_layer = (H * (self.q_rows + 2 * self.kv_rows) + self.q_rows * H + 3 * H * F + 2 * H)
        if self.qk_norm:
            per_layer += 2 * self.head_dim
        head = V * H
        return self.n_layers * per_layer + H + head + H  # final norm, LM head, one embedding row

    def weight_bytes_per_token(self) -> int:
        return 2 * self.param_count()

    def linear_rows(self) -> int:
        """Output rows of every linear layer (the LM head included): one INT8 scale each."""
        return self.n_layers * (self.q_rows + 2 * self.kv_rows + self.hidden + 2 * self.ffn + self.hidden) + self.vocab

    def int8_weight_bytes_per_token(self) -> int:
        """Weight-only INT8: one byte per linear weight, one FP32 scale per linear row, and the BF16
        norm gains and embedding row."""
        H, F, V = self.hidden, self.ffn, self.vocab
        linear = self.n_layers * (H * (self.q_rows + 2 * self.kv_rows) + self.q_rows * H + 3 * H * F) + V * H
        gains = self.n_layers * (2 * H + (2 * self.head_dim if self.qk_norm else 0)) + H
        return linear + 4 * self.linear_rows() + 2 * gains + 2 * H

    def kv_bytes_per_position(self) -> int:
        """K and V bytes of one position over all layers (BF16)."""
        return 2 * 2 * self.n_layers * self.n_kv_heads * self.head_dim

    def int8_kv_bytes_per_position(self) -> int:
        """INT8 KV cache: K and V codes (one byte per element) and their two FP32 scales, all layers."""
        return self.n_layers * self.n_kv_heads * (2 * self.head_dim + 8)


@dataclass(frozen=True)
class Workload:
    """A decode run: ``n_cached`` positions already in the KV cache, then
    ``n_steps`` greedy steps (one launch of up to 64 steps each)."""
    key: str
    model: ModelConfig
    n_cached: int
    n_steps: int
    prompt_len: int = 0          # >0: prefill that many prompt tokens one step at a time
    key_scale: bool = False      # per-(layer, kv head, channel) key scales ~ U(0.5, 4)
    description: str = ""
    weights: str = "bf16"        # "int8": weight-only INT8 linear layers (per-row codes and scales)
    sampling: Optional[tuple] = None  # (temperature, top_k, top_p): sampled steps instead of greedy
    kv: str = "bf16"             # "int8": INT8 KV cache with smoothed keys

    @property
    def capacity(self) -> int:
        return self.n_cached + self.prompt_len + self.n_steps

    def avg_attended(self) -> float:
        """Mean attended positions L over the timed steps (L = cached + 1 at
        the first step)."""
        return self.n_cached + (self.n_steps + 1) / 2.0

    def bytes_per_token(self) -> float:
        """Algorithmic HBM bytes per decoded token: weights read once, K/V of
        every attended position read once, one K/V position written."""
        m = self.model
        wb = m.int8_weight_bytes_per_token() if self.weights == "int8" else m.weight_bytes_per_token()
        kvp = m.int8_kv_bytes_per_position() if self.kv == "int8" else m.kv_bytes_per_position()
        return wb + kvp * self.avg_attended() + kvp


TINY = ModelConfig("tiny", 2, 256, 4, 2, 64, 1024, 4096, 1e4, 1e-5, False)
LLAMA_1B = ModelConfig("llama-3.2-1b-shaped", 16, 2048, 32, 8, 64, 8192, 128256, 5e5, 1e-5, False)
QWEN3_06B = ModelConfig("qwen3-0.6b-shaped", 28, 1024, 16, 8, 128, 3072, 151936, 1e6, 1e-6, True)
QWEN3_4B = ModelConfig("qwen3-4b-shaped", 36, 2560, 32, 8, 128, 9728, 151936, 1e6, 1e-6, True)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", TINY, 0, 15, prompt_len=8,
                     description="tiny decoder: 8-token prompt prefilled one token per step, "
                                 "then 16 greedy tokens (23 forward steps)"),
    "llama1b": Workload("llama1b", LLAMA_1B, 1023, 64,
                        description="Llama-3.2-1B-shaped decode, 64 tokens after 1023 cached positions"),
    "qwen06b": Workload("qwen06b", QWEN3_06B, 1023, 64,
                        description="Qwen3-0.6B-shaped decode, 64 tokens after 1023 cached positions"),
    "qwen4b": Workload("qwen4b", QWEN3_4B, 1023, 64,
                       description="Qwen3-4B-shaped decode, 64 tokens after 1023 cached positions"),
    "qwen4b_32k": Workload("qwen4b_32k", QWEN3_4B, 32767, 32, key_scale=True,
                           description="Qwen3-4B-shaped decode, 32 tokens after 32767 cached positions, "
                                       "per-channel key scales"),
    # weight-only INT8 linear layers (the roadmap page's "M8 so far" row), same shapes and inputs
    "llama1b_sampled": Workload("llama1b_sampled", LLAMA_1B, 1023, 64, sampling=(0.6, 20, 0.95),
                                description="Llama-3.2-1B-shaped decode with top-k/top-p sampling inside the launch "
                                            "(temperature 0.6, top-k 20, top-p 0.95), 64 tokens after 1023 cached "
                                            "positions"),
    "llama1b_kv8": Workload("llama1b_kv8", LLAMA_1B, 1023, 64, kv="int8",
                            description="Llama-3.2-1B-shaped decode with an INT8 KV cache (smoothed keys), "
                                        "64 tokens after 1023 cached positions"),
    "qwen4b_32k_kv8": Workload("qwen4b_32k_kv8", QWEN3_4B, 32767, 32, key_scale=True, kv="int8",
                               description="Qwen3-4B-shaped decode with an INT8 KV cache (smoothed keys), 32 tokens "
                                           "after 32767 cached positions, cached keys with per-channel scales "
                                           "U(0.5, 4)"),
    "llama1b_int8": Workload("llama1b_int8", LLAMA_1B, 1023, 64, weights="int8",
                             description="Llama-3.2-1B-shaped decode with weight-only INT8 linear layers, "
                                         "64 tokens after 1023 cached positions"),
    "qwen06b_int8": Workload("qwen06b_int8", QWEN3_06B, 1023, 64, weights="int8",
                             description="Qwen3-0.6B-shaped decode with weight-only INT8 linear layers, "
                                         "64 tokens after 1023 cached positions"),
    "qwen4b_int8": Workload("qwen4b_int8", QWEN3_4B, 1023, 64, weights="int8",
                            description="Qwen3-4B-shaped decode with weight-only INT8 linear layers, "
                                        "64 tokens after 1023 cached positions"),
}


def scaled(cfg: ModelConfig, **kw) -> ModelConfig:
    """A copy of ``cfg`` with some fields replaced (e.g. fewer layers)."""
    return replace(cfg, **kw)
