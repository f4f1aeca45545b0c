"""CPU oracle for batch-1 greedy BF16 decoding of a Llama/Qwen3-style decoder.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
anything from this package.  The GPU library never calls it, and it shares no
code with the GPU library (no kernels, headers, helpers, tables or constants):
it is a plain, slow, obviously correct restatement of what one decode step
computes, written from the pages' description of the workload:

* Tiles page ("Tiles: Scheduling LLM Decoding as a Graph of Tiles"), intro:
  Llama 3.2 1B in BF16 at batch size one, one stream of tokens; "What the code
  contains": a CPU reference with greedy selection; "Scope and code release":
  greedy decoding, BF16 weights, prefill one token per step.
* TileInfer.jl roadmap ("History and roadmap"), "M8 so far" table: the decode
  step is norm, RoPE, KV write, attention, residual add, RMSNorm and SwiGLU,
  with per-head q/k norm for Qwen3; "Milestones" M5: split-KV decode attention
  (which the oracle does NOT split: it is the unsplit softmax definition).

Arithmetic: FP32 activations and FP32 accumulation over BF16-rounded weights
(or, with ``weight_format="int8"``, the weights of every linear layer dequantized
from per-row INT8 codes) and a BF16 KV cache (``dtype=np.float64`` switches every activation to FP64
for pinning).  Every reading of a point the pages leave open is listed in the
module docstring of :mod:`oracle.decoder`.
"""

from .decoder import (  # noqa: F401
    bf16_round,
    bf16_bits_to_float,
    float_to_bf16_bits,
    quantize_rows_int8,
    dequantize_rows_int8,
    sample_token,
    quantize_rows_f32_int8,
    convert_kv_int8,
    dequantize_kv_rows,
    LINEAR_WEIGHTS,
    rmsnorm,
    rope_cos_sin,
    apply_rope,
    attend,
    silu,
    OracleModel,
)
