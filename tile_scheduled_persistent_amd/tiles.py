"""Python binding of ``include/tiles.h`` (ctypes; argument marshalling only).

Every step of the decode runs in the HIP library; this module only converts
torch tensors to raw device pointers and back.  If ``libtiles.so`` is missing the
import of the library raises: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from .configs import ModelConfig

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtiles.so")

TILES_OK = 0
TILES_E_ARG = -1
TILES_E_CONFIG = -2
TILES_E_PLAN = -3
TILES_E_DEVICE = -4
TILES_E_HIP = -5
TILES_E_KERNEL = -6

TILES_DEBUG_HIDDEN = 0x1
TILES_TRACE = 0x2
TRACE_WORDS = 12  # see tiles_read_debug in include/tiles.h
TILES_POISON = 0x4

WAVE_KINDS = {1: "qkv", 2: "attn", 3: "combine", 4: "o_proj", 5: "gate_up", 6: "down", 7: "lm_head"}


class TilesError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"tiles error {code}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
        ("vocab", ctypes.c_int32), ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
        ("qk_norm", ctypes.c_int32), ("tie_embeddings", ctypes.c_int32), ("max_positions", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("kv_splits", ctypes.c_int32), ("combine_mode", ctypes.c_int32),
        ("attn_heads", ctypes.c_int32), ("n_workers", ctypes.c_int32), ("stream", ctypes.c_void_p),
        ("o_placement", ctypes.c_int32), ("weight_format", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("temperature", ctypes.c_float), ("top_p", ctypes.c_float),
        ("kv_format", ctypes.c_int32), ("tokens_per_step", ctypes.c_int32),
    ]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ["attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "mlp_norm", "w_gate", "w_up", "w_down"]]


class Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("layers", ctypes.POINTER(LayerWeights)), ("on_device", ctypes.c_int32)]


class KV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("capacity", ctypes.c_int64),
                ("length", ctypes.c_int64), ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("k_smooth", ctypes.c_void_p)]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("n_workers", ctypes.c_int32), ("block_threads", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
        ("waves_per_step", ctypes.c_int32), ("n_tiles", ctypes.c_int32), ("kv_splits", ctypes.c_int32),
        ("combine_mode", ctypes.c_int32), ("occupancy", ctypes.c_int32), ("packed_bytes", ctypes.c_int64),
        ("weight_bytes_per_step", ctypes.c_int64), ("max_over_mean", ctypes.c_double),
        ("checksum", ctypes.c_uint64), ("build_id", ctypes.c_uint64), ("attn_heads", ctypes.c_int32),
        ("o_workers", ctypes.c_int32), ("weight_format", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("kv_format", ctypes.c_int32), ("tokens_per_step", ctypes.c_int32), ("stage_batches", ctypes.c_int32),
    ]


class WaveInfo(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("layer", ctypes.c_int32), ("busy_workers", ctypes.c_int32),
                ("pad", ctypes.c_int32), ("weight_bytes", ctypes.c_int64), ("max_worker_bytes", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded ``libtiles.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m tile_scheduled_persistent_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.tiles_plan_create.restype = ctypes.c_void_p
        L.tiles_plan_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights)]
        L.tiles_decode.restype = ctypes.c_int
        L.tiles_decode.argtypes = [ctypes.c_void_p, ctypes.POINTER(KV), ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p]
        L.tiles_decode_noalloc.restype = ctypes.c_int
        L.tiles_decode_noalloc.argtypes = [ctypes.c_void_p, ctypes.POINTER(KV), ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_void_p]
        L.tiles_kv_convert_int8.restype = ctypes.c_int
        L.tiles_kv_convert_int8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.POINTER(KV)]
        L.tiles_decode_sampled.restype = ctypes.c_int
        L.tiles_decode_sampled.argtypes = [ctypes.c_void_p, ctypes.POINTER(KV), ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.tiles_verify.restype = ctypes.c_int
        L.tiles_verify.argtypes = [ctypes.c_void_p, ctypes.POINTER(KV), ctypes.c_void_p, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p]
        L.tiles_plan_destroy.restype = None
        L.tiles_plan_destroy.argtypes = [ctypes.c_void_p]
        L.tiles_last_error.restype = ctypes.c_char_p
        L.tiles_last_error.argtypes = []
        L.tiles_plan_info.restype = ctypes.c_int
        L.tiles_plan_info.argtypes = [ctypes.c_void_p, ctypes.POINTER(PlanInfo)]
        L.tiles_plan_wave.restype = ctypes.c_int
        L.tiles_plan_wave.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(WaveInfo)]
        L.tiles_plan_debug_validate.restype = ctypes.c_int
        L.tiles_plan_debug_validate.argtypes = [ctypes.POINTER(Config), ctypes.c_int32, ctypes.c_int32]
        L.tiles_plan_dry_run.restype = ctypes.c_int
        L.tiles_plan_dry_run.argtypes = [ctypes.POINTER(Config), ctypes.c_int32, ctypes.POINTER(PlanInfo)]
        L.tiles_plan_set_stream.restype = ctypes.c_int
        L.tiles_plan_set_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.tiles_plan_status.restype = ctypes.c_int
        L.tiles_plan_status.argtypes = [ctypes.c_void_p]
        L.tiles_read_debug.restype = ctypes.c_int
        L.tiles_read_debug.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.POINTER(ctypes.c_int32)]
        L.tiles_plan_debug_corrupt.restype = ctypes.c_int
        L.tiles_plan_debug_corrupt.argtypes = [ctypes.c_void_p]
        L.tiles_plan_debug_corrupt_device.restype = ctypes.c_int
        L.tiles_plan_debug_corrupt_device.argtypes = [ctypes.c_void_p]
        L.tiles_plan_debug_spin_limit.restype = ctypes.c_int
        L.tiles_plan_debug_spin_limit.argtypes = [ctypes.c_void_p, ctypes.c_uint32]
        L.tiles_quantize_rows_int8.restype = ctypes.c_int
        L.tiles_quantize_rows_int8.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                               ctypes.c_void_p]
        L.tiles_stream_read.restype = ctypes.c_int
        L.tiles_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p]
        L.tiles_edge_latency.restype = ctypes.c_int
        L.tiles_edge_latency.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32,
                                         ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def last_error() -> str:
    return lib().tiles_last_error().decode()


def _check(rc: int):
    if rc != TILES_OK:
        raise TilesError(rc, last_error())


WEIGHTS = {"bf16": 0, "int8": 1}
KV_FORMATS = {"bf16": 0, "int8": 1}


def make_config(m: ModelConfig, max_positions: int, flags: int = 0, kv_splits: int = 0, combine_mode: int = 0,
                n_workers: int = 0, stream: Optional[int] = None, attn_heads: int = 0, o_placement: int = 0,
                weights: str = "bf16", sampling: Optional[tuple] = None, kv: str = "bf16",
                tokens_per_step: int = 0) -> Config:
    """``sampling`` = (temperature, top_k, top_p) makes a sampling plan (tiles_decode_sampled);
    ``kv`` = "int8" an INT8 KV plan (see KVCache.int8); ``tokens_per_step`` = 2 .. 4 a verify plan
    (tiles_verify only) whose steps take that many positions through every tile at once."""
    temperature, top_k, top_p = sampling if sampling is not None else (1.0, 0, 1.0)
    return Config(m.n_layers, m.hidden, m.n_heads, m.n_kv_heads, m.head_dim, m.ffn, m.vocab, float(m.rope_theta),
                  float(m.rms_eps), int(m.qk_norm), int(m.tie_embeddings), int(max_positions), int(flags),
                  int(kv_splits), int(combine_mode), int(attn_heads), int(n_workers), stream, int(o_placement),
                  WEIGHTS[weights], int(top_k), float(temperature), float(top_p), KV_FORMATS[kv],
                  int(tokens_per_step))


def dry_run(m: ModelConfig, max_positions: int, n_workers: int = 256, **kw) -> PlanInfo:
    """Plan on the host only (no GPU); raises TilesError if planning/validation fails."""
    info = PlanInfo()
    cfg = make_config(m, max_positions, **kw)
    _check(lib().tiles_plan_dry_run(ctypes.byref(cfg), n_workers, ctypes.byref(info)))
    return info


def debug_validate(m: ModelConfig, max_positions: int, mutation: int, n_workers: int = 256, **kw) -> int:
    """Plan on the host, plant mistake number `mutation` (tiles_plan_debug_validate) and return the
    validator's status code (the message is in last_error())."""
    cfg = make_config(m, max_positions, **kw)
    return lib().tiles_plan_debug_validate(ctypes.byref(cfg), n_workers, mutation)


def quantize_rows_int8(bf16_bits: np.ndarray):
    """The library's weight-only INT8 quantizer (tiles_quantize_rows_int8, host only) on a uint16
    [rows, cols] array of BF16 bit patterns: (int8 codes [rows, cols], float32 scales [rows])."""
    w = np.ascontiguousarray(np.atleast_2d(bf16_bits), dtype=np.uint16)
    q = np.zeros(w.shape, dtype=np.int8)
    s = np.zeros(w.shape[0], dtype=np.float32)
    _check(lib().tiles_quantize_rows_int8(w.ctypes.data, w.shape[0], w.shape[1], q.ctypes.data, s.ctypes.data))
    return q, s


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def stream_read(buf: torch.Tensor, n_groups: int, sink: torch.Tensor, stream=None) -> None:
    """Launch the stream-read ceiling kernel over the bytes of a device tensor (tiles_stream_read):
    XORs every word into sink (an int32/uint32 device tensor of one element).  Asynchronous."""
    s = stream if stream is not None else torch.cuda.current_stream()
    _check(lib().tiles_stream_read(ctypes.c_void_p(_ptr(buf)), buf.numel() * buf.element_size(), n_groups,
                                   ctypes.c_void_p(_ptr(sink)), ctypes.c_void_p(s.cuda_stream)))


def edge_latency(words: torch.Tensor, peer: int, iters: int, out: torch.Tensor, spin_limit: int = 1 << 22,
                 stream=None) -> None:
    """Launch the edge-latency ping-pong (tiles_edge_latency): words is a zeroed int32 device tensor
    of at least 17 elements, out an int64 device tensor of 3 (ticks, peer gave up, workgroup 0
    gave up).  Asynchronous."""
    if words.numel() * words.element_size() < 17 * 4 or out.numel() * out.element_size() < 3 * 8:
        raise TilesError(TILES_E_ARG, "words needs 17 int32, out 3 int64")
    s = stream if stream is not None else torch.cuda.current_stream()
    _check(lib().tiles_edge_latency(ctypes.c_void_p(_ptr(words)), peer, iters, spin_limit, ctypes.c_void_p(_ptr(out)),
                                    ctypes.c_void_p(s.cuda_stream)))


@dataclass
class KVCache:
    """Caller-owned cache (device): BF16 k, v [n_layers, n_kv_heads, capacity, head_dim]; or, for an
    INT8 KV plan, k the interleaved int8 codes [n_layers, n_kv_heads, capacity, 2 * head_dim] (v None),
    k_scale, v_scale float32 [n_layers, n_kv_heads, capacity] and k_smooth float32 [n_layers,
    n_kv_heads, head_dim] (see tiles_kv_convert_int8 in include/tiles.h)."""
    k: torch.Tensor
    v: Optional[torch.Tensor]
    length: int = 0
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None
    k_smooth: Optional[torch.Tensor] = None

    @property
    def capacity(self) -> int:
        return self.k.shape[2]

    @property
    def int8(self) -> bool:
        return self.k.dtype == torch.int8

    def struct(self) -> "KV":
        return KV(_ptr(self.k), _ptr(self.v), self.capacity, self.length, _ptr(self.k_scale), _ptr(self.v_scale),
                  _ptr(self.k_smooth))

    def clone(self) -> "KVCache":
        c = lambda t: None if t is None else t.clone()
        return KVCache(c(self.k), c(self.v), self.length, c(self.k_scale), c(self.v_scale), c(self.k_smooth))

    @staticmethod
    def convert_int8(plan: "Plan", k_bf16: torch.Tensor, v_bf16: torch.Tensor, length: int) -> "KVCache":
        """The INT8 cache of an INT8 KV plan from the first ``length`` positions of a BF16 cache
        (tiles_kv_convert_int8, on the plan's stream; smoothing factors from those positions)."""
        L, H, cap, hd = k_bf16.shape
        dev = k_bf16.device
        out = KVCache(torch.zeros((L, H, cap, 2 * hd), dtype=torch.int8, device=dev), None, 0,
                      torch.zeros((L, H, cap), dtype=torch.float32, device=dev),
                      torch.zeros((L, H, cap), dtype=torch.float32, device=dev),
                      torch.zeros((L, H, hd), dtype=torch.float32, device=dev))
        c = out.struct()
        _check(lib().tiles_kv_convert_int8(plan._h, _ptr(k_bf16.contiguous()), _ptr(v_bf16.contiguous()), cap, length,
                                           ctypes.byref(c)))
        out.length = c.length
        return out


class Plan:
    """A tile plan for one model on the current device (owns a packed copy of the weights)."""

    def __init__(self, m: ModelConfig, weights: Dict, max_positions: int, flags: int = 0, kv_splits: int = 0,
                 combine_mode: int = 0, stream: Optional[torch.cuda.Stream] = None, attn_heads: int = 0,
                 o_placement: int = 0, weight_format: str = "bf16", sampling: Optional[tuple] = None,
                 kv_format: str = "bf16", tokens_per_step: int = 0):
        self.model = m
        self.sampling = sampling
        self.kv_format = kv_format
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self._cfg = make_config(m, max_positions, flags, kv_splits, combine_mode, 0, self.stream.cuda_stream,
                                attn_heads, o_placement, weight_format, sampling, kv_format, tokens_per_step)
        on_device = weights["embed"].is_cuda
        layers = (LayerWeights * m.n_layers)()
        for i, d in enumerate(weights["layers"]):
            for name, _ in LayerWeights._fields_:
                t = d.get(name)
                if t is not None:
                    if t.dtype != torch.bfloat16 or t.is_cuda != on_device:
                        raise ValueError(f"layer {i} {name}: expected bf16 on the same device as embed")
                    setattr(layers[i], name, _ptr(t))
        w = Weights(_ptr(weights["embed"]), _ptr(weights["final_norm"]), _ptr(weights.get("lm_head")), layers,
                    1 if on_device else 0)
        self._weights_struct = (w, layers)
        h = lib().tiles_plan_create(ctypes.byref(self._cfg), ctypes.byref(w))
        if not h:
            raise TilesError(-99, last_error())
        self._h = h
        self._weights_struct = None

    def close(self):
        if getattr(self, "_h", None):
            lib().tiles_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # ------------------------------------------------------------------
    def decode(self, kv: KVCache, token: int, n_steps: int, out_tokens: torch.Tensor,
               out_logits: Optional[torch.Tensor] = None, noalloc: bool = False,
               uniforms: Optional[torch.Tensor] = None) -> int:
        """Enqueue one cooperative launch of ``n_steps`` steps; returns TILES_OK or raises.
        Greedy plans call tiles_decode (``noalloc``: tiles_decode_noalloc, scratch in the library's
        static device array); sampling plans call tiles_decode_sampled with ``uniforms`` (a device
        float32 tensor of n_steps values in [0, 1))."""
        if uniforms is not None and (uniforms.dtype != torch.float32 or not uniforms.is_cuda
                                     or uniforms.numel() < n_steps):
            raise ValueError("uniforms must be a device float32 tensor with n_steps entries")
        if out_tokens.dtype != torch.int32 or not out_tokens.is_cuda or out_tokens.numel() < n_steps:
            raise ValueError("out_tokens must be a device int32 tensor with n_steps entries")
        if out_logits is not None and (out_logits.dtype != torch.float32 or not out_logits.is_cuda
                                       or out_logits.numel() < n_steps * self.model.vocab):
            raise ValueError("out_logits must be a device float32 tensor [n_steps, vocab]")
        if kv.int8:
            for t in (kv.k, kv.k_scale, kv.v_scale, kv.k_smooth):
                if t is None or not t.is_cuda or not t.is_contiguous():
                    raise ValueError("INT8 KV tensors must be contiguous device tensors")
        else:
            for t in (kv.k, kv.v):
                if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
                    raise ValueError("KV tensors must be contiguous device bf16")
        c = kv.struct()
        if uniforms is not None or self.sampling is not None:
            rc = lib().tiles_decode_sampled(self._h, ctypes.byref(c), int(token), int(n_steps), _ptr(uniforms),
                                            _ptr(out_tokens), _ptr(out_logits))
        else:
            fn = lib().tiles_decode_noalloc if noalloc else lib().tiles_decode
            rc = fn(self._h, ctypes.byref(c), int(token), int(n_steps), _ptr(out_tokens), _ptr(out_logits))
        _check(rc)
        kv.length = c.length
        return rc

    def verify(self, kv: KVCache, tokens: Sequence[int], out_argmax: Optional[torch.Tensor] = None,
               out_logits: Optional[torch.Tensor] = None):
        """A greedy verify step (tiles_verify): ``tokens`` = [last accepted token, draft 1, ...]
        (a verify plan: a multiple of its tokens_per_step).  Synchronizes the device and returns
        (argmax int64 [m], accepted count n, verified tokens [n + 1]: the accepted drafts, then the
        argmax after them); kv.length becomes its value before the call + n + 1."""
        tokens = [int(t) for t in tokens]
        m = len(tokens)
        if out_argmax is None:
            out_argmax = torch.empty(m, dtype=torch.int32, device="cuda")
        if out_argmax.dtype != torch.int32 or not out_argmax.is_cuda or out_argmax.numel() < m:
            raise ValueError("out_argmax must be a device int32 tensor with m entries")
        if out_logits is not None and (out_logits.dtype != torch.float32 or not out_logits.is_cuda
                                       or out_logits.numel() < m * self.model.vocab):
            raise ValueError("out_logits must be a device float32 tensor [m, vocab]")
        length0 = kv.length
        c = kv.struct()
        buf = (ctypes.c_int32 * max(m, 1))(*tokens)
        _check(lib().tiles_verify(self._h, ctypes.byref(c), buf, m, _ptr(out_argmax), _ptr(out_logits)))
        torch.cuda.synchronize()
        st = self.status()
        if st != TILES_OK:
            raise RuntimeError(f"tiles_verify: launch status {st}: {last_error()}")
        a = out_argmax[:m].cpu().numpy().astype(np.int64)
        n = 0
        while n < m - 1 and int(a[n]) == tokens[n + 1]:
            n += 1
        kv.length = length0 + n + 1
        return a, n, np.array(tokens[1:n + 1] + [int(a[n])], dtype=np.int64)

    def status(self) -> int:
        return lib().tiles_plan_status(self._h)

    def info(self) -> PlanInfo:
        info = PlanInfo()
        _check(lib().tiles_plan_info(self._h, ctypes.byref(info)))
        return info

    def waves(self) -> List[WaveInfo]:
        out = []
        for i in range(self.info().waves_per_step):
            wi = WaveInfo()
            _check(lib().tiles_plan_wave(self._h, i, ctypes.byref(wi)))
            out.append(wi)
        return out

    def read_debug(self, hidden: bool = True, trace: bool = False):
        """(hidden [n_steps, n_layers, H] float32 or None, trace [kernel steps, waves, W, TRACE_WORDS] uint64 or
        None; a verify plan's kernel step runs tokens_per_step positions)."""
        info = self.info()
        n = ctypes.c_int32(0)
        _check(lib().tiles_read_debug(self._h, None, None, ctypes.byref(n)))
        hid = tr = None
        hp = tp = None
        if hidden:
            hid = np.zeros((n.value, self.model.n_layers, self.model.hidden), dtype=np.float32)
            hp = hid.ctypes.data
        if trace:
            tr = np.zeros((n.value // info.tokens_per_step, info.waves_per_step, info.n_workers, TRACE_WORDS),
                          dtype=np.uint64)
            tp = tr.ctypes.data
        _check(lib().tiles_read_debug(self._h, hp, tp, None))
        return hid, tr

    def set_stream(self, stream: torch.cuda.Stream):
        self.stream = stream
        _check(lib().tiles_plan_set_stream(self._h, stream.cuda_stream))

    def debug_corrupt(self):
        _check(lib().tiles_plan_debug_corrupt(self._h))

    def debug_corrupt_device(self):
        """Flip one bit of the device copy of the schedule (the next launch must detect it)."""
        _check(lib().tiles_plan_debug_corrupt_device(self._h))

    def debug_spin_limit(self, rounds: int):
        """Watchdog of every wait in later decodes (0 restores the default)."""
        _check(lib().tiles_plan_debug_spin_limit(self._h, int(rounds)))
