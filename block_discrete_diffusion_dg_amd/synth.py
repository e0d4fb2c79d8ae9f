"""Seeded synthetic inputs: model shapes, random-init weights, token ids.

This module is the only code shared by the CPU oracle and the HIP path. It
holds shapes and random-number generation, and none of the denoising step's
arithmetic.

Weights are drawn from a counter-based integer hash so that the same tensor
comes out bit-identical on the CPU and on the GPU (the generator runs on
whatever device the caller names, with integer torch ops plus one IEEE fp32
multiply). Each element is an Irwin-Hall sum of four 22-bit uniforms, scaled
to the requested standard deviation and rounded to bfloat16 (round to
nearest even). The sum of four uniforms stands in for the normal
distribution the workloads ask for: same mean and variance, support bounded
at about 3.46 standard deviations.

Shapes follow the model the pages describe (codemajin.net DiffusionGemma
explainer, §2.1: MoE with 128 experts, 8 routed plus 1 shared per token;
§3.2: 256-token canvas, block-autoregressive KV cache).
"""
from __future__ import annotations

import dataclasses
import math
import zlib
from typing import Dict, Optional

import torch

_M32 = 0xFFFFFFFF
_MIX = 0x45D9F3B  # odd multiplier below 2**31: products of 32-bit values fit int64


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    """Shape and fixed hyper-parameters of the MoE transformer."""

    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    d_expert: int
    d_shared: int
    vocab: int
    canvas: int = 256
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    tau_first: float = 0.8
    tau_last: float = 0.4
    weight_std: float = 0.02

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


@dataclasses.dataclass(frozen=True)
class Workload:
    """One measured or tested configuration: model plus loop shape."""

    name: str
    model: ModelConfig
    prefix: int
    n_steps: int
    n_blocks: int = 1
    n_req: int = 1
    seed: int = 0

    @property
    def max_ctx(self) -> int:
        return self.prefix + (self.n_blocks + 1) * self.model.canvas


TINY = ModelConfig("tiny", n_layers=1, d_model=256, n_q_heads=4, n_kv_heads=2,
                   head_dim=64, n_experts=8, top_k=2, d_expert=512, d_shared=512,
                   vocab=4096, canvas=32)
FULL = ModelConfig("full", n_layers=30, d_model=2048, n_q_heads=16, n_kv_heads=8,
                   head_dim=128, n_experts=128, top_k=8, d_expert=704, d_shared=2048,
                   vocab=262144, canvas=256)
ONE_LAYER = dataclasses.replace(FULL, name="one_layer", n_layers=1)

WORKLOADS: Dict[str, Workload] = {
    # 1: tiny CPU-checkable step
    "tiny": Workload("tiny", TINY, prefix=64, n_steps=4),
    # 2: one full-width layer, random prefix KV, random hidden states
    "one_layer": Workload("one_layer", ONE_LAYER, prefix=2048, n_steps=1),
    # 3: full 30-layer stack plus LM head over 262,144 ids
    "full": Workload("full", FULL, prefix=2048, n_steps=16),
    # 4: long prefix, four consecutive blocks
    "long": Workload("long", FULL, prefix=32768, n_steps=12, n_blocks=4),
    # 5: eight independent requests batched into one step
    "batch": Workload("batch", FULL, prefix=4096, n_steps=16, n_req=8),
}


# --------------------------------------------------------------------------
# counter-based hash generator (integer torch ops: identical bits on any device)
# --------------------------------------------------------------------------

def tensor_seed(model_seed: int, layer: int, name: str) -> int:
    """Stable 32-bit stream id for one named tensor."""
    return zlib.crc32(f"dg/{model_seed}/{layer}/{name}".encode()) & _M32


def _mix32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = (x * _MIX) & _M32
    x = x ^ (x >> 16)
    x = (x * _MIX) & _M32
    x = x ^ (x >> 16)
    return x


def _hash_words(start: int, n: int, seed32: int, lane: int, device) -> torch.Tensor:
    """32-bit hash of element counters start..start+n-1, sub-stream `lane`."""
    idx = torch.arange(start, start + n, dtype=torch.int64, device=device)
    x = ((idx * 4 + lane) & _M32) ^ seed32
    x = _mix32(x)
    seed_b = ((seed32 * 2654435761) & _M32) >> 1
    return _mix32(x ^ seed_b)


def _f32_to_bf16_bits(f: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16 round-to-nearest-even, in integer ops (finite inputs)."""
    b = f.view(torch.int32).to(torch.int64) & _M32
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) & 0xFFFF
    r = torch.where(r >= 0x8000, r - 0x10000, r)
    return r.to(torch.int16)


def hashed_normal(shape, seed32: int, std: float, device="cpu",
                  dtype=torch.bfloat16, chunk: int = 1 << 24) -> torch.Tensor:
    """Irwin-Hall(4) approximately-normal values, mean 0, standard deviation std.

    Returned as bfloat16 (RNE-rounded) or as float32 holding those bf16 values.
    """
    numel = 1
    for s in shape:
        numel *= int(s)
    out16 = torch.empty(numel, dtype=torch.int16, device=device)
    half_range = 2 * ((1 << 22) - 1)
    scale = torch.tensor(std * math.sqrt(3.0) / float(1 << 22), dtype=torch.float32,
                         device=device)
    for start in range(0, numel, chunk):
        n = min(chunk, numel - start)
        acc = torch.zeros(n, dtype=torch.int64, device=device)
        for lane in range(4):
            acc += _hash_words(start, n, seed32, lane, device) >> 10
        f = (acc - half_range).to(torch.float32) * scale
        out16[start:start + n] = _f32_to_bf16_bits(f)
    out = out16.view(torch.bfloat16).reshape(tuple(int(s) for s in shape))
    if dtype == torch.bfloat16:
        return out
    return out.to(dtype)


def hashed_uniform_ids(n: int, seed32: int, vocab: int, device="cpu") -> torch.Tensor:
    """n token ids uniform over [0, vocab) (int32)."""
    h = _hash_words(0, n, seed32, 0, device)
    return ((h * vocab) >> 32).to(torch.int32)


def norm_gain(n: int, seed32: int, jitter: float, device="cpu") -> torch.Tensor:
    """RMSNorm gain vector: ones, or 1 + jitter * (approximately normal), in bf16."""
    if jitter == 0.0:
        return torch.ones(n, dtype=torch.bfloat16, device=device)
    g = hashed_normal((n,), seed32, 1.0, device=device, dtype=torch.float32)
    f = (1.0 + jitter * g).to(torch.float32)
    return _f32_to_bf16_bits(f).view(torch.bfloat16)


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------

LAYER_TENSORS = ("attn_norm", "w_qkv", "w_o", "moe_norm", "w_router",
                 "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")


def layer_shapes(cfg: ModelConfig) -> Dict[str, tuple]:
    d, E, F, Fs = cfg.d_model, cfg.n_experts, cfg.d_expert, cfg.d_shared
    return {
        "attn_norm": (d,),
        "w_qkv": (cfg.qkv_rows, d),
        "w_o": (d, cfg.n_q_heads * cfg.head_dim),
        "moe_norm": (d,),
        "w_router": (E, d),
        "w_gate": (E, F, d),
        "w_up": (E, F, d),
        "w_down": (E, d, F),
        "ws_gate": (Fs, d),
        "ws_up": (Fs, d),
        "ws_down": (d, Fs),
    }


def make_layer_weights(cfg: ModelConfig, layer: int, model_seed: int = 0,
                       device="cpu", gain_jitter: float = 0.0) -> Dict[str, torch.Tensor]:
    """All bf16 tensors of one layer, in the [out][in] layout (y = x W^T)."""
    out = {}
    for name, shape in layer_shapes(cfg).items():
        s = tensor_seed(model_seed, layer, name)
        if name.endswith("norm"):
            out[name] = norm_gain(shape[0], s, gain_jitter, device)
        else:
            out[name] = hashed_normal(shape, s, cfg.weight_std, device)
    return out


def make_embedding(cfg: ModelConfig, model_seed: int = 0, device="cpu") -> torch.Tensor:
    """[vocab][d_model] bf16; also the (tied) LM head."""
    return hashed_normal((cfg.vocab, cfg.d_model), tensor_seed(model_seed, -1, "embed"),
                         cfg.weight_std, device)


SELFCOND_TENSORS = ("sc_gate", "sc_up", "sc_down")


def selfcond_shapes(cfg: ModelConfig, width: int) -> Dict[str, tuple]:
    """The self-conditioning feed-forward layer: a SwiGLU block d -> width -> d."""
    d = cfg.d_model
    return {"sc_gate": (width, d), "sc_up": (width, d), "sc_down": (d, width)}


def make_selfcond_weights(cfg: ModelConfig, width: int, model_seed: int = 0,
                          device="cpu") -> Dict[str, torch.Tensor]:
    """bf16 weights of the self-conditioning feed-forward layer ([out][in])."""
    return {name: hashed_normal(shape, tensor_seed(model_seed, -2, name), cfg.weight_std, device)
            for name, shape in selfcond_shapes(cfg, width).items()}


def make_final_norm(cfg: ModelConfig, model_seed: int = 0, device="cpu",
                    gain_jitter: float = 0.0) -> torch.Tensor:
    return norm_gain(cfg.d_model, tensor_seed(model_seed, -1, "final_norm"), gain_jitter,
                     device)


def make_prompt(n: int, vocab: int, seed: int, req: int = 0, device="cpu") -> torch.Tensor:
    """Prompt ids uniform over the vocabulary (stand-in for benchmark prompts)."""
    return hashed_uniform_ids(n, tensor_seed(seed, req, "prompt"), vocab, device)


def make_random_kv(shape, seed: int, layer: int, which: str, device="cpu") -> torch.Tensor:
    """Random prefix K or V rows (bf16, unit variance), written straight into a cache."""
    return hashed_normal(shape, tensor_seed(seed, layer, "kv_" + which), 1.0, device)


def make_hidden(rows: int, d: int, seed: int, device="cpu", std: float = 1.0) -> torch.Tensor:
    """Random residual-stream rows (fp32 holding bf16 values)."""
    return hashed_normal((rows, d), tensor_seed(seed, 0, "hidden"), std, device,
                         dtype=torch.float32)


class ModelWeights:
    """Lazily generated weights of a model (one layer materialised at a time on demand)."""

    def __init__(self, cfg: ModelConfig, model_seed: int = 0, device="cpu",
                 gain_jitter: float = 0.0, cache: bool = True):
        self.cfg = cfg
        self.model_seed = model_seed
        self.device = device
        self.gain_jitter = gain_jitter
        self._cache = cache
        self._layers: Dict[int, Dict[str, torch.Tensor]] = {}
        self._embed: Optional[torch.Tensor] = None
        self._final: Optional[torch.Tensor] = None

    def layer(self, i: int) -> Dict[str, torch.Tensor]:
        if i in self._layers:
            return self._layers[i]
        w = make_layer_weights(self.cfg, i, self.model_seed, self.device, self.gain_jitter)
        if self._cache:
            self._layers[i] = w
        return w

    @property
    def embed(self) -> torch.Tensor:
        if self._embed is None:
            self._embed = make_embedding(self.cfg, self.model_seed, self.device)
        return self._embed

    @property
    def final_norm(self) -> torch.Tensor:
        if self._final is None:
            self._final = make_final_norm(self.cfg, self.model_seed, self.device,
                                          self.gain_jitter)
        return self._final
