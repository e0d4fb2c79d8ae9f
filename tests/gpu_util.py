"""Helpers of the GPU parity tests: build engines, mirror weights on the host
for the oracle, and compare with explicit tolerances."""
import sys

import numpy as np
import torch

from block_discrete_diffusion_dg_amd import synth
from block_discrete_diffusion_dg_amd.engine import Engine, gpu_weights
from oracle import fp8
from oracle import model as om

# Floating-point bar: max |gpu - oracle| / max |oracle| per tensor (bf16
# operands, fp32 accumulation on the GPU; float64 oracle on the bf16 weights).
REL_TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def max_rel(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(gpu - ref)) / max(np.max(np.abs(ref)), 1e-30))


EXPERT_FIELDS = ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")


class _DequantizedBank:
    """bank[e] -> the oracle's FP8-dequantised float64 weights of expert e
    (computed on first use: a layer touches only its routed experts)."""

    def __init__(self, bank):
        self._bank = bank
        self._cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self._cache:
            self._cache[e] = fp8.dequantize_bank(om.f64(self._bank[e]))
        return self._cache[e]


class HostWeights:
    """Host (CPU) copies of GPU weights, one layer at a time, for the oracle.
    With expert_format "fp8" the expert matrices are the oracle's dequantised
    FP8 weights (the GPU quantises the same bf16 weights bit-identically)."""

    def __init__(self, layers, embed, final_norm, expert_format="bf16"):
        self._layers = layers
        self._embed = embed
        self._final = final_norm
        self._fmt = expert_format
        self._cache = {}

    def layer(self, i):
        if i not in self._cache:
            lw = {k: v.cpu() for k, v in self._layers[i].items()}
            if self._fmt == "fp8":
                for n in EXPERT_FIELDS:
                    lw[n] = _DequantizedBank(lw[n]) if n.startswith("w_") else fp8.dequantize_bank(om.f64(lw[n]))
            self._cache = {i: lw}
        return self._cache[i]

    @property
    def embed(self):
        if not isinstance(self._embed, torch.Tensor) or self._embed.is_cuda:
            self._embed = self._embed.cpu()
        return self._embed

    @property
    def final_norm(self):
        return self._final.cpu()


def make_engine(cfg, max_ctx, max_requests=1, max_rows=None, gain_jitter=0.1, seed=0, expert_format="bf16"):
    say(f"[engine] {cfg.name} L={cfg.n_layers} d={cfg.d_model} V={cfg.vocab} max_ctx={max_ctx} "
        f"experts={expert_format}")
    layers, embed, final = gpu_weights(cfg, seed, gain_jitter)
    torch.cuda.synchronize()
    eng = Engine(cfg, layers, embed, final, max_ctx, max_requests, max_rows, expert_format=expert_format)
    return eng, HostWeights(layers, embed, final, expert_format)


def tie_gap_ok(keys, k, band):
    """True when the k-th and (k+1)-th largest keys differ by more than band
    (the selected set is then unique up to floating-point noise)."""
    s = np.sort(np.asarray(keys, np.float64))[::-1]
    if k <= 0 or k >= len(s):
        return True
    return (s[k - 1] - s[k]) > band
