"""Helpers of the GPU parity tests: build engines, mirror weights on the host
for the oracle, and compare with explicit tolerances."""
import sys

import numpy as np
import scipy.special
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


# Element-wise relative errors are reported beside the per-tensor bar, each
# element's error taken against max(|o|, ELEM_FLOOR * max|o|) so that
# elements near zero do not dominate.
ELEM_FLOOR = 1e-3


def elem_stats(gpu, ref):
    """Element-wise |g - o| / max(|o|, 1e-3 max|o|): its maximum, 99th
    percentile and median over the tensor."""
    gpu = np.asarray(gpu, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    floor = ELEM_FLOOR * max(float(np.max(np.abs(ref))), 1e-30)
    e = np.abs(gpu - ref) / np.maximum(np.abs(ref), floor)
    return {"max": float(e.max()), "p99": float(np.percentile(e, 99)), "median": float(np.median(e))}


def fmt_elem(stats):
    return "/".join(f"{stats[k]:.1e}" for k in ("max", "p99", "median"))


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


def make_selfcond(cfg, width, seed=0):
    """Self-conditioning weights on the GPU, scaled by 32 (exact in bf16) so
    that the signal is not negligible next to the embeddings."""
    return {k: (v * 32).to(torch.bfloat16) for k, v in synth.make_selfcond_weights(cfg, width, seed, "cuda").items()}


def make_engine(cfg, max_ctx, max_requests=1, max_rows=None, gain_jitter=0.1, seed=0, expert_format="bf16",
                selfcond=None, lmhead_format="bf16"):
    say(f"[engine] {cfg.name} L={cfg.n_layers} d={cfg.d_model} V={cfg.vocab} max_ctx={max_ctx} "
        f"experts={expert_format} selfcond={None if selfcond is None else selfcond['sc_gate'].shape[0]} "
        f"lmhead={lmhead_format}")
    layers, embed, final = gpu_weights(cfg, seed, gain_jitter)
    torch.cuda.synchronize()
    eng = Engine(cfg, layers, embed, final, max_ctx, max_requests, max_rows, expert_format=expert_format,
                 selfcond=selfcond, lmhead_format=lmhead_format)
    return eng, HostWeights(layers, embed, final, expert_format)


def tie_gap_ok(keys, k, band):
    """True when the k-th and (k+1)-th largest keys differ by more than band
    (the selected set is then unique up to floating-point noise)."""
    s = np.sort(np.asarray(keys, np.float64))[::-1]
    if k <= 0 or k >= len(s):
        return True
    return (s[k - 1] - s[k]) > band


def moe_with_experts(keep, lw, cfg, idx):
    """The oracle's layer output with another implementation's expert choice
    imposed: keep holds the oracle's own intermediates of the layer (h_mid,
    u_moe, z); the routing weights are the softmax of the oracle's own logits
    at the imposed experts. Used only where the two choices differ inside
    the router's tie band (the integer decision is then the kernel's)."""
    idx = np.asarray(idx, np.int64)
    sel = np.take_along_axis(keep["z"], idx, axis=1)
    w = scipy.special.softmax(sel, axis=1)
    return keep["h_mid"] + om.moe(keep["u_moe"], idx, w, lw, cfg.n_experts)


def router_band(u, w_router):
    """Per row: the largest change of a gap between two router logits that
    rounding the router's input row u to bf16 can cause. Each element moves by
    at most half an ulp (relative 2^-9), so a logit z_e = sum_k u_k W_ek moves
    by at most 2^-9 sum_k |u_k W_ek|, and a gap by twice the largest such sum.
    A bound fixed by the arithmetic (bf16 operands), not by measured errors."""
    return 2.0 ** -8 * (np.abs(np.asarray(u, np.float64)) @ np.abs(om.f64(w_router)).T).max(axis=1)


def router_swaps(idx_gpu, z_or, top_k, band):
    """Rows whose expert sets differ; asserts each lies inside its tie band
    (the oracle's k-th and (k+1)-th logits closer than band[t])."""
    swaps = []
    for t in range(idx_gpu.shape[0]):
        if set(np.asarray(idx_gpu[t]).tolist()) != set(np.argsort(-z_or[t], kind="stable")[:top_k].tolist()):
            assert not tie_gap_ok(z_or[t], top_k, band[t]), (t, band[t])
            swaps.append(t)
    return swaps
