"""CPU oracle of one block-diffusion denoising step (NumPy, float64).

TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's CPU
baseline may import this module. The product path (the HIP library and its
Python binding) never does, and this module imports nothing from it.

Every function is a plain transcription of what the pages describe, computed
in float64 on float64 copies of the bf16 weights. No blocking or fusion beyond
what the definitions state; loops run over heads, experts and requests so the
code can be checked against the pages by eye.

Sources (cited by page and section):
  [explainer]  codemajin.net DiffusionGemma architecture explainer
               §2.1 base model (MoE: 8 of 128 experts plus 1 shared per token)
               §3.1 discrete diffusion (uniform-state forward process, the
                    network predicts clean-token distributions for all
                    canvas positions in parallel)
               §3.2 weight-shared causal encoder / bidirectional decoder,
                    block-autoregressive KV cache, committed blocks never
                    rewritten, tokens inside the block may still change
               §3.3 sampler (confidence-ordered acceptance, re-noise the rest
                    to uniform ids, temperature 0.8 -> 0.4 linear)
               §5.1 TPF / TPS definitions
  [aibars]     aibars.net news item: low-confidence tokens are re-noised to
               random tokens; blocks are committed to the KV cache
  [aiboss]     aiboss88.com product page: prefill uses causal attention into
               the KV cache, denoising uses bidirectional attention over the
               canvas; confident tokens are fixed step by step

Readings where the pages are silent:
  pre-norm RMSNorm (eps 1e-6) before attention and MoE plus a final norm;
  rotate-half RoPE, theta 10000, canvas at absolute positions P..P+C-1;
  scale 1/sqrt(head_dim), no soft-cap, no sliding window;
  GQA: q head h reads kv head floor(h * Hkv / Hq);
  router = top-k of the router logits (ties to the lower expert id), softmax
  over the k selected logits, shared expert added with weight 1;
  SwiGLU experts; LM head tied to the embedding, no input scaling;
  confidence = log of the temperature-tau probability of the candidate token,
  or (entropy mode) minus the entropy of the position's temperature-tau
  distribution;
  adaptive stopping compares the mean entropy of that distribution with the
  threshold, requires every argmax to equal the previous step's, and then
  accepts every position (the step acts as the block's last);
  candidate = held token for committed positions, greedy argmax otherwise
  (or a sample of softmax(L/tau) by Gumbel-max, from counter-based uniforms);
  cumulative schedule k_s = floor(s * C / S);
  committed positions hold their token until they fall out of the top-k_s;
  self-conditioning (optional): the previous step's predicted distribution
  p_i = softmax(L_i) (the network's own prediction, temperature 1) through
  the tied embedding, e_i = sum_v p_iv E_v, then a SwiGLU feed-forward layer
  d -> F_sc -> d, added to the next step's input embedding of position i;
  nothing is added at the first step of a block.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from .philox import gumbel_uniforms, uniform_ids


def f64(a) -> np.ndarray:
    """float64 copy of a weight or activation (bf16 values are exact in float64)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# building blocks
# ----------------------------------------------------------------------------

def rms_norm(x: np.ndarray, gain, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain, per row (pre-norm reading)."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * f64(gain)


def rope_angles(positions, head_dim: int, theta: float) -> np.ndarray:
    """angle[p, j] = pos_p * theta^(-2j/head_dim), j < head_dim/2."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * j / head_dim)
    return np.asarray(positions, np.float64)[:, None] * inv_freq[None, :]


def rope(x: np.ndarray, positions, theta: float) -> np.ndarray:
    """Rotate-half RoPE: pairs (j, j + dh/2) rotated by angle[pos, j].

    x: [n, heads, dh]; positions: [n].
    """
    dh = x.shape[-1]
    half = dh // 2
    ang = rope_angles(positions, dh, theta)
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_prefix: int,
              causal: bool) -> np.ndarray:
    """softmax(q k^T / sqrt(dh)) v per query head.

    q: [n, Hq, dh] for the n canvas (or block) positions;
    k, v: [n_prefix + n, Hkv, dh] = cached prefix rows followed by the rows of
    the same n positions. Denoising is bidirectional over the canvas (no mask);
    the causal encoder lets position i see the prefix and block positions <= i.
    """
    n, Hq, dh = q.shape
    Hkv = k.shape[1]
    nk = k.shape[0]
    assert nk == n_prefix + n
    o = np.empty_like(q, dtype=np.float64)
    for h in range(Hq):
        g = (h * Hkv) // Hq
        s = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(dh)
        if causal:
            key_pos = np.arange(nk)[None, :]
            limit = n_prefix + np.arange(n)[:, None]
            s = np.where(key_pos <= limit, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        o[:, h, :] = p @ v[:, g, :]
    return o


def route(z: np.ndarray, top_k: int):
    """Top-k experts per row (descending logit, ties to the lower expert id) and
    the softmax of the k selected logits.

    Returns idx int64 [n, k] (selection order) and w float64 [n, k].
    """
    z = np.asarray(z, np.float64)
    n, E = z.shape
    idx = np.empty((n, top_k), np.int64)
    for t in range(n):
        row = z[t].copy()
        for j in range(top_k):
            best = int(np.argmax(row))  # first maximum: the lower id wins ties
            idx[t, j] = best
            row[best] = -np.inf
    sel = np.take_along_axis(z, idx, axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = ex / ex.sum(axis=1, keepdims=True)
    return idx, w


def permutation(idx: np.ndarray, n_experts: int):
    """Token -> expert grouping: counts, exclusive offsets, slot order, inverse.

    perm lists token ids grouped by expert, tokens ascending within an expert;
    slot[t, j] is the position in perm of token t's j-th selection.
    """
    n, k = idx.shape
    cnt = np.array([np.count_nonzero(idx == e) for e in range(n_experts)], np.int64)
    off = np.zeros(n_experts + 1, np.int64)
    for e in range(n_experts):
        off[e + 1] = off[e] + cnt[e]
    perm = np.empty(n * k, np.int64)
    slot = np.empty((n, k), np.int64)
    for e in range(n_experts):
        tok, sel = np.nonzero(idx == e)  # row-major: tokens ascending
        perm[off[e]:off[e + 1]] = tok
        slot[tok, sel] = off[e] + np.arange(len(tok))
    return cnt, off, perm, slot


def silu(a: np.ndarray) -> np.ndarray:
    return a / (1.0 + np.exp(-a))


def swiglu(x: np.ndarray, w_gate, w_up, w_down) -> np.ndarray:
    """(silu(x Wg^T) * (x Wu^T)) Wd^T."""
    return (silu(x @ f64(w_gate).T) * (x @ f64(w_up).T)) @ f64(w_down).T


def moe(u: np.ndarray, idx: np.ndarray, w: np.ndarray, lw: Dict, n_experts: int,
        perm_info=None) -> np.ndarray:
    """sum_j w_tj * Expert_{idx_tj}(u_t) + Shared(u_t), experts run on their token groups."""
    out = swiglu(u, lw["ws_gate"], lw["ws_up"], lw["ws_down"])
    cnt, off, perm, slot = perm_info if perm_info is not None else permutation(idx, n_experts)
    n, k = idx.shape
    slot_weight = np.empty(n * k, np.float64)
    for t in range(n):
        for j in range(k):
            slot_weight[slot[t, j]] = w[t, j]
    wg, wu, wd = lw["w_gate"], lw["w_up"], lw["w_down"]
    for e in range(n_experts):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        rows = perm[lo:hi]
        y = swiglu(u[rows], wg[e], wu[e], wd[e])
        out[rows] += slot_weight[lo:hi, None] * y
    return out


# ----------------------------------------------------------------------------
# one transformer layer over the rows of one request
# ----------------------------------------------------------------------------

def layer_forward(h: np.ndarray, lw: Dict, cfg, cache_k: np.ndarray, cache_v: np.ndarray,
                  n_prefix: int, causal: bool, keep: Optional[Dict] = None):
    """One pre-norm attention + MoE layer on n rows at positions n_prefix..n_prefix+n-1.

    cache_k, cache_v: [>= n_prefix, Hkv, dh] prefix rows (K already rotated).
    Returns (new h, k rows [n, Hkv, dh] rotated, v rows). `keep`, when given,
    receives the intermediates by name.
    """
    n, d = h.shape
    Hq, Hkv, dh = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    pos = n_prefix + np.arange(n)
    u = rms_norm(h, lw["attn_norm"], cfg.rms_eps)
    qkv = u @ f64(lw["w_qkv"]).T
    q = qkv[:, : Hq * dh].reshape(n, Hq, dh)
    k = qkv[:, Hq * dh: (Hq + Hkv) * dh].reshape(n, Hkv, dh)
    v = qkv[:, (Hq + Hkv) * dh:].reshape(n, Hkv, dh)
    q = rope(q, pos, cfg.rope_theta)
    k = rope(k, pos, cfg.rope_theta)
    k_all = np.concatenate([f64(cache_k[:n_prefix]), k], axis=0)
    v_all = np.concatenate([f64(cache_v[:n_prefix]), v], axis=0)
    o = attention(q, k_all, v_all, n_prefix, causal)
    h1 = h + o.reshape(n, Hq * dh) @ f64(lw["w_o"]).T
    u2 = rms_norm(h1, lw["moe_norm"], cfg.rms_eps)
    z = u2 @ f64(lw["w_router"]).T
    idx, w = route(z, cfg.top_k)
    pinfo = permutation(idx, cfg.n_experts)
    h2 = h1 + moe(u2, idx, w, lw, cfg.n_experts, pinfo)
    if keep is not None:
        keep.update(u_attn=u, q=q, k=k, v=v, attn_o=o, h_mid=h1, u_moe=u2, z=z,
                    idx=idx, w=w, cnt=pinfo[0], off=pinfo[1], perm=pinfo[2],
                    slot=pinfo[3], h_out=h2)
    return h2, k, v


# ----------------------------------------------------------------------------
# LM head statistics and the confidence sampler
# ----------------------------------------------------------------------------

def tau_at(step: int, n_steps: int, tau_first: float, tau_last: float, precision: str = "float64"):
    """Temperature falling linearly from tau_first (step 1) to tau_last (step S).

    precision "float32" evaluates tau_first + ((tau_last - tau_first) * (s-1)) / (S-1)
    in IEEE float32, operation by operation (the precision of a float32
    implementation of the same schedule)."""
    if precision == "float32":
        f = np.float32
        if n_steps <= 1:
            return f(tau_first)
        return f(f(tau_first) + f(f(f(tau_last) - f(tau_first)) * f(step - 1)) / f(n_steps - 1))
    if n_steps <= 1:
        return float(tau_first)
    return float(tau_first) + (float(tau_last) - float(tau_first)) * (step - 1) / (n_steps - 1)


def commit_count(step: int, n_steps: int, canvas: int) -> int:
    """Cumulative number of canvas positions accepted after step s: floor(s*C/S)."""
    return (step * canvas) // n_steps


def expected_embedding(L: np.ndarray, embed, chunk: int = 32768) -> np.ndarray:
    """e_i = sum_v p_iv E_v with p_i = softmax(L_i) over the whole vocabulary:
    the predicted clean-token distribution passed through the embedding
    matrix (explainer §3.2, self-conditioning). float64 [n, d]."""
    L = np.asarray(L, np.float64)
    p = np.exp(L - L.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    V = L.shape[1]
    e = np.zeros((L.shape[0], embed.shape[1]), np.float64)
    for v0 in range(0, V, chunk):
        e += p[:, v0:v0 + chunk] @ f64(embed[v0:v0 + chunk])
    return e


def self_condition(L: np.ndarray, embed, sc: Dict, chunk: int = 32768) -> np.ndarray:
    """Self-conditioning signal of a step (explainer §3.2): the expected
    embedding under the step's predicted distribution, through a small
    feed-forward layer (SwiGLU, weights sc_gate, sc_up [F_sc][d], sc_down
    [d][F_sc]). Added to the next step's input embedding."""
    e = expected_embedding(L, embed, chunk)
    return swiglu(e, sc["sc_gate"], sc["sc_up"], sc["sc_down"])


def logits(h: np.ndarray, final_norm, embed, cfg, chunk: int = 32768) -> np.ndarray:
    """RMSNorm(h) E^T over the whole vocabulary (tied LM head), float64 [n, V]."""
    hf = rms_norm(h, final_norm, cfg.rms_eps)
    V = embed.shape[0]
    out = np.empty((h.shape[0], V), np.float64)
    for v0 in range(0, V, chunk):
        out[:, v0:v0 + chunk] = hf @ f64(embed[v0:v0 + chunk]).T
    return out


def row_stats(L: np.ndarray, held: np.ndarray, tau: float):
    """Per row: max M, first argmax a, log Z with Z = sum_v exp((L_v - M)/tau),
    and the logit of the held token."""
    M = L.max(axis=1)
    a = np.argmax(L, axis=1)
    logZ = np.log(np.sum(np.exp((L - M[:, None]) / tau), axis=1))
    gx = L[np.arange(L.shape[0]), held]
    return M, a, logZ, gx


def row_entropy(L: np.ndarray, tau: float, chunk: int = 16) -> np.ndarray:
    """Entropy in nats of each row's temperature-tau distribution,
    H_i = -sum_v p_iv log p_iv with p_i = softmax(L_i / tau); a term with
    p_iv = 0 contributes 0. (explainer §3.3: the sampler's uncertainty
    measure is the predicted entropy of each canvas position.)"""
    L = np.asarray(L, np.float64)
    H = np.empty(L.shape[0], np.float64)
    for r0 in range(0, L.shape[0], chunk):
        S = L[r0:r0 + chunk] / tau
        e = np.exp(S - S.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        with np.errstate(divide="ignore", invalid="ignore"):
            plogp = np.where(p > 0, p * np.log(p), 0.0)
        H[r0:r0 + chunk] = -plogp.sum(axis=1)
    return H


def gumbel_candidates(L: np.ndarray, tau: float, seed: int, step: int, block: int, request: int,
                      rows: Optional[Sequence[int]] = None):
    """Sampled candidates y_i ~ softmax(L_i / tau) by the Gumbel-max identity:
    y_i = argmax_v (L_iv / tau - ln(-ln u_iv)) with the position's uniforms
    u (philox.gumbel_uniforms), ties to the lower id. Returns (y, L_i[y_i])
    for the given rows (default: all)."""
    L = np.asarray(L, np.float64)
    rows = range(L.shape[0]) if rows is None else rows
    ys, ly = [], []
    for i in rows:
        u = gumbel_uniforms(seed, i, step, block, request, L.shape[1])
        key = L[i] / tau - np.log(-np.log(u))
        y = int(np.argmax(key))
        ys.append(y)
        ly.append(L[i, y])
    return np.array(ys, np.int64), np.array(ly, np.float64)


def adaptive_stop(H: np.ndarray, a: np.ndarray, a_prev: Optional[np.ndarray],
                  threshold: float) -> bool:
    """Adaptive stopping (explainer §3.3): the block stops when the mean
    predicted entropy over the canvas is below the threshold and every
    position's most likely token is the one it had at the previous step.
    The first step of a block has no previous prediction and never stops."""
    if a_prev is None:
        return False
    return bool(np.mean(H) < threshold and np.array_equal(np.asarray(a), np.asarray(a_prev)))


def sample(x: np.ndarray, m: np.ndarray, M, a, logZ, gx, tau: float, step: int,
           n_steps: int, seed: int, block: int, request: int, vocab: int,
           confidence: str = "prob", H: Optional[np.ndarray] = None, stop: bool = False,
           drawn: Optional[tuple] = None, precision: str = "float64"):
    """Confidence-ordered acceptance with uniform re-noise.

    Candidate y_i: the held token if position i is committed, else the argmax
    or, when `drawn` = (ids, their logits) is given, the sampled candidate
    (gumbel_candidates).
    Confidence, by `confidence`:
      "prob":    c_i = log p_tau(y_i) = (L[y_i] - M_i)/tau - log Z_i;
      "entropy": c_i = -H_i, so low-entropy positions come first
                 (explainer §3.3).
    The k_s positions of highest confidence (ties to the lower position) are
    accepted (x_i = y_i, committed); every other position is re-noised to a
    uniform id from Philox at counter (i, step, block, request). When the
    block stops early (`stop`), the step acts as the last one: every position
    is accepted.
    precision "float32" takes the statistics, tau and every operation of the
    confidence in IEEE float32, so that the ranking is decided in the
    precision of a float32 implementation fed the same statistics.
    Returns (new x, new committed mask, c, accepted-set boolean mask).
    """
    C = x.shape[0]
    committed = np.asarray(m).astype(bool)
    cand, Lc = (a, M) if drawn is None else drawn
    y = np.where(committed, x, cand)
    ft = np.float32 if precision == "float32" else np.float64
    if confidence == "prob":
        Ly = np.where(committed, np.asarray(gx, ft), np.asarray(Lc, ft))
        c = (Ly - np.asarray(M, ft)) / ft(tau) - np.asarray(logZ, ft)
    elif confidence == "entropy":
        c = -np.asarray(H, ft)
    else:
        raise ValueError(confidence)
    k_s = C if stop else commit_count(step, n_steps, C)
    order = sorted(range(C), key=lambda i: (-c[i], i))
    accept = np.zeros(C, bool)
    accept[order[:k_s]] = True
    noise = uniform_ids(seed, np.arange(C), step, block, request, vocab)
    x_new = np.where(accept, y, noise)
    m_new = accept.astype(np.uint8)
    return x_new.astype(np.int64), m_new, c, accept


def init_canvas(seed: int, block: int, request: int, canvas: int, vocab: int):
    """Canvas of uniform random placeholders (Philox step 0), nothing committed."""
    x = uniform_ids(seed, np.arange(canvas), 0, block, request, vocab)
    return x.astype(np.int64), np.zeros(canvas, np.uint8)


# ----------------------------------------------------------------------------
# request state and the three calls of the loop
# ----------------------------------------------------------------------------

class Request:
    """KV cache of one request: per layer K (rotated) and V rows, float64."""

    def __init__(self, cfg, max_ctx: int):
        self.cfg = cfg
        L, Hkv, dh = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
        self.k = np.zeros((L, max_ctx, Hkv, dh), np.float64)
        self.v = np.zeros((L, max_ctx, Hkv, dh), np.float64)
        self.length = 0


def forward_rows(weights, cfg, req: Request, ids: np.ndarray, causal: bool,
                 keep_layers: Optional[List[Dict]] = None, stop_layer: Optional[int] = None,
                 sc_prev: Optional[np.ndarray] = None):
    """Embed ids and run the layer stack at positions req.length.. (no cache
    write). sc_prev, when given, is added to the input embeddings
    (self-conditioning from the previous denoising step)."""
    h = f64(weights.embed[ids])
    if sc_prev is not None:
        h = h + sc_prev
    P = req.length
    ks, vs = [], []
    for l in range(cfg.n_layers if stop_layer is None else stop_layer):
        keep = {} if keep_layers is not None else None
        h, k, v = layer_forward(h, weights.layer(l), cfg, req.k[l], req.v[l], P, causal, keep)
        if keep_layers is not None:
            keep_layers.append(keep)
        ks.append(k)
        vs.append(v)
    return h, ks, vs


def append_rows(weights, cfg, req: Request, ids: np.ndarray):
    """Causal encoder pass over ids; their K/V rows are appended to the cache.

    Rows [0, length) are never written (committed blocks are immutable).
    """
    n = len(ids)
    assert req.length + n <= req.k.shape[1]
    _, ks, vs = forward_rows(weights, cfg, req, np.asarray(ids), causal=True)
    P = req.length
    for l in range(cfg.n_layers):
        req.k[l, P:P + n] = ks[l]
        req.v[l, P:P + n] = vs[l]
    req.length = P + n


def prefill(weights, cfg, req: Request, ids: np.ndarray):
    """Causal prefill of a prompt into the KV cache."""
    append_rows(weights, cfg, req, ids)


def commit_block(weights, cfg, req: Request, canvas_ids: np.ndarray):
    """Append a finished block: the same causal pass as prefill, over the canvas."""
    append_rows(weights, cfg, req, canvas_ids)


def denoise_step(weights, cfg, req: Request, x: np.ndarray, m: np.ndarray, step: int,
                 n_steps: int, seed: int, block: int, request: int,
                 keep: Optional[Dict] = None, confidence: str = "prob",
                 stop_entropy: float = 0.0, a_prev: Optional[np.ndarray] = None,
                 candidate: str = "argmax", sc: Optional[Dict] = None,
                 sc_prev: Optional[np.ndarray] = None):
    """One denoising step of one request's canvas.

    The canvas attends bidirectionally to itself and to the cached prefix; the
    LM head gives per-row statistics; the sampler accepts the top-k_s positions
    and re-noises the rest. The cache is read, never written. With
    stop_entropy > 0 the step checks adaptive stopping against a_prev, the
    argmax of the previous step (None at the first step of a block). With
    self-conditioning weights sc, sc_prev (the previous step's signal, None
    at the first step of a block) is added to the input embeddings and this
    step's signal is left in keep["sc"].
    """
    layers = [] if keep is not None else None
    h, _, _ = forward_rows(weights, cfg, req, np.asarray(x), causal=False, keep_layers=layers,
                           sc_prev=sc_prev)
    tau = tau_at(step, n_steps, cfg.tau_first, cfg.tau_last)
    L = logits(h, weights.final_norm, weights.embed, cfg)
    M, a, logZ, gx = row_stats(L, np.asarray(x), tau)
    H = row_entropy(L, tau)
    stop = stop_entropy > 0 and adaptive_stop(H, a, a_prev, stop_entropy)
    drawn = gumbel_candidates(L, tau, seed, step, block, request) if candidate == "sample" else None
    x_new, m_new, c, accept = sample(x, m, M, a, logZ, gx, tau, step, n_steps, seed, block,
                                     request, cfg.vocab, confidence=confidence, H=H, stop=stop,
                                     drawn=drawn)
    if keep is not None:
        keep.update(layers=layers, h=h, logits=L, M=M, a=a, logZ=logZ, gx=gx, c=c,
                    accept=accept, tau=tau, H=H, stop=stop, drawn=drawn,
                    sc=self_condition(L, weights.embed, sc) if sc is not None else None)
    return x_new, m_new


def ar_step(weights, cfg, req: Request, token: int):
    """One autoregressive decode step: the causal pass over the single token
    at position req.length appends its K/V rows, and the LM head over that
    row gives the next token, the greedy argmax (lowest id on ties). The
    explainer's §5.2 compares a denoising step with one such step.
    Returns (next token, the row's logits)."""
    ids = np.asarray([token], np.int64)
    h, ks, vs = forward_rows(weights, cfg, req, ids, causal=True)
    P = req.length
    assert P + 1 <= req.k.shape[1]
    for l in range(cfg.n_layers):
        req.k[l, P:P + 1] = ks[l]
        req.v[l, P:P + 1] = vs[l]
    req.length = P + 1
    L = logits(h, weights.final_norm, weights.embed, cfg)[0]
    return int(np.argmax(L)), L


def generate_block(weights, cfg, req: Request, n_steps: int, seed: int, block: int,
                   request: int, confidence: str = "prob", stop_entropy: float = 0.0,
                   sc: Optional[Dict] = None):
    """Denoise one block from uniform noise for at most n_steps (fewer when
    adaptive stopping fires), then commit it. With self-conditioning weights
    sc, each step after the first adds the previous step's signal to its
    input. Returns (x, m, steps taken)."""
    x, m = init_canvas(seed, block, request, cfg.canvas, cfg.vocab)
    a_prev = None
    sc_prev = None
    taken = 0
    for s in range(1, n_steps + 1):
        keep: Dict = {}
        x, m = denoise_step(weights, cfg, req, x, m, s, n_steps, seed, block, request, keep=keep,
                            confidence=confidence, stop_entropy=stop_entropy, a_prev=a_prev,
                            sc=sc, sc_prev=sc_prev)
        a_prev = keep["a"]
        sc_prev = keep["sc"]
        taken = s
        if keep["stop"]:
            break
    commit_block(weights, cfg, req, x)
    return x, m, taken
