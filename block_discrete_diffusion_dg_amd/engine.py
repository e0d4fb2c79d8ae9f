"""Engine: torch-allocated device memory around one libdg context.

PyTorch supplies device memory and the current HIP stream; every step of the
denoising path runs in libdg's kernels. This module only marshals tensors into
the C entry points (include/dg.h) and strings them into the block loop the
pages describe (codemajin.net DiffusionGemma explainer §3.2: denoise a
256-token block to completion, append it to the KV cache, start the next).
"""
from __future__ import annotations

import ctypes
from typing import Dict, List, Optional, Sequence

import torch

from . import binding as B
from .synth import LAYER_TENSORS, ModelConfig


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def pack_weight(t: torch.Tensor) -> torch.Tensor:
    """Fragment-major copy of a row-major bf16 GPU matrix (dg_pack_weight);
    a [E][N][K] bank is packed as one [E*N][K] matrix."""
    lib = B.load()
    assert t.dtype == torch.bfloat16 and t.is_cuda and t.is_contiguous()
    k = t.shape[-1]
    out = torch.empty_like(t)
    st = lib.dg_pack_weight(_stream(), t.data_ptr(), out.data_ptr(), t.numel() // k, k)
    if st != B.DG_OK:
        raise B.DGError(st, f"dg_pack_weight failed for shape {tuple(t.shape)}")
    return out


def quantize_fp8(t: torch.Tensor, lmhead: bool = False):
    """FP8 (E4M3) codes of a row-major bf16 matrix or expert bank (uint8,
    same element count; the experts' fragment-major layout, or with lmhead
    the LM head's step-major layout) and its fp32 row scales, made on the GPU
    by dg_quantize_fp8 / dg_quantize_fp8_lmhead."""
    assert t.dtype == torch.bfloat16 and t.is_cuda and t.is_contiguous()
    k = t.shape[-1]
    n = t.numel() // k
    lib = B.load()
    codes = torch.empty(t.numel(), dtype=torch.uint8, device=t.device)
    scale = torch.empty(n, dtype=torch.float32, device=t.device)
    fn = lib.dg_quantize_fp8_lmhead if lmhead else lib.dg_quantize_fp8
    st = fn(_stream(), t.data_ptr(), codes.data_ptr(), scale.data_ptr(), n, k)
    if st != B.DG_OK:
        raise B.DGError(st, f"FP8 quantisation failed for shape {tuple(t.shape)}")
    return codes, scale


def v_to_cache_order(v: torch.Tensor) -> torch.Tensor:
    """V rows [..., n, dh] (n % 32 == 0) -> the cache's element order: inside
    each 32-key block, key o = 16*half + 4*g + r and dim c sit at
    (g*dh + c)*8 + 4*half + r. Returns [..., n, dh]-shaped storage."""
    *lead, n, dh = v.shape
    assert n % 32 == 0, n
    nl = len(lead)
    t = v.reshape(*lead, n // 32, 2, 4, 4, dh)  # blk, half, g, r, c
    t = t.permute(*range(nl), nl, nl + 2, nl + 4, nl + 1, nl + 3)  # blk, g, c, half, r
    return t.reshape(*lead, n, dh)


def v_from_cache_order(raw: torch.Tensor) -> torch.Tensor:
    """Inverse of v_to_cache_order: [..., n, dh] cache storage -> V rows."""
    *lead, n, dh = raw.shape
    nl = len(lead)
    t = raw.reshape(*lead, n // 32, 4, dh, 2, 4)  # blk, g, c, half, r
    t = t.permute(*range(nl), nl, nl + 3, nl + 1, nl + 4, nl + 2)  # blk, half, g, r, c
    return t.reshape(*lead, n, dh)


class Engine:
    """One context: weights (bf16, on the GPU), KV cache and workspace tensors.

    `layers` and `embed` hold row-major tensors (the synth/oracle
    convention); the streamed matrices (projections, experts, embedding) are
    repacked on the GPU into the library's fragment-major layout, and only the
    packed copies are kept."""

    def __init__(self, cfg: ModelConfig, layers: Sequence[Dict[str, torch.Tensor]],
                 embed: torch.Tensor, final_norm: torch.Tensor, max_ctx: int,
                 max_requests: int = 1, max_rows: Optional[int] = None,
                 expert_format: str = "bf16", selfcond: Optional[Dict[str, torch.Tensor]] = None,
                 lmhead_format: str = "bf16"):
        """selfcond: the self-conditioning feed-forward layer (sc_gate, sc_up
        [F][d], sc_down [d][F], bf16, row-major), or None for none.
        lmhead_format "fp8": the LM head reads an FP8 copy of the embedding."""
        self.lib = B.load()
        self.cfg = cfg
        dev = embed.device
        if dev.type != "cuda":
            raise RuntimeError("Engine needs weights on a GPU device")
        self.max_rows = max_rows or cfg.canvas * max_requests
        c = B.DGConfig()
        for name in ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "n_experts",
                     "top_k", "d_expert", "d_shared", "vocab", "canvas"):
            setattr(c, name, getattr(cfg, name))
        c.max_ctx, c.max_requests, c.max_rows = max_ctx, max_requests, self.max_rows
        c.rms_eps, c.rope_theta = cfg.rms_eps, cfg.rope_theta
        c.tau_first, c.tau_last = cfg.tau_first, cfg.tau_last
        c.expert_format = B.WEIGHT_FORMAT[expert_format]
        c.d_selfcond = 0 if selfcond is None else selfcond["sc_gate"].shape[0]
        c.lmhead_format = B.WEIGHT_FORMAT[lmhead_format]
        self.lmhead_format = lmhead_format
        self.expert_format = expert_format
        self.c_cfg = c
        sc_ptrs = [None] * 4
        self._keep = []
        if selfcond is not None:
            # the contraction over the vocabulary streams the transposed embedding
            embed_t = pack_weight(embed.t().contiguous())
            packed = [pack_weight(selfcond[n].contiguous()) for n in ("sc_gate", "sc_up", "sc_down")]
            self._keep += packed + [embed_t]
            sc_ptrs = [t.data_ptr() for t in packed] + [embed_t.data_ptr()]
        lm8_ptrs = [None, None]
        if lmhead_format == "fp8":
            codes, scale = quantize_fp8(embed, lmhead=True)
            self._keep += [codes, scale]
            lm8_ptrs = [codes.data_ptr(), scale.data_ptr()]
        embed = pack_weight(embed)  # the tied LM head streams it fragment-major
        self._keep += [embed, final_norm]
        arr = (B.DGLayerWeights * max(1, len(layers)))()
        for i, lw in enumerate(layers):
            for name in LAYER_TENSORS:
                t = lw[name]
                assert t.dtype == torch.bfloat16 and t.is_contiguous() and t.device == dev, name
                if expert_format == "fp8" and name in B.EXPERT_FIELDS:
                    t, scale = quantize_fp8(t)
                    self._keep.append(scale)
                    setattr(arr[i], B.SCALE_FIELDS[B.EXPERT_FIELDS.index(name)], scale.data_ptr())
                elif name in B.PACKED_FIELDS:
                    t = pack_weight(t)
                self._keep.append(t)
                setattr(arr[i], name, t.data_ptr())
        self._layer_arr = arr
        w = B.DGWeights(embed.data_ptr(), final_norm.data_ptr(), arr, *sc_ptrs, *lm8_ptrs)
        kv_bytes = self.lib.dg_kv_cache_bytes(ctypes.byref(c))
        ws_bytes = self.lib.dg_workspace_bytes(ctypes.byref(c))
        if ws_bytes == 0:
            raise B.DGError(B.DG_EINVAL, "unsupported configuration")
        self.kv = torch.zeros(max(256, max_requests * kv_bytes), dtype=torch.uint8, device=dev)
        self.kv_bytes = max_requests * kv_bytes
        self.ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        h = ctypes.c_void_p()
        st = self.lib.dg_create(ctypes.byref(c), ctypes.byref(w), self.kv.data_ptr(),
                                self.ws.data_ptr(), ws_bytes, ctypes.byref(h))
        if st != B.DG_OK:
            raise B.DGError(st, "dg_create failed")
        self.ctx = h
        self.layout = B.DGWsLayout()
        self._check(self.lib.dg_workspace_layout(ctypes.byref(c), ctypes.byref(self.layout)))
        self.max_ctx = max_ctx
        self.max_requests = max_requests

    # ------------------------------------------------------------------ plumbing
    def close(self):
        if getattr(self, "ctx", None):
            self.lib.dg_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, status: int):
        if status != B.DG_OK:
            msg = self.lib.dg_last_error(self.ctx).decode() if getattr(self, "ctx", None) else ""
            raise B.DGError(status, msg)

    def cache_rows(self, slot: int, layer: int, lo: int, hi: int):
        """K and V rows [lo, hi) of one slot and layer, each [kv_head][hi-lo][head_dim]
        bf16 on the device (V converted from the cache's block order)."""
        kv = self.kv_view()
        k = kv[slot, layer, 0, :, lo:hi]
        b0, b1 = lo // 32 * 32, -(-hi // 32) * 32
        v = v_from_cache_order(kv[slot, layer, 1, :, b0:b1])[:, lo - b0:hi - b0]
        return k, v

    def set_cache_rows(self, slot: int, layer: int, k: torch.Tensor, v: torch.Tensor):
        """Write K and V rows [0, n) of one slot and layer (n % 32 == 0), each
        [kv_head][n][head_dim] bf16, in the cache's layout."""
        n = k.shape[1]
        kv = self.kv_view()
        kv[slot, layer, 0, :, :n] = k.to(kv.device)
        kv[slot, layer, 1, :, :n] = v_to_cache_order(v.to(kv.device))

    def kv_view(self) -> torch.Tensor:
        """[slot][layer][K|V][kv_head][max_ctx][head_dim] bf16 view of the raw
        cache; V planes are in block operand order (v_from_cache_order)."""
        c = self.cfg
        return self.kv[:self.kv_bytes].view(torch.bfloat16).view(
            self.max_requests, c.n_layers, 2, c.n_kv_heads, self.max_ctx, c.head_dim)

    def ws_view(self, name: str, dtype: torch.dtype, shape) -> torch.Tensor:
        off = getattr(self.layout, name)
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        return self.ws[off:off + nbytes].view(dtype).view(*shape)

    def moe_counters(self) -> Dict[str, int]:
        """Running expert-kernel counters kept in the workspace (waits for the
        GPU): spin timeouts, touched experts summed over layer calls, calls."""
        w = self.ws_view("items", torch.int32, (B.ITEMS_PERMUTE_CALLS + 2,)).cpu()
        w64 = w[B.ITEMS_TOUCHED_TOTAL:B.ITEMS_PERMUTE_CALLS + 2].view(torch.int64)
        return {"spin_timeouts": int(w[B.ITEMS_SPIN_TIMEOUTS]), "touched_total": int(w64[0]),
                "permute_calls": int(w64[1])}

    def sync(self):
        """Wait for the current stream and raise if a bounded wait of the
        expert kernel ran out since the previous check (dg_sync)."""
        self._check(self.lib.dg_sync(self.ctx, _stream()))

    def cache_len(self, req: int) -> int:
        return self.lib.dg_cache_len(self.ctx, req)

    def set_cache_len(self, req: int, n: int):
        self._check(self.lib.dg_set_cache_len(self.ctx, req, n))

    def _args(self, reqs, canvas, committed, step, n_steps, seeds, blocks, stats,
              confidence: str = "prob", stop_entropy: float = 0.0,
              stop: Optional[torch.Tensor] = None, candidate: str = "argmax"):
        n = len(reqs)
        a = B.DGStepArgs()
        a.n_req = n
        self._req_arr = (ctypes.c_int32 * n)(*reqs)
        self._seed_arr = (ctypes.c_uint64 * n)(*[int(s) & (2**64 - 1) for s in seeds])
        self._block_arr = (ctypes.c_int32 * n)(*blocks)
        a.req = self._req_arr
        a.seed = self._seed_arr
        a.block = self._block_arr
        assert canvas.dtype == torch.int32 and canvas.is_cuda and canvas.is_contiguous()
        assert committed.dtype == torch.uint8 and committed.is_cuda and committed.is_contiguous()
        assert canvas.numel() == n * self.cfg.canvas and committed.numel() == n * self.cfg.canvas
        a.d_canvas = canvas.data_ptr()
        a.d_committed = committed.data_ptr()
        a.step, a.n_steps = step, n_steps
        a.d_stats = _ptr(stats)
        a.confidence = B.CONFIDENCE[confidence]
        a.stop_entropy = float(stop_entropy)
        if stop is not None:
            assert stop.dtype == torch.int32 and stop.is_cuda and stop.numel() >= n
        a.d_stop = _ptr(stop)
        a.candidate = B.CANDIDATE[candidate]
        return a

    # ------------------------------------------------------------------ the calls
    def prefill(self, req: int, ids: torch.Tensor):
        assert ids.dtype == torch.int32 and ids.is_cuda and ids.is_contiguous()
        self._check(self.lib.dg_prefill(self.ctx, _stream(), req, ids.data_ptr(), ids.numel()))

    def init_canvas(self, reqs, canvas, committed, seeds, blocks):
        a = self._args(reqs, canvas, committed, 0, 1, seeds, blocks, None)
        self._check(self.lib.dg_init_canvas(self.ctx, _stream(), ctypes.byref(a)))

    def denoise_step(self, reqs, canvas, committed, step, n_steps, seeds, blocks,
                     stats: Optional[torch.Tensor] = None, confidence: str = "prob",
                     stop_entropy: float = 0.0, stop: Optional[torch.Tensor] = None,
                     candidate: str = "argmax"):
        """One denoising step; `stop` (device int32 [n_req]) receives 1 where
        adaptive stopping ended the request's block at this step."""
        a = self._args(reqs, canvas, committed, step, n_steps, seeds, blocks, stats, confidence,
                       stop_entropy, stop, candidate)
        self._check(self.lib.dg_denoise_step(self.ctx, _stream(), ctypes.byref(a)))

    def ar_step(self, reqs, tokens: torch.Tensor) -> torch.Tensor:
        """One greedy autoregressive step per request: appends the tokens'
        K/V rows and returns the next tokens (device int32 [n_req])."""
        assert tokens.dtype == torch.int32 and tokens.is_cuda and tokens.numel() == len(reqs)
        arr = (ctypes.c_int32 * len(reqs))(*reqs)
        nxt = torch.empty(len(reqs), dtype=torch.int32, device=tokens.device)
        self._check(self.lib.dg_ar_step(self.ctx, _stream(), len(reqs), arr, tokens.data_ptr(), nxt.data_ptr()))
        return nxt

    def commit_block(self, reqs, canvas):
        arr = (ctypes.c_int32 * len(reqs))(*reqs)
        self._check(self.lib.dg_commit_block(self.ctx, _stream(), len(reqs), arr, canvas.data_ptr()))

    def new_stats(self, n_req: int) -> torch.Tensor:
        return torch.zeros((n_req * self.cfg.canvas, B.ROW_STATS_BYTES // 4), dtype=torch.int32,
                           device=self.kv.device)

    # ------------------------------------------------------------------ per-stage timing
    def timing(self, enable: bool):
        self._check(self.lib.dg_timing_enable(self.ctx, int(enable)))

    def timing_read(self) -> Dict[str, tuple]:
        """{stage: (total ms, launches)} since the last read (waits for the GPU)."""
        n = len(B.STAGES)
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int32 * n)()
        self._check(self.lib.dg_timing_read(self.ctx, ms, cnt, n))
        return {name: (ms[i], cnt[i]) for i, name in enumerate(B.STAGES)}

    # ------------------------------------------------------------------ stage-level entry points
    def test_layer(self, req: int, layer: int, h: torch.Tensor, causal: bool):
        assert h.dtype == torch.float32 and h.is_cuda and h.is_contiguous()
        self._check(self.lib.dg_test_layer(self.ctx, _stream(), req, layer, h.data_ptr(),
                                           h.shape[0], int(causal)))

    def test_route(self, z: torch.Tensor):
        rows = z.shape[0]
        k, E = self.cfg.top_k, self.cfg.n_experts
        dev = z.device
        out = dict(idx=torch.empty((rows, k), dtype=torch.int32, device=dev),
                   w=torch.empty((rows, k), dtype=torch.float32, device=dev),
                   cnt=torch.empty(E, dtype=torch.int32, device=dev),
                   off=torch.empty(E + 1, dtype=torch.int32, device=dev),
                   perm=torch.empty(rows * k, dtype=torch.int32, device=dev),
                   slot=torch.empty((rows, k), dtype=torch.int32, device=dev))
        self._check(self.lib.dg_test_route(self.ctx, _stream(), z.data_ptr(), rows,
                                           *[out[n].data_ptr() for n in
                                             ("idx", "w", "cnt", "off", "perm", "slot")]))
        return out

    def test_forward(self, reqs, canvas, committed, step, n_steps, seeds, blocks, stats=None,
                     confidence: str = "prob", candidate: str = "argmax"):
        """dg_denoise_step, returning the residual stream after the embedding
        and after every layer (fp32 [n_layers + 1][rows][d]) and every
        layer's expert choices (int32 [n_layers][rows][top_k])."""
        c = self.cfg
        rows = len(reqs) * c.canvas
        dev = self.kv.device
        hs = torch.empty((c.n_layers + 1, rows, c.d_model), dtype=torch.float32, device=dev)
        idx = torch.empty((max(1, c.n_layers), rows, c.top_k), dtype=torch.int32, device=dev)
        a = self._args(reqs, canvas, committed, step, n_steps, seeds, blocks, stats, confidence, 0.0, None,
                       candidate)
        self._check(self.lib.dg_test_forward(self.ctx, _stream(), ctypes.byref(a), hs.data_ptr(),
                                             idx.data_ptr()))
        return hs, idx[:c.n_layers]

    def test_sample(self, reqs, stats_in: torch.Tensor, canvas, committed, step, n_steps, seeds, blocks,
                    stats=None, confidence: str = "prob", stop_entropy: float = 0.0, stop=None,
                    candidate: str = "argmax"):
        """The sampler alone, fed per-row statistics stats_in (int32 [rows][10]
        in the dg_row_stats layout)."""
        assert stats_in.is_cuda and stats_in.is_contiguous() and stats_in.dtype == torch.int32
        a = self._args(reqs, canvas, committed, step, n_steps, seeds, blocks, stats, confidence,
                       stop_entropy, stop, candidate)
        self._check(self.lib.dg_test_sample(self.ctx, _stream(), ctypes.byref(a), stats_in.data_ptr()))

    def test_attention(self, req: int, layer: int, q: torch.Tensor, causal: bool) -> torch.Tensor:
        """Attention of q (bf16 [n][Hq][dh], rotated) over cache rows
        [0, len + n) of (req, layer); returns bf16 [n][Hq*dh]."""
        assert q.dtype == torch.bfloat16 and q.is_cuda and q.is_contiguous()
        n = q.shape[0]
        o = torch.empty((n, self.cfg.n_q_heads * self.cfg.head_dim), dtype=torch.bfloat16, device=q.device)
        self._check(self.lib.dg_test_attention(self.ctx, _stream(), req, layer, q.data_ptr(), n, int(causal),
                                               o.data_ptr()))
        return o

    def test_head(self, reqs, h, canvas, committed, step, n_steps, seeds, blocks, stats=None,
                  confidence: str = "prob", stop_entropy: float = 0.0, stop=None, candidate: str = "argmax"):
        a = self._args(reqs, canvas, committed, step, n_steps, seeds, blocks, stats, confidence,
                       stop_entropy, stop, candidate)
        self._check(self.lib.dg_test_head(self.ctx, _stream(), ctypes.byref(a), h.data_ptr()))


def stats_tensor(max_logit, log_z, held_logit, argmax, entropy=None, sample=None, sample_logit=None):
    """Pack per-row statistics (host arrays) into an int32 [rows][10] CPU
    tensor in the dg_row_stats layout (floats stored as float32 bits)."""
    import numpy as np
    rows = len(max_logit)
    out = np.zeros((rows, B.ROW_STATS_BYTES // 4), np.int32)
    f = out.view(np.float32)
    f[:, 0] = np.asarray(max_logit, np.float32)
    f[:, 1] = np.asarray(log_z, np.float32)
    f[:, 2] = np.asarray(held_logit, np.float32)
    out[:, 4] = np.asarray(argmax, np.int32)
    if entropy is not None:
        f[:, 6] = np.asarray(entropy, np.float32)
    if sample is not None:
        out[:, 7] = np.asarray(sample, np.int32)
    if sample_logit is not None:
        f[:, 8] = np.asarray(sample_logit, np.float32)
    return torch.from_numpy(out)


def stats_fields(stats: torch.Tensor) -> Dict[str, torch.Tensor]:
    """Split a [rows][10] int32 dg_row_stats tensor into named CPU tensors."""
    s = stats.cpu()
    f = s.view(torch.float32)
    return dict(max_logit=f[:, 0], log_z=f[:, 1], held_logit=f[:, 2], conf=f[:, 3],
                argmax=s[:, 4], accepted=s[:, 5], entropy=f[:, 6], sample=s[:, 7], sample_logit=f[:, 8])


def gpu_weights(cfg: ModelConfig, model_seed: int = 0, gain_jitter: float = 0.0,
                device: str = "cuda"):
    """Generate a model's weights directly on the GPU (same bits as on the CPU)."""
    from . import synth
    layers = [synth.make_layer_weights(cfg, l, model_seed, device, gain_jitter)
              for l in range(cfg.n_layers)]
    embed = synth.make_embedding(cfg, model_seed, device)
    final = synth.make_final_norm(cfg, model_seed, device, gain_jitter)
    return layers, embed, final
