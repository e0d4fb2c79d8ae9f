#!/usr/bin/env python3
"""Benchmark: denoising steps of the full block-diffusion step on one MI355X.

A step is one pass of the whole hot path over one 256-token canvas: embedding,
30 layers (RMSNorm, QKV + RoPE, canvas attention over [prefix ; canvas],
output projection, router top-8 + permutation, grouped SwiGLU experts + the
shared expert, combine), final norm, LM head with fused vocabulary
statistics, and the confidence sampler. Inputs (weights, KV cache, canvas)
are resident in HBM before the timed region; weights are seeded random-init
bf16 with the workload's shapes.

Prints one JSON line (stdout). Progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "denoise steps/s + canvas tok/s (256-tok block), % HBM/MFMA roofline, 1 GPU"
HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # flop/s, dense bf16
PAGES_TPF = 19.74          # tokens per forward, codemajin.net explainer §5.3


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse_clocks(text):
    """rocm-smi --showclocks --json output -> {"card0": {"sclk": MHz, ...}}
    (every "<name> clock speed:" entry of each card; None when the text
    holds none)."""
    import re
    try:
        data = json.loads(text)
    except ValueError:
        return None
    out = {}
    for card, fields in data.items() if isinstance(data, dict) else ():
        if not isinstance(fields, dict):
            continue
        clk = {}
        for key, val in fields.items():
            m = re.match(r"\s*(\w+) clock speed", key)
            v = re.search(r"(\d+(?:\.\d+)?)\s*Mhz", str(val), re.IGNORECASE)
            if m and v:
                clk[m.group(1)] = float(v.group(1))
        if clk:
            out[card] = clk
    return out or None


def clocks_under_load(step, max_s=5.0):
    """The GPU clocks while the step runs back to back: rocm-smi runs as a
    child process and samples them while this process keeps launching
    steps (untimed). Best effort: None when rocm-smi is missing or fails."""
    import shutil
    import subprocess
    import torch
    exe = shutil.which("rocm-smi") or ("/opt/rocm/bin/rocm-smi" if os.path.exists("/opt/rocm/bin/rocm-smi") else None)
    if exe is None:
        return None
    try:
        proc = subprocess.Popen([exe, "--showclocks", "--json"], stdout=subprocess.PIPE,
                                stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None
    t0 = time.time()
    while proc.poll() is None and time.time() - t0 < max_s:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    try:
        text, _ = proc.communicate(timeout=max(1.0, max_s - (time.time() - t0)))
    except subprocess.TimeoutExpired:
        proc.kill()
        proc.communicate()
        return None
    return parse_clocks(text) if proc.returncode == 0 else None


def fp8_expert_bytes(cfg, touched_experts):
    """Algorithmic bytes of one expert-kernel launch with FP8 expert weights:
    one byte per weight plus a 4-byte scale per weight row, for the touched
    experts and the shared expert."""
    d, F, Fs = cfg.d_model, cfg.d_expert, cfg.d_shared
    return touched_experts * (3 * F * d + (2 * F + d) * 4) + 3 * Fs * d + (2 * Fs + d) * 4


def algorithmic_model(cfg, prefix, rows, touched_experts):
    """Bytes and flops per kernel class (per launch) that one denoising step
    must move / do.

    Weights: only the touched experts (the measured mean over the timed
    layers), plus attention, router, shared expert weights and the tied LM
    head, each read once; the prefix + canvas KV read once per layer;
    activations ignored (< 1% of the bytes).
    """
    d, E, F, Fs, V = cfg.d_model, cfg.n_experts, cfg.d_expert, cfg.d_shared, cfg.vocab
    L, Hq, Hkv, dh, k = cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.top_k
    nk = prefix + cfg.canvas
    kinds = {
        "qkv": (cfg.qkv_rows * d * 2, 2 * rows * cfg.qkv_rows * d),
        "attn": (nk * Hkv * dh * 2 * 2, 4 * rows * Hq * nk * dh),
        "oproj": (d * Hq * dh * 2, 2 * rows * d * Hq * dh),
        "router": (E * d * 2, 2 * rows * E * d),
        "experts": (touched_experts * 3 * F * d * 2 + 3 * Fs * d * 2,
                    2 * rows * k * 3 * F * d + 2 * rows * 3 * Fs * d),
    }
    per_step = {name: (b * L, f * L) for name, (b, f) in kinds.items()}
    per_step["lmhead"] = (V * d * 2, 2 * rows * V * d)
    return kinds, per_step


class _HostWeights:
    """Host copies of the GPU weights, one layer at a time, for the oracle."""

    def __init__(self, layers, embed, final_norm):
        self._layers, self.embed, self.final_norm = layers, embed.cpu(), final_norm.cpu()
        self._cache = {}

    def layer(self, i):
        if i not in self._cache:
            self._cache = {i: {k: v.cpu() for k, v in self._layers[i].items()}}
        return self._cache[i]


def cpu_baseline(eng, hw, cfg, canvas_ids, prefix, n_layers_sample, step, n_steps):
    """Time the float64 oracle on a bounded sample of the same step."""
    import numpy as np
    from oracle import model as om
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 0) for i in threadpool_info()), default=0)
    except Exception:
        blas_threads = 0
    cores = len(os.sched_getaffinity(0))
    req = om.Request(cfg, prefix + cfg.canvas)
    x = canvas_ids.astype(np.int64)
    t0 = time.perf_counter()
    h = om.f64(hw.embed[x])
    t_embed = time.perf_counter() - t0
    t_layers = 0.0
    for l in range(n_layers_sample):
        lw = hw.layer(l)
        k_rows, v_rows = eng.cache_rows(0, l, 0, prefix)
        ck = om.f64(k_rows.permute(1, 0, 2).cpu())
        cv = om.f64(v_rows.permute(1, 0, 2).cpu())
        t0 = time.perf_counter()
        h, _, _ = om.layer_forward(h, lw, cfg, ck, cv, prefix, False)
        t_layers += time.perf_counter() - t0
        log(f"cpu baseline: layer {l} {time.perf_counter() - t0:.2f}s")
    t0 = time.perf_counter()
    tau = om.tau_at(step, n_steps, cfg.tau_first, cfg.tau_last)
    Lg = om.logits(h, hw.final_norm, hw.embed, cfg)
    M, a, logZ, gx = om.row_stats(Lg, x, tau)
    om.sample(x, np.zeros_like(x, dtype=np.uint8), M, a, logZ, gx, tau, step, n_steps, 0, 0, 0,
              cfg.vocab)
    t_head = time.perf_counter() - t0
    log(f"cpu baseline: head {t_head:.2f}s")
    t_step = t_embed + t_layers * cfg.n_layers / n_layers_sample + t_head
    return {
        "value": 1.0 / t_step,
        "unit": "denoise steps/s",
        "cores": cores,
        "blas_threads": blas_threads,
        "kind": "oracle",
        "ms_per_step": t_step * 1e3,
        "sample": (f"float64 NumPy oracle: embedding + layers 0..{n_layers_sample - 1} of "
                   f"{cfg.n_layers} on all {cfg.canvas} canvas rows (timed "
                   f"{t_layers:.1f}s, scaled x{cfg.n_layers / n_layers_sample:g}) + full LM head over "
                   f"{cfg.vocab} ids + sampler (timed {t_head:.1f}s)"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="full", choices=["full", "long", "batch", "tiny", "one_layer"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=2)
    ap.add_argument("--n-req", type=int, default=0,
                    help="override the workload's number of requests (batch-size sweep; 0 = the workload's)")
    ap.add_argument("--no-fp8-variant", action="store_true",
                    help="skip the extra measurement with FP8 expert weights")
    ap.add_argument("--profile", action="store_true",
                    help="for hardware-counter runs: skip the block commit, so that every dispatch after the "
                         "canvas set-up (init_canvas_kernel) belongs to a denoising step; the prefill runs as "
                         "usual, so routing and attention see the same inputs as the headline run")
    ap.add_argument("--fp8-profile", action="store_true",
                    help="with --profile only: the headline engine reads FP8 expert and LM-head weights, so that "
                         "counter runs see the FP8 kernels on the headline's dispatches (never a headline number)")
    ap.add_argument("--no-variants", action="store_true",
                    help="measure the headline step only (no sampled-candidate, AR, FP8 or self-conditioning runs)")
    ap.add_argument("--no-selfcond-variant", action="store_true",
                    help="skip the extra measurement with self-conditioning")
    ap.add_argument("--graph-steps", type=int, default=50,
                    help="also time this many graph-launched steps (median reported; 0 = skip)")
    ap.add_argument("--copy-probe-mib", type=int, default=512,
                    help="after the run, copy this many MiB device-to-device with a plain copy "
                         "kernel (reference for hardware byte counters)")
    args = ap.parse_args()
    if args.fp8_profile and not args.profile:
        print("--fp8-profile is for counter runs and needs --profile", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the denoising step "
              "is measured on a single MI355X; multi-GPU sharding is not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_discrete_diffusion_dg_amd import synth
    from block_discrete_diffusion_dg_amd.engine import Engine, gpu_weights

    wl = synth.WORKLOADS[args.workload]
    cfg, P, S, n_req = wl.model, wl.prefix, wl.n_steps, args.n_req or wl.n_req
    C = cfg.canvas
    rows = n_req * C
    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(f"workload {wl.name}: L={cfg.n_layers} d={cfg.d_model} E={cfg.n_experts} V={cfg.vocab} "
        f"prefix={P} canvas={C} n_req={n_req}")
    t0 = time.time()
    layers, embed, final = gpu_weights(cfg, wl.seed, 0.0, dev)
    torch.cuda.synchronize()
    log(f"weights generated on the GPU in {time.time() - t0:.1f}s")
    fmt = {"expert_format": "fp8", "lmhead_format": "fp8"} if args.fp8_profile else {}
    eng = Engine(cfg, layers, embed, final, max_ctx=P + 2 * C, max_requests=n_req, max_rows=rows, **fmt)
    reqs = list(range(n_req))
    seeds = [wl.seed + r for r in reqs]
    blocks = [0] * n_req
    t0 = time.time()
    for r in reqs:
        eng.prefill(r, synth.make_prompt(P, cfg.vocab, wl.seed, r, device=dev))
    torch.cuda.synchronize()
    log(f"prefill of {n_req} x {P} tokens: {time.time() - t0:.2f}s")
    x = torch.empty(rows, dtype=torch.int32, device=dev)
    m = torch.empty(rows, dtype=torch.uint8, device=dev)
    eng.init_canvas(reqs, x, m, seeds, blocks)
    canvas0 = x.cpu().numpy()

    def run(n, start):
        for i in range(n):
            s = (start + i) % S + 1
            eng.denoise_step(reqs, x, m, s, S, seeds, blocks)

    run(args.warmup, 0)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")
    moe0 = eng.moe_counters()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    run(args.steps, args.warmup)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / args.steps
    log(f"timed {args.steps} steps: {ms:.3f} ms/step (events), wall {wall * 1e3 / args.steps:.3f} ms/step")
    moe1 = eng.moe_counters()
    if moe1["spin_timeouts"] != moe0["spin_timeouts"]:
        raise RuntimeError("expert kernel waits ran out during the timed steps")
    touched = (moe1["touched_total"] - moe0["touched_total"]) / max(1, moe1["permute_calls"] - moe0["permute_calls"])

    # per-stage durations: a second pass with per-launch events on the same stream
    eng.timing(True)
    moe2 = eng.moe_counters()
    run(args.steps, args.warmup + args.steps)
    stages = eng.timing_read()
    moe3 = eng.moe_counters()
    # mean touched experts per layer over the launches the stage timing covers
    touched_staged = (moe3["touched_total"] - moe2["touched_total"]) / max(
        1, moe3["permute_calls"] - moe2["permute_calls"])
    eng.timing(False)
    stage_ms = {k: v[0] / args.steps for k, v in stages.items() if v[1]}
    launches = {k: v[1] // args.steps for k, v in stages.items() if v[1]}
    log("stage ms/step: " + ", ".join(f"{k}={v:.3f}" for k, v in stage_ms.items()))

    # graph-launched steps: median of --graph-steps replays
    graph = None
    if args.graph_steps:
        moe_g0 = eng.moe_counters()
        times = graph_timing(eng, reqs, x, m, S, seeds, blocks, args.warmup, args.graph_steps)
        eng.sync()
        if times is not None:
            t = np.sort(np.array(times))
            graph = {"median_ms": round(float(np.median(t)), 4), "p10_ms": round(float(t[len(t) // 10]), 4),
                     "p90_ms": round(float(t[(9 * len(t)) // 10]), 4), "steps": len(t),
                     "steps_per_s_median": round(1e3 / float(np.median(t)), 3)}
            log(f"graph-launched: median {graph['median_ms']:.3f} ms/step over {len(t)} replays")
        if eng.moe_counters()["spin_timeouts"] != moe_g0["spin_timeouts"]:
            raise RuntimeError("expert kernel waits ran out during the graph-launched steps")

    # the engine and memory clocks while steps run back to back (rocm-smi)
    clocks = None
    if not args.profile:
        n_clk = [0]

        def one_step():
            run(1, n_clk[0])
            n_clk[0] += 1
        clocks = clocks_under_load(one_step)
        log(f"clocks under load: {clocks}")

    # commit (the +K-1 forward of each block), timed once, then the length restored
    commit_ms = None
    if not args.profile:
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        eng.commit_block(reqs, x)
        c1.record(stream)
        torch.cuda.synchronize()
        commit_ms = c0.elapsed_time(c1)
        for r in reqs:
            eng.set_cache_len(r, P)

    kinds, per_step = algorithmic_model(cfg, P, rows, touched)
    t_roof = sum(max(b / HBM_PEAK, f / MFMA_BF16_PEAK) for b, f in per_step.values())
    b_ex, f_ex = algorithmic_model(cfg, P, rows, touched_staged)[0]["experts"]
    # measured HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a
    # plain copy), only while the kernel's sources match the recorded hash
    from block_discrete_diffusion_dg_amd.profiles import traffic_for
    # the counter records are taken on the workloads as defined (a request
    # count given on the command line is another workload: no record)
    rec_stem = wl.name if not args.n_req or args.n_req == wl.n_req else None
    traffic = traffic_for("moe_experts", f"moe_experts_{rec_stem}_traffic") if rec_stem else None
    traffic = round(traffic) if traffic is not None else None
    ex_launch_ms = stages["experts"][0] / max(1, stages["experts"][1])
    achieved = b_ex / (ex_launch_ms * 1e-3)
    # every kernel class against its own roof: algorithmic bytes and flops per
    # launch over the launch's measured duration
    kinds_staged = dict(algorithmic_model(cfg, P, rows, touched_staged)[0])
    kinds_staged["lmhead"] = per_step["lmhead"]
    kernels = {}
    for name, (b, f) in kinds_staged.items():
        if name not in stages or not stages[name][1]:
            continue
        t = stages[name][0] / stages[name][1] * 1e-3
        hbm = b / HBM_PEAK >= f / MFMA_BF16_PEAK
        kernels[name] = {"bound": "hbm" if hbm else "mfma",
                         "achieved": round((b / t / 1e9) if hbm else (f / t / 1e12), 1),
                         "unit": "GB/s" if hbm else "TFLOP/s",
                         "peak": HBM_PEAK / 1e9 if hbm else MFMA_BF16_PEAK / 1e12,
                         "frac": round(max(b / HBM_PEAK, f / MFMA_BF16_PEAK) / t, 4),
                         "bytes_per_launch": round(b), "flops_per_launch": round(f),
                         "avg_launch_ms": round(t * 1e3, 4)}
    lm_traffic = traffic_for("lmhead", f"lmhead_{rec_stem}_traffic") if rec_stem else None
    if "lmhead" in kernels:
        kernels["lmhead"]["traffic"] = round(lm_traffic) if lm_traffic is not None else None
    attn_traffic = traffic_for("attn", f"attn_{rec_stem}_traffic") if rec_stem else None
    if "attn" in kernels:
        kernels["attn"]["traffic"] = round(attn_traffic) if attn_traffic is not None else None
    steps_per_s = 1e3 / ms
    out = {
        "metric": METRIC,
        "value": round(steps_per_s, 3),
        "unit": "denoise steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if not args.fp8_profile else "bf16 (fp8 expert and LM-head weights, counter run)",
        "data": "synthetic: seeded random-init bf16 weights, uniform prompt ids (no datasets or checkpoints)",
        "config": {"workload": wl.name, "layers": cfg.n_layers, "d_model": cfg.d_model,
                   "experts": f"{cfg.n_experts} routed top-{cfg.top_k} + 1 shared",
                   "vocab": cfg.vocab, "prefix": P, "canvas": C, "n_req": n_req,
                   "denoise_steps_per_block": S},
        "canvas_tok_s": round(steps_per_s * rows, 1),
        "effective_tok_s": {"tpf_pages_19.74": round(steps_per_s * PAGES_TPF * n_req, 1),
                            f"tpf_loop_{C / S:g}": round(steps_per_s * C / S * n_req, 1)},
        "step_roofline": {"t_roof_ms": round(t_roof * 1e3, 4), "frac": round(t_roof * 1e3 / ms, 4),
                          "touched_experts_per_layer": round(touched, 2)},
        "roofline": {"kernel": "moe_experts (routed + shared experts: gate/up + SwiGLU + down)",
                     "bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK, 4),
                     "bytes_per_launch": round(b_ex), "avg_launch_ms": round(ex_launch_ms, 4),
                     "traffic": traffic},
        "kernel_rooflines": kernels,
        "stages_ms_per_step": {k: round(v, 4) for k, v in stage_ms.items()},
        "launches_per_step": launches,
        "commit_ms": round(commit_ms, 3) if commit_ms is not None else None,
        "graph_launched": graph,
        "clocks_mhz": clocks,
    }
    if not args.no_cpu_baseline and args.workload in ("full", "one_layer", "tiny"):
        hw = _HostWeights(layers, embed, final)
        log("cpu baseline: timing the oracle on a sample of the step")
        out["cpu_baseline"] = cpu_baseline(eng, hw, cfg, canvas0[:C], P,
                                           min(args.cpu_layers, cfg.n_layers), 1, S)
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record(stream)
        dst.copy_(src)
        p1.record(stream)
        torch.cuda.synchronize()
        copy_gbs = 2 * n / (p0.elapsed_time(p1) * 1e-3) / 1e9
        out["copy_probe"] = {"bytes_read": n, "bytes_written": n, "ms": round(p0.elapsed_time(p1), 4),
                             "GB_s_read_plus_write": round(copy_gbs, 1)}
        # the dominant kernel also against the HBM rate a plain device copy
        # reaches on this GPU in the same run
        out["roofline"]["peak_measured"] = round(copy_gbs, 1)
        out["roofline"]["frac_measured"] = round(out["roofline"]["achieved"] / copy_gbs, 4)
    if args.workload == "full" and not args.n_req and not args.no_variants:
        out["variants"] = {"sampled_candidates": sampled_variant(args, eng, reqs, seeds, blocks, x, m, S),
                           "ar_step": ar_variant(args, eng, reqs, P, ms)}
        if not args.no_fp8_variant:
            out["variants"]["fp8_experts"] = fp8_variant(args, cfg, wl, layers, embed, final, reqs, seeds,
                                                         blocks, canvas0, dev)
        if not args.no_selfcond_variant:
            out["variants"]["self_conditioning"] = selfcond_variant(args, cfg, wl, layers, embed, final, reqs,
                                                                    seeds, blocks, canvas0, dev)
    # every launch on the headline engine (timed, staged, graph-launched,
    # commit and the variants that reuse it) ran with no expert-kernel wait
    # running out, or this raises
    eng.sync()
    print(json.dumps(out), flush=True)


def graph_timing(eng, reqs, x, m, S, seeds, blocks, n_warm, n_timed):
    """Graph-launched steps: one HIP graph per step index s = 1..S (the
    step's temperature and commit count are launch arguments, fixed at
    capture), replayed in block order on the canvas, each replay timed with
    its own pair of events on the replay stream. Returns the per-step
    durations in ms (after n_warm untimed replays), or None when capture is
    not available."""
    import torch
    x0, m0 = x.clone(), m.clone()
    graphs = []
    try:
        for s in range(1, S + 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                eng.denoise_step(reqs, x, m, s, S, seeds, blocks)
            graphs.append(g)
    except Exception as e:  # capture unsupported: report eager timing only
        log(f"graph capture failed: {e}")
        return None
    x.copy_(x0)
    m.copy_(m0)
    stream = torch.cuda.current_stream()
    for i in range(n_warm):
        graphs[i % S].replay()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_timed)]
    torch.cuda.synchronize()
    for i in range(n_timed):
        ev[i][0].record(stream)
        graphs[(n_warm + i) % S].replay()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def ar_variant(args, eng, reqs, P, denoise_ms):
    """Greedy autoregressive decode steps (one token per request, causal pass
    plus a one-row LM head) at the same prefix: the explainer's §5.2 compares
    a denoising step with one such step (3.2x on its hardware)."""
    import torch
    tok = torch.zeros(len(reqs), dtype=torch.int32, device=f"cuda:{torch.cuda.current_device()}")
    for _ in range(args.warmup):
        tok = eng.ar_step(reqs, tok)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        tok = eng.ar_step(reqs, tok)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    eng.sync()  # raises if a bounded wait of the expert kernel ran out
    for r in reqs:
        eng.set_cache_len(r, P)
    log(f"ar step: {ms:.3f} ms")
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(1e3 / ms * len(reqs), 1),
            "denoise_over_ar": round(denoise_ms / ms, 3)}


def sampled_variant(args, eng, reqs, seeds, blocks, x, m, S):
    """The same step with sampled candidates (Gumbel-max over the vocabulary
    in the LM-head epilogue) instead of the argmax: the cost of the draw."""
    import torch

    def run(n, start):
        for i in range(n):
            eng.denoise_step(reqs, x, m, (start + i) % S + 1, S, seeds, blocks, candidate="sample")

    run(args.warmup, 0)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    run(args.steps, args.warmup)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    eng.timing(True)
    run(args.steps, args.warmup + args.steps)
    stages = eng.timing_read()
    eng.timing(False)
    eng.sync()  # raises if a bounded wait of the expert kernel ran out
    log(f"sampled candidates: {ms:.3f} ms/step")
    return {"ms_per_step": round(ms, 4), "steps_per_s": round(1e3 / ms, 3),
            "lmhead_ms": round(stages["lmhead"][0] / max(1, stages["lmhead"][1]), 4),
            "merge_ms": round(stages["merge"][0] / max(1, stages["merge"][1]), 4)}


def selfcond_variant(args, cfg, wl, layers, embed, final, reqs, seeds, blocks, canvas0, dev):
    """The same step with self-conditioning (explainer §3.2): each step's
    predicted distribution softmax(L) over the whole vocabulary, contracted
    with the tied embedding and passed through a SwiGLU feed-forward layer of
    width d_expert, is added to the next step's input embeddings. The pages
    time it inside their "sampling" stage (explainer §5.2)."""
    import torch
    from block_discrete_diffusion_dg_amd import synth
    from block_discrete_diffusion_dg_amd.engine import Engine
    P, S, C = wl.prefix, wl.n_steps, cfg.canvas
    rows = len(reqs) * C
    sc = synth.make_selfcond_weights(cfg, cfg.d_expert, wl.seed, dev)
    eng = Engine(cfg, layers, embed, final, max_ctx=P + 2 * C, max_requests=len(reqs), max_rows=rows,
                 selfcond=sc)
    for r in reqs:
        eng.prefill(r, synth.make_prompt(P, cfg.vocab, wl.seed, r, device=dev))
    x = torch.from_numpy(canvas0).to(dev)
    m = torch.zeros(rows, dtype=torch.uint8, device=dev)

    def run(n, start):
        for i in range(n):
            eng.denoise_step(reqs, x, m, (start + i) % S + 1, S, seeds, blocks)

    run(args.warmup, 0)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    run(args.steps, args.warmup)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    eng.timing(True)
    run(args.steps, args.warmup + args.steps)
    stages = eng.timing_read()
    eng.timing(False)
    eng.sync()
    log(f"self-conditioning: {ms:.3f} ms/step, signal {stages['selfcond'][0] / args.steps:.3f} ms/step")
    eng.close()
    return {"ms_per_step": round(ms, 4), "steps_per_s": round(1e3 / ms, 3),
            "canvas_tok_s": round(1e3 / ms * rows, 1), "width": cfg.d_expert,
            "selfcond_ms_per_step": round(stages["selfcond"][0] / args.steps, 4),
            "lmhead_ms_per_step": round(stages["lmhead"][0] / args.steps, 4)}


def fp8_variant(args, cfg, wl, layers, embed, final, reqs, seeds, blocks, canvas0, dev):
    """The same step with the expert matrices and the LM head's copy of the
    embedding stored as FP8 (E4M3 codes and power-of-two row scales,
    quantised on the GPU from the same bf16 weights): a separate variant at
    reduced weight precision, reported beside the bf16 headline, never in its
    place."""
    import torch
    from block_discrete_diffusion_dg_amd import synth
    from block_discrete_diffusion_dg_amd.engine import Engine
    P, S, C = wl.prefix, wl.n_steps, cfg.canvas
    rows = len(reqs) * C
    eng = Engine(cfg, layers, embed, final, max_ctx=P + 2 * C, max_requests=len(reqs), max_rows=rows,
                 expert_format="fp8", lmhead_format="fp8")
    for r in reqs:
        eng.prefill(r, synth.make_prompt(P, cfg.vocab, wl.seed, r, device=dev))
    x = torch.from_numpy(canvas0).to(dev)
    m = torch.zeros(rows, dtype=torch.uint8, device=dev)

    def run(n, start):
        for i in range(n):
            eng.denoise_step(reqs, x, m, (start + i) % S + 1, S, seeds, blocks)

    run(args.warmup, 0)
    moe0 = eng.moe_counters()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    run(args.steps, args.warmup)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    eng.timing(True)
    moe1 = eng.moe_counters()
    run(args.steps, args.warmup + args.steps)
    stages = eng.timing_read()
    moe2 = eng.moe_counters()
    eng.timing(False)
    if moe2["spin_timeouts"] != moe0["spin_timeouts"]:
        raise RuntimeError("expert kernel waits ran out during the FP8 steps")
    touched = (moe2["touched_total"] - moe1["touched_total"]) / max(1, moe2["permute_calls"] - moe1["permute_calls"])
    ex_ms = stages["experts"][0] / max(1, stages["experts"][1])
    b = fp8_expert_bytes(cfg, touched)
    log(f"fp8 experts: {ms:.3f} ms/step, expert launch {ex_ms * 1e3:.1f} us")
    eng.close()
    from block_discrete_diffusion_dg_amd.profiles import traffic_for
    traffic = traffic_for("moe_experts", f"moe_experts_fp8_{wl.name}_traffic")
    return {"ms_per_step": round(ms, 4), "steps_per_s": round(1e3 / ms, 3),
            "canvas_tok_s": round(1e3 / ms * rows, 1),
            "weights": ("expert matrices and the LM head's copy of the embedding E4M3 + per-row power-of-two "
                        "scales; everything else bf16"),
            "lmhead_kernel": {"bound": "hbm", "bytes_per_launch": cfg.vocab * cfg.d_model + cfg.vocab * 4,
                              "avg_launch_ms": round(stages["lmhead"][0] / max(1, stages["lmhead"][1]), 4)},
            "experts_kernel": {"bound": "hbm", "bytes_per_launch": round(b), "avg_launch_ms": round(ex_ms, 4),
                               "achieved": round(b / (ex_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                               "peak": HBM_PEAK / 1e9, "frac": round(b / (ex_ms * 1e-3) / HBM_PEAK, 4),
                               "touched_experts_per_layer": round(touched, 2),
                               "traffic": round(traffic) if traffic is not None else None},
            "stages_ms_per_step": {k: round(v[0] / args.steps, 4) for k, v in stages.items() if v[1]}}


if __name__ == "__main__":
    main()
