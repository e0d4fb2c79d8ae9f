"""GPU-vs-oracle parity of each stage of the denoising step, through the C ABI.

Integer outputs (router indices, permutation, argmax, accepted set, re-noised
ids) must match bit for bit when both sides see the same float inputs; a
swap is tolerated only where the oracle's own keys are tied within a stated
band. Floating-point outputs must satisfy max|gpu - oracle| / max|oracle| <=
2e-2 (bf16 operands, fp32 accumulation), or the tighter bound stated where
both sides start from the same bf16 operands.
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_discrete_diffusion_dg_amd import synth
from block_discrete_diffusion_dg_amd.engine import Engine, stats_fields
from oracle import model as om
from oracle.philox import uniform_ids
from tests.gpu_util import (REL_TOL, HostWeights, elem_stats, fmt_elem, make_engine, make_selfcond, max_rel,
                            moe_with_experts, router_band, router_swaps, say, tie_gap_ok)

pytestmark = pytest.mark.gpu


def _zero_layer_engine(cfg, max_rows, max_requests=1, lmhead_format="bf16"):
    cfg0 = dataclasses.replace(cfg, n_layers=0)
    return make_engine(cfg0, max_ctx=4 * cfg.canvas, max_requests=max_requests, max_rows=max_rows,
                       lmhead_format=lmhead_format)


# ------------------------------------------------------------------------ generator

def test_synth_generator_identical_on_gpu_and_cpu():
    for shape, seed in [((1000, 37), 5), ((3, 704, 256), 77)]:
        a = synth.hashed_normal(shape, seed, 0.02, "cpu")
        b = synth.hashed_normal(shape, seed, 0.02, "cuda").cpu()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(synth.make_prompt(999, 262144, 3), synth.make_prompt(999, 262144, 3, device="cuda").cpu())


# ------------------------------------------------------------------------ weight layout

def _fragment_major_reference(w):
    """The packed layout by axis permutation: W[16nb + r][64ks + 32q + 8g + e]
    goes to position (nb, ks, q, g, r, e)."""
    n, k = w.shape
    t = w.reshape(n // 16, 16, k // 64, 2, 4, 8)          # nb, r, ks, q, g, e
    return np.ascontiguousarray(t.transpose(0, 2, 3, 4, 1, 5)).reshape(n, k)


@pytest.mark.parametrize("shape", [(16, 64), (48, 192), (3 * 704, 256), (4096, 2048)])
def test_pack_weight_bit_exact(shape):
    from block_discrete_diffusion_dg_amd.engine import pack_weight
    say(f"[pack] shape={shape}")
    w = synth.hashed_normal(shape, 11 + shape[0], 0.02, "cuda")
    got = pack_weight(w).cpu().view(torch.int16).numpy()
    ref = _fragment_major_reference(w.cpu().view(torch.int16).numpy())
    assert np.array_equal(got, ref)
    # spot-check the index formula of the header on a few elements
    n, k = shape
    wc = w.cpu().view(torch.int16).numpy()
    for i, j in [(0, 0), (n - 1, k - 1), (17 % n, 33 % k), (n // 2, 63 % k)]:
        idx = (i // 16) * 16 * k + (j // 64) * 1024 + ((j % 64) // 32) * 512 + \
            (((j % 32) // 8) * 16 + i % 16) * 8 + j % 8
        assert got.reshape(-1)[idx] == wc[i, j]


# ------------------------------------------------------------------------ router

def _router_logits(rows, E, seed):
    z = synth.hashed_normal((rows, E), synth.tensor_seed(seed, 0, "z"), 1.0, dtype=torch.float32)
    z = z.clone()
    if rows > 2:
        z[0, 5] = z[0, 3] = 9.0       # exact tie at the top: lower id first
        z[1, :] = 0.25                 # all tied: experts 0..k-1
        z[2, E - 1] = z[2, E - 2] = z[2, 0] = -9.0
    return z


# 5003 and 8192 rows exceed the permutation's LDS tables (2368 rows of 128
# experts) and take its chunked form; 8192 rows is 32 requests of one block.
@pytest.mark.parametrize("model,rows", [(synth.TINY, 32), (synth.TINY, 37), (synth.FULL, 256),
                                        (synth.FULL, 2048), (synth.FULL, 5), (synth.FULL, 5003),
                                        (synth.FULL, 8192)])
def test_route_bit_exact(model, rows):
    say(f"[route] E={model.n_experts} k={model.top_k} rows={rows}")
    eng, _ = _zero_layer_engine(model, max_rows=max(rows, model.canvas))
    z = _router_logits(rows, model.n_experts, rows)
    c0 = eng.moe_counters()
    out = eng.test_route(z.cuda())
    torch.cuda.synchronize()
    c1 = eng.moe_counters()
    idx, w = om.route(z.double().numpy(), model.top_k)
    cnt, off, perm, slot = om.permutation(idx, model.n_experts)
    # running statistics: one call, touching exactly the experts with rows
    assert c1["permute_calls"] - c0["permute_calls"] == 1
    assert c1["touched_total"] - c0["touched_total"] == int((cnt > 0).sum())
    assert np.array_equal(out["idx"].cpu().numpy(), idx)
    assert np.abs(out["w"].cpu().double().numpy() - w).max() < 2e-6
    assert np.array_equal(out["cnt"].cpu().numpy(), cnt)
    assert np.array_equal(out["off"].cpu().numpy(), off)
    assert np.array_equal(out["perm"].cpu().numpy(), perm)
    assert np.array_equal(out["slot"].cpu().numpy(), slot)


# ------------------------------------------------------------------------ FP8 weights

def _unpack8(codes, n, k):
    """Row-major [n][k] view of FP8 fragment-major bytes (the layout dg.h
    documents for dg_quantize_fp8)."""
    nn, kk = np.meshgrid(np.arange(n), np.arange(k), indexing="ij")
    idx = ((nn >> 4) * 16 * k + (kk >> 6) * 1024 + (((kk & 31) >> 3) * 16 + (nn & 15)) * 16
           + ((kk & 63) >> 5) * 8 + (kk & 7))
    return codes[idx]


@pytest.mark.parametrize("which", ["tiny_bank", "full_down", "edges"])
def test_quantize_fp8_bit_exact(which):
    from block_discrete_diffusion_dg_amd.engine import quantize_fp8
    from oracle import fp8
    say(f"[fp8] quantize {which}")
    if which == "tiny_bank":
        w = synth.make_layer_weights(synth.TINY, 0, 7)["w_gate"]  # [E][F][d]
    elif which == "full_down":
        w = synth.make_layer_weights(dataclasses.replace(synth.FULL, n_experts=2), 0, 7)["w_down"][1]
    else:
        # a zero row, rows whose maximum sits exactly on 448 * 2^e or just
        # above it, tiny rows (subnormal codes), negative zeros, ties
        rng = np.random.default_rng(3)
        w = rng.standard_normal((64, 128)).astype(np.float32) * 0.02
        w[0] = 0.0
        w[1, 5] = 448.0
        w[2, 7] = -448.0 * 2.0 ** -10
        w[3, 9] = 449.0
        w[4] = rng.standard_normal(128) * 1e-6
        w[5, :8] = -0.0
        w[6, 0] = 448.0
        w[6, 1:9] = [1 + 1 / 16, 1 + 3 / 16, 2.0 ** -8 * 1.5, 300.0, 432.0, -432.0, 2.0 ** -9 * 0.5, 7.5]
        w = torch.from_numpy(w).to(torch.bfloat16)
    w2 = w.reshape(-1, w.shape[-1]).contiguous()
    n, k = w2.shape
    codes, scale = quantize_fp8(w2.cuda())
    torch.cuda.synchronize()
    codes = _unpack8(codes.cpu().numpy(), n, k)
    want_codes, want_e = fp8.quantize_rows(om.f64(w2))
    assert np.array_equal(scale.cpu().double().numpy(), np.exp2(want_e.astype(np.float64)))
    assert np.array_equal(codes, want_codes)


def _unpack_lm8(codes, n, k):
    """Row-major [n][k] view of the LM head's step-major FP8 bytes (the
    layout dg.h documents for dg_quantize_fp8_lmhead)."""
    nn, kk = np.meshgrid(np.arange(n), np.arange(k), indexing="ij")
    idx = (kk >> 5) * n * 32 + (nn >> 4) * 512 + (((kk & 31) >> 3) * 16 + (nn & 15)) * 8 + (kk & 7)
    return codes[idx]


@pytest.mark.parametrize("which", ["tiny_embed", "edges"])
def test_quantize_fp8_lmhead_bit_exact(which):
    from block_discrete_diffusion_dg_amd.engine import quantize_fp8
    from oracle import fp8
    say(f"[fp8 lm] quantize {which}")
    if which == "tiny_embed":
        w = synth.make_embedding(synth.TINY, 0)
    else:
        rng = np.random.default_rng(5)
        w = rng.standard_normal((48, 192)).astype(np.float32) * 0.02
        w[0] = 0.0
        w[1, 3] = 448.0
        w[2, 70] = -449.0
        w[3] = rng.standard_normal(192) * 1e-6
        w = torch.from_numpy(w).to(torch.bfloat16)
    n, k = w.shape
    codes, scale = quantize_fp8(w.contiguous().cuda(), lmhead=True)
    torch.cuda.synchronize()
    want_codes, want_e = fp8.quantize_rows(om.f64(w))
    assert np.array_equal(scale.cpu().double().numpy(), np.exp2(want_e.astype(np.float64)))
    assert np.array_equal(_unpack_lm8(codes.cpu().numpy(), n, k), want_codes)


# ------------------------------------------------------------------------ LM head + sampler

def _head_case(model, n_req, step, n_steps, seed=3):
    C = model.canvas
    rows = n_req * C
    h = synth.make_hidden(rows, model.d_model, seed)
    canvas = synth.hashed_uniform_ids(rows, synth.tensor_seed(seed, 1, "canvas"), model.vocab)
    committed = (synth.hashed_uniform_ids(rows, synth.tensor_seed(seed, 2, "m"), 2) == 1).to(torch.uint8)
    return h, canvas, committed


# The FP8 case at full width uses 16,384 vocabulary rows: the tile is the
# full model's (K = 2048), and the oracle's dequantisation of all 262,144
# rows would take minutes.
@pytest.mark.parametrize("model,n_req,lm", [(synth.TINY, 1, "bf16"), (synth.TINY, 3, "bf16"), (synth.FULL, 1, "bf16"),
                                           (synth.TINY, 2, "fp8"),
                                           (dataclasses.replace(synth.FULL, vocab=16384), 1, "fp8")])
def test_head_statistics_and_sampler(model, n_req, lm):
    """With lm "fp8" the LM head reads E4M3 codes of the embedding; the oracle
    multiplies with its own dequantisation of the same bf16 embedding."""
    say(f"[head] V={model.vocab} d={model.d_model} n_req={n_req} lmhead={lm}")
    C = model.canvas
    rows = n_req * C
    eng, hw = _zero_layer_engine(model, max_rows=rows, max_requests=n_req, lmhead_format=lm)
    if lm == "fp8":
        from oracle import fp8
        hw = HostWeights([], torch.from_numpy(fp8.dequantize_bank(om.f64(hw.embed))), hw.final_norm)
    step, n_steps = 5, 16
    h, canvas, committed = _head_case(model, n_req, step, n_steps)
    reqs = list(range(n_req))
    seeds = [11 + r for r in reqs]
    blocks = [2] * n_req
    x_dev, m_dev = canvas.cuda(), committed.cuda()
    stats = eng.new_stats(n_req)
    eng.test_head(reqs, h.cuda(), x_dev, m_dev, step, n_steps, seeds, blocks, stats)
    torch.cuda.synchronize()
    st = stats_fields(stats)
    u_gpu = eng.ws_view("u", torch.bfloat16, (rows, model.d_model)).cpu()
    tau = om.tau_at(step, n_steps, model.tau_first, model.tau_last)
    x_np, m_np = canvas.numpy().astype(np.int64), committed.numpy()

    # (1) same bf16 operand on both sides: logits agree to fp32 rounding
    L_u = om.f64(u_gpu) @ om.f64(hw.embed).T
    M1, a1, logZ1, gx1 = om.row_stats(L_u, x_np, tau)
    scale = np.abs(L_u).max()
    assert np.abs(st["max_logit"].double().numpy() - M1).max() < 1e-5 * scale
    assert np.abs(st["held_logit"].double().numpy() - gx1).max() < 1e-5 * scale
    assert np.abs(st["log_z"].double().numpy() - logZ1).max() < 1e-4
    H1 = om.row_entropy(L_u, tau)
    assert np.abs(st["entropy"].double().numpy() - H1).max() < 1e-4 * max(1.0, H1.max())
    top2 = np.sort(L_u, axis=1)[:, -2:]
    clear = (top2[:, 1] - top2[:, 0]) > 1e-5 * scale
    assert np.array_equal(st["argmax"].numpy()[clear], a1[clear])
    assert np.all(L_u[np.arange(rows), st["argmax"].numpy()] >= M1 - 1e-5 * scale)

    # (2) from the residual stream: the float64 oracle end to end
    L = om.logits(h.double().numpy(), hw.final_norm, hw.embed, model)
    M, a, logZ, gx = om.row_stats(L, x_np, tau)
    big = np.abs(L).max()
    assert max_rel(st["max_logit"], M) <= REL_TOL
    assert np.abs((st["max_logit"].double().numpy() / tau + st["log_z"].double().numpy())
                  - (M / tau + logZ)).max() <= REL_TOL * big / tau
    assert np.all(L[np.arange(rows), st["argmax"].numpy()] >= M - REL_TOL * big)
    assert np.abs(st["entropy"].double().numpy() - om.row_entropy(L, tau)).max() <= REL_TOL * big / tau

    # (3) sampler: the oracle's sampler on the GPU's own statistics, per request
    x_new = x_dev.cpu().numpy()
    m_new = m_dev.cpu().numpy()
    for r in reqs:
        sl = slice(r * C, (r + 1) * C)
        xo, mo, c, acc = om.sample(x_np[sl], m_np[sl], st["max_logit"].double().numpy()[sl],
                                   st["argmax"].numpy()[sl], st["log_z"].double().numpy()[sl],
                                   st["held_logit"].double().numpy()[sl], tau, step, n_steps,
                                   seeds[r], blocks[r], r, model.vocab)
        assert np.abs(st["conf"].double().numpy()[sl] - c).max() < 1e-4
        k_s = om.commit_count(step, n_steps, C)
        acc_gpu = st["accepted"].numpy()[sl].astype(bool)
        assert acc_gpu.sum() == k_s and np.array_equal(m_new[sl].astype(bool), acc_gpu)
        if tie_gap_ok(c, k_s, 1e-4):
            assert np.array_equal(acc_gpu, acc)
            assert np.array_equal(x_new[sl], xo)
        noise = uniform_ids(seeds[r], np.arange(C), step, blocks[r], r, model.vocab)
        assert np.array_equal(x_new[sl][~acc_gpu], noise[~acc_gpu])


@pytest.mark.parametrize("model,n_req", [(synth.TINY, 2), (synth.FULL, 1)])
def test_entropy_confidence_and_adaptive_stop(model, n_req):
    """Entropy ranking on the GPU's own statistics matches the oracle's
    sampler bit for bit; the stop fires only when the previous step of the
    same block had the same argmax everywhere and the mean entropy is below
    the threshold, and a stopped step accepts every position."""
    say(f"[entropy] V={model.vocab} n_req={n_req}")
    C = model.canvas
    rows = n_req * C
    eng, hw = _zero_layer_engine(model, max_rows=rows, max_requests=n_req)
    step, n_steps = 3, 8
    h, canvas, committed = _head_case(model, n_req, step, n_steps, seed=5)
    h = h.cuda()
    reqs = list(range(n_req))
    seeds, blocks = [21 + r for r in reqs], [1] * n_req
    tau = om.tau_at(step, n_steps, model.tau_first, model.tau_last)
    x_np, m_np = canvas.numpy().astype(np.int64), committed.numpy()
    stop = torch.full((n_req,), -7, dtype=torch.int32, device="cuda")

    def run(thr):
        x_dev, m_dev = canvas.cuda(), committed.cuda()
        stats = eng.new_stats(n_req)
        eng.test_head(reqs, h, x_dev, m_dev, step, n_steps, seeds, blocks, stats, confidence="entropy",
                      stop_entropy=thr, stop=stop)
        torch.cuda.synchronize()
        return x_dev.cpu().numpy(), m_dev.cpu().numpy(), stats_fields(stats), stop.cpu().numpy().copy()

    # first step of the block: no previous argmax, never stops
    x1, m1, st, stop1 = run(1e9)
    assert np.array_equal(stop1, np.zeros(n_req))
    H = st["entropy"].double().numpy()
    k_s = om.commit_count(step, n_steps, C)
    for r in reqs:
        sl = slice(r * C, (r + 1) * C)
        xo, mo, c, acc = om.sample(x_np[sl], m_np[sl], st["max_logit"].double().numpy()[sl],
                                   st["argmax"].numpy()[sl], st["log_z"].double().numpy()[sl],
                                   st["held_logit"].double().numpy()[sl], tau, step, n_steps, seeds[r],
                                   blocks[r], r, model.vocab, confidence="entropy", H=H[sl])
        assert np.array_equal(st["conf"].double().numpy()[sl], c)
        assert np.array_equal(st["accepted"].numpy()[sl].astype(bool), acc)
        assert np.array_equal(x1[sl], xo) and np.array_equal(m1[sl], mo) and mo.sum() == k_s
    mean_h = H.reshape(n_req, C).astype(np.float32).mean(1)
    # the same rows again: unchanged argmax, but entropy above the threshold
    _, m2, _, stop2 = run(float(mean_h.min()) * 0.5)
    assert np.array_equal(stop2, np.zeros(n_req)) and m2.sum() == n_req * k_s
    # unchanged argmax and a threshold above the mean: the block stops
    x3, m3, st3, stop3 = run(float(mean_h.max()) * 1.01)
    assert np.array_equal(stop3, np.ones(n_req)) and m3.all() and st3["accepted"].numpy().all()
    y = np.where(m_np.astype(bool), x_np, st3["argmax"].numpy())
    assert np.array_equal(x3, y)
    # a new block forgets the previous argmax
    xi = torch.empty(rows, dtype=torch.int32, device="cuda")
    mi = torch.empty(rows, dtype=torch.uint8, device="cuda")
    eng.init_canvas(reqs, xi, mi, seeds, blocks)
    _, _, _, stop4 = run(1e9)
    assert np.array_equal(stop4, np.zeros(n_req))


def _gumbel_keys(L_row, tau, seed, pos, step, block, req):
    from oracle.philox import gumbel_uniforms
    u = gumbel_uniforms(seed, pos, step, block, req, L_row.shape[0])
    return L_row / tau - np.log(-np.log(u))


@pytest.mark.parametrize("model,n_req", [(synth.TINY, 2), (synth.FULL, 1)])
def test_sampled_candidates_match_the_oracle(model, n_req):
    """DG_CAND_SAMPLE: the Gumbel-max draw over the whole vocabulary equals
    the oracle's draw with the same uniforms on the same bf16 operand, except
    where the oracle's two best keys lie within the float32 band; the sampler
    then ranks the drawn candidates exactly as the oracle's sampler does."""
    say(f"[sample] V={model.vocab} n_req={n_req}")
    C = model.canvas
    rows = n_req * C
    eng, hw = _zero_layer_engine(model, max_rows=rows, max_requests=n_req)
    step, n_steps = 4, 12
    h, canvas, committed = _head_case(model, n_req, step, n_steps, seed=9)
    reqs = list(range(n_req))
    seeds, blocks = [31 + r for r in reqs], [3] * n_req
    x_dev, m_dev = canvas.cuda(), committed.cuda()
    stats = eng.new_stats(n_req)
    eng.test_head(reqs, h.cuda(), x_dev, m_dev, step, n_steps, seeds, blocks, stats, candidate="sample")
    torch.cuda.synchronize()
    st = stats_fields(stats)
    u_gpu = eng.ws_view("u", torch.bfloat16, (rows, model.d_model)).cpu()
    L_u = om.f64(u_gpu) @ om.f64(hw.embed).T
    tau = om.tau_at(step, n_steps, model.tau_first, model.tau_last)
    scale = np.abs(L_u).max()
    sample = st["sample"].numpy()
    mismatches = 0
    for row in range(rows):
        r, i = divmod(row, C)
        key = _gumbel_keys(L_u[row], tau, seeds[r], i, step, blocks[r], r)
        top = np.argsort(key)[::-1][:2]
        assert key[sample[row]] >= key[top[0]] - 1e-4 * (1 + abs(key[top[0]]))
        assert abs(st["sample_logit"].double().numpy()[row] - L_u[row, sample[row]]) < 1e-5 * scale
        if key[top[0]] - key[top[1]] > 1e-4 * (1 + abs(key[top[0]])):
            assert sample[row] == top[0], row
        elif sample[row] != top[0]:
            mismatches += 1
    say(f"  draws within the tie band: {mismatches}")
    x_np, m_np = canvas.numpy().astype(np.int64), committed.numpy()
    x_new, m_new = x_dev.cpu().numpy(), m_dev.cpu().numpy()
    for r in reqs:
        sl = slice(r * C, (r + 1) * C)
        drawn = (sample[sl].astype(np.int64), st["sample_logit"].double().numpy()[sl])
        xo, mo, c, acc = om.sample(x_np[sl], m_np[sl], st["max_logit"].double().numpy()[sl],
                                   st["argmax"].numpy()[sl], st["log_z"].double().numpy()[sl],
                                   st["held_logit"].double().numpy()[sl], tau, step, n_steps, seeds[r],
                                   blocks[r], r, model.vocab, drawn=drawn)
        assert np.abs(st["conf"].double().numpy()[sl] - c).max() < 1e-4
        k_s = om.commit_count(step, n_steps, C)
        if tie_gap_ok(c, k_s, 1e-4):
            assert np.array_equal(st["accepted"].numpy()[sl].astype(bool), acc)
            assert np.array_equal(x_new[sl], xo) and np.array_equal(m_new[sl], mo)


@pytest.mark.parametrize("model,n_req,confidence,candidate",
                         [(synth.TINY, 1, "prob", "argmax"), (synth.TINY, 2, "entropy", "argmax"),
                          (synth.TINY, 1, "prob", "sample"), (synth.FULL, 1, "prob", "argmax"),
                          (synth.FULL, 1, "entropy", "argmax")])
def test_sampler_fed_the_oracles_statistics(model, n_req, confidence, candidate):
    """The GPU sampler (dg_test_sample) fed the oracle's own per-position
    statistics of float64 logits (held logit, max, argmax, log Z, entropy;
    the Gumbel-max draws for sampled candidates), rounded once to float32:
    accepted set, canvas, mask and confidence equal the oracle's sampler bit
    for bit, the ranking decided in float32 on both sides."""
    say(f"[sampler<-oracle] V={model.vocab} n_req={n_req} {confidence} {candidate}")
    from block_discrete_diffusion_dg_amd.engine import stats_tensor
    C = model.canvas
    rows = n_req * C
    eng, hw = _zero_layer_engine(model, max_rows=rows, max_requests=n_req)
    step, n_steps = 6, 16
    h, canvas, committed = _head_case(model, n_req, step, n_steps, seed=13)
    reqs = list(range(n_req))
    seeds, blocks = [41 + r for r in reqs], [4] * n_req
    tau64 = om.tau_at(step, n_steps, model.tau_first, model.tau_last)
    tau32 = om.tau_at(step, n_steps, model.tau_first, model.tau_last, precision="float32")
    x_np, m_np = canvas.numpy().astype(np.int64), committed.numpy()
    L = om.logits(h.double().numpy(), hw.final_norm, hw.embed, model)
    M, a, logZ, gx = om.row_stats(L, x_np, tau64)
    H = om.row_entropy(L, tau64)
    drawn = None
    if candidate == "sample":
        drawn = [om.gumbel_candidates(L[r * C:(r + 1) * C], tau64, seeds[r], step, blocks[r], r) for r in reqs]
        ys = np.concatenate([d[0] for d in drawn])
        lys = np.concatenate([d[1] for d in drawn])
    st_in = stats_tensor(M, logZ, gx, a, H, ys if drawn else None, lys if drawn else None).cuda()
    x_dev, m_dev = canvas.cuda(), committed.cuda()
    stats = eng.new_stats(n_req)
    eng.test_sample(reqs, st_in, x_dev, m_dev, step, n_steps, seeds, blocks, stats, confidence=confidence,
                    candidate=candidate)
    torch.cuda.synchronize()
    st = stats_fields(stats)
    f32 = lambda v: np.asarray(v, np.float32)
    x_new, m_new = x_dev.cpu().numpy(), m_dev.cpu().numpy()
    for r in reqs:
        sl = slice(r * C, (r + 1) * C)
        dr = None if drawn is None else (drawn[r][0], f32(drawn[r][1]))
        xo, mo, c, acc = om.sample(x_np[sl], m_np[sl], f32(M[sl]), a[sl], f32(logZ[sl]), f32(gx[sl]), tau32,
                                   step, n_steps, seeds[r], blocks[r], r, model.vocab, confidence=confidence,
                                   H=f32(H[sl]), drawn=dr, precision="float32")
        assert np.array_equal(st["conf"].numpy()[sl].view(np.int32), c.astype(np.float32).view(np.int32))
        assert np.array_equal(st["accepted"].numpy()[sl].astype(bool), acc)
        assert np.array_equal(x_new[sl], xo) and np.array_equal(m_new[sl], mo)
        assert mo.sum() == om.commit_count(step, n_steps, C)


@pytest.mark.parametrize("model,n_req,width", [(synth.TINY, 2, 64), (synth.FULL, 1, 704)])
def test_self_conditioning_signal(model, n_req, width):
    """The self-conditioning signal a step leaves for its slot's next step:
    the expected embedding under softmax(L) (temperature 1, the whole
    vocabulary) through the SwiGLU feed-forward layer, against the oracle on
    the same bf16 final-normed rows."""
    say(f"[selfcond] V={model.vocab} d={model.d_model} width={width} n_req={n_req}")
    C = model.canvas
    rows = n_req * C
    sc = make_selfcond(model, width, 3)
    cfg0 = dataclasses.replace(model, n_layers=0)
    eng, hw = make_engine(cfg0, max_ctx=4 * C, max_requests=n_req + 1, max_rows=rows, selfcond=sc)
    h, canvas, committed = _head_case(model, n_req, 2, 8, seed=17)
    reqs = [n_req - r for r in range(n_req)]  # slots in reverse order: the signal is stored per slot
    eng.test_head(reqs, h.cuda(), canvas.cuda(), committed.cuda(), 2, 8, [5] * n_req, [0] * n_req)
    torch.cuda.synchronize()
    u_gpu = eng.ws_view("u", torch.bfloat16, (rows, model.d_model)).cpu()
    L_u = om.f64(u_gpu) @ om.f64(hw.embed).T
    sc_cpu = {k: v.cpu() for k, v in sc.items()}
    want = om.self_condition(L_u, hw.embed, sc_cpu)
    state = eng.ws_view("sc_state", torch.float32, (n_req + 1, C, model.d_model)).cpu()
    e_gpu = om.f64(eng.ws_view("sc_e", torch.bfloat16, (rows, model.d_model)).cpu())
    err_e = max_rel(e_gpu, om.expected_embedding(L_u, hw.embed))
    errs = [max_rel(om.f64(state[reqs[r]]), want[r * C:(r + 1) * C]) for r in range(n_req)]
    say(f"  expected embedding error {err_e:.2e}; signal errors {[f'{e:.2e}' for e in errs]}; "
        f"max |s| {np.abs(want).max():.3e}")
    assert err_e <= REL_TOL and max(errs) <= REL_TOL
    assert np.abs(want).max() > 1e-6


# ------------------------------------------------------------------------ attention alone

@pytest.mark.parametrize("model,P,n,causal", [(synth.TINY, 64, 32, False), (synth.TINY, 75, 37, True),
                                              (synth.TINY, 0, 32, True), (synth.FULL, 2048, 256, False),
                                              (synth.FULL, 2048, 256, True), (synth.FULL, 32768, 256, False),
                                              (synth.FULL, 1000, 300, False)])
def test_attention_alone_matches_the_oracle(model, P, n, causal):
    """dg_test_attention on given rotated queries and cache rows against the
    oracle's softmax(q K^T / sqrt(dh)) V in float64 on the same bf16 inputs
    (the kernel rounds the probabilities and the output to bf16)."""
    say(f"[attention] dh={model.head_dim} Hq={model.n_q_heads} Hkv={model.n_kv_heads} P={P} n={n} causal={causal}")
    cfg = dataclasses.replace(model, n_layers=1)
    total = -(-(P + n) // 32) * 32
    eng, _ = make_engine(cfg, max_ctx=max(total, 2 * cfg.canvas), max_rows=max(n, cfg.canvas))
    k = synth.make_random_kv((cfg.n_kv_heads, total, cfg.head_dim), 3, 0, "k", "cuda")
    v = synth.make_random_kv((cfg.n_kv_heads, total, cfg.head_dim), 3, 0, "v", "cuda")
    eng.set_cache_rows(0, 0, k, v)
    eng.set_cache_len(0, P)
    q = synth.make_random_kv((n, cfg.n_q_heads, cfg.head_dim), 5, 0, "q", "cuda")
    o = eng.test_attention(0, 0, q, causal)
    torch.cuda.synchronize()
    kc = om.f64(k.cpu()).transpose(1, 0, 2)[:P + n]
    vc = om.f64(v.cpu()).transpose(1, 0, 2)[:P + n]
    want = om.attention(om.f64(q.cpu()), kc, vc, P, causal).reshape(n, -1)
    err = max_rel(om.f64(o.cpu()), want)
    say(f"  max rel error {err:.2e}")
    assert err <= 1e-2
    assert eng.cache_len(0) == P


def test_init_canvas_matches_philox():
    model = synth.TINY
    eng, _ = _zero_layer_engine(model, max_rows=2 * model.canvas, max_requests=2)
    x = torch.zeros(2 * model.canvas, dtype=torch.int32, device="cuda")
    m = torch.ones(2 * model.canvas, dtype=torch.uint8, device="cuda")
    eng.init_canvas([1, 0], x, m, [2**40 + 7, 5], [3, 0])
    torch.cuda.synchronize()
    want0, _ = om.init_canvas(2**40 + 7, 3, 1, model.canvas, model.vocab)
    want1, _ = om.init_canvas(5, 0, 0, model.canvas, model.vocab)
    assert np.array_equal(x.cpu().numpy(), np.concatenate([want0, want1]))
    assert not m.any()


# ------------------------------------------------------------------------ one layer

def _fill_prefix(eng, cfg, P, seed=7, slot=0, layer=0):
    k = synth.make_random_kv((cfg.n_kv_heads, P, cfg.head_dim), seed, layer, "k", "cuda")
    v = synth.make_random_kv((cfg.n_kv_heads, P, cfg.head_dim), seed, layer, "v", "cuda")
    eng.set_cache_rows(slot, layer, k, v)
    eng.set_cache_len(slot, P)


def _cache_rows(eng, slot, layer, lo, hi):
    k, v = eng.cache_rows(slot, layer, lo, hi)
    return k.permute(1, 0, 2).contiguous().cpu(), v.permute(1, 0, 2).contiguous().cpu()


# (workload, causal, prefix, rows, model overrides): the workloads' own layer
# shapes, plus the full-width layer with a 32,768-token prefix (the
# long-context workload's attention) and with 2,048 rows in one call (the
# batch workload's tokens per step: ~128 rows per expert, several 128-row
# chunks for hot experts) and with 4,096 rows (16 requests' worth: the fused
# router's permutation then runs in chunks), and a small layer whose projection widths (K = 768
# and 384) are not a power-of-two multiple of 256, so the dense projections
# take their streaming-tile form instead of the split-K form.
@pytest.mark.parametrize("name,causal,P,C,over,fmt", [
    ("tiny", False, None, None, None, "bf16"), ("tiny", True, None, None, None, "bf16"),
    ("one_layer", False, None, None, None, "bf16"),
    ("one_layer", True, None, None, None, "bf16"),
    ("one_layer", False, 32768, None, None, "bf16"),
    ("one_layer", False, None, 2048, None, "bf16"),
    ("one_layer", False, None, 4096, None, "bf16"),
    ("tiny", False, None, None, {"d_model": 768, "n_q_heads": 6}, "bf16"),
    ("tiny", False, None, None, None, "fp8"),
    ("one_layer", False, None, None, None, "fp8"),
    ("one_layer", False, None, 2048, None, "fp8")])
def test_layer_parity(name, causal, P, C, over, fmt):
    """With fmt "fp8" the experts stream E4M3 weights; the oracle multiplies
    with its own dequantisation of the same bf16 weights."""
    wl = synth.WORKLOADS[name]
    cfg = dataclasses.replace(wl.model, n_layers=1, **(over or {}))
    P = P or wl.prefix
    C = C or cfg.canvas
    say(f"[layer] {name} {over or ''} causal={causal} P={P} rows={C} experts={fmt}")
    eng, hw = make_engine(cfg, max_ctx=P + 2 * C, max_rows=C, expert_format=fmt)
    _fill_prefix(eng, cfg, P)
    h = synth.make_hidden(C, cfg.d_model, 21)
    h_dev = h.cuda()
    eng.test_layer(0, 0, h_dev, causal)
    torch.cuda.synchronize()
    ck, cv = _cache_rows(eng, 0, 0, 0, P)
    keep = {}
    h_or, k_or, v_or = om.layer_forward(h.double().numpy(), hw.layer(0), cfg, om.f64(ck), om.f64(cv),
                                        P, causal, keep)
    k_gpu, v_gpu = _cache_rows(eng, 0, 0, P, P + C)
    q_gpu = eng.ws_view("q", torch.bfloat16, (C, cfg.n_q_heads, cfg.head_dim)).cpu()
    o_gpu = eng.ws_view("attn_o", torch.bfloat16, (C, cfg.n_q_heads * cfg.head_dim)).cpu()
    z_gpu = eng.ws_view("z", torch.float32, (C, cfg.n_experts)).cpu()
    idx_gpu = eng.ws_view("idx", torch.int32, (C, cfg.top_k)).cpu().numpy()
    pairs = dict(q=(om.f64(q_gpu), keep["q"]), k=(om.f64(k_gpu), k_or), v=(om.f64(v_gpu), v_or),
                 attn=(om.f64(o_gpu), keep["attn_o"].reshape(C, -1)), z=(om.f64(z_gpu), keep["z"]))
    errs = {n: max_rel(g, o) for n, (g, o) in pairs.items()}
    # router decisions on the GPU's own logits are bit-exact
    idx_from_gpu_z, _ = om.route(om.f64(z_gpu), cfg.top_k)
    assert np.array_equal(idx_gpu, idx_from_gpu_z)
    # the logits themselves, on the GPU's own bf16 router input: fp32
    # accumulation over d terms, bounded by 1e-4 * sum_k |u_k W_ek|
    u2 = om.f64(eng.ws_view("u", torch.bfloat16, (C, cfg.d_model)).cpu())
    lw = hw.layer(0)
    absdot = np.abs(u2) @ np.abs(om.f64(lw["w_router"])).T
    assert np.all(np.abs(om.f64(z_gpu) - u2 @ om.f64(lw["w_router"]).T) <= 1e-4 * absdot)
    # the fused router's permutation, bit for bit on its own expert ids
    cnt, off, perm, slot = om.permutation(idx_gpu.astype(np.int64), cfg.n_experts)
    assert np.array_equal(eng.ws_view("cnt", torch.int32, (cfg.n_experts,)).cpu().numpy(), cnt)
    assert np.array_equal(eng.ws_view("off", torch.int32, (cfg.n_experts + 1,)).cpu().numpy(), off)
    assert np.array_equal(eng.ws_view("perm", torch.int32, (C * cfg.top_k,)).cpu().numpy(), perm)
    assert np.array_equal(eng.ws_view("slot", torch.int32, (C, cfg.top_k)).cpu().numpy(), slot)
    # against the oracle's own logits: a different expert set only inside the
    # fixed tie band of bf16 router inputs, and in few rows
    swaps = router_swaps(idx_gpu, keep["z"], cfg.top_k, router_band(keep["u_moe"], lw["w_router"]))
    assert len(swaps) <= max(2, C // 20), len(swaps)
    # hidden state: the oracle takes the expert choice the kernel made in the
    # swapped rows (the integer decision is taken in the kernel's precision)
    h_forced = moe_with_experts(keep, lw, cfg, np.where(np.isin(np.arange(C), swaps)[:, None], idx_gpu,
                                                        keep["idx"]))
    errs["h"] = max_rel(h_dev.cpu(), h_forced)
    errs["h_free"] = max_rel(h_dev.cpu(), h_or)
    pairs["h"] = (h_dev.cpu(), h_forced)
    say(f"  router swaps within band: {len(swaps)}/{C}; max rel errors:",
        {k: f"{v:.2e}" for k, v in errs.items()})
    say("  element-wise rel errors (max/p99/median, floor 1e-3 max|o|):",
        {n: fmt_elem(elem_stats(g, o)) for n, (g, o) in pairs.items()})
    for k_, e in errs.items():
        if k_ != "h_free" or not swaps:
            assert e <= REL_TOL, (k_, e)
    # experts on identical operands: the GPU's MoE-normed rows and routing weights
    w_gpu = om.f64(eng.ws_view("w", torch.float32, (C, cfg.top_k)).cpu())
    slot_gpu = eng.ws_view("slot", torch.int32, (C, cfg.top_k)).cpu().numpy()
    n_slots = eng.max_rows * cfg.top_k
    y = om.f64(eng.ws_view("y", torch.bfloat16, (n_slots, cfg.d_model)).cpu())
    ys = om.f64(eng.ws[eng.layout.y + n_slots * cfg.d_model * 2:][:eng.max_rows * cfg.d_model * 4]
                .view(torch.float32).view(eng.max_rows, cfg.d_model).cpu())
    ys_ref = om.swiglu(u2, lw["ws_gate"], lw["ws_up"], lw["ws_down"])
    assert max_rel(ys[:C], ys_ref) <= REL_TOL
    for t in range(0, C, max(1, C // 16)):
        for j in range(cfg.top_k):
            e = idx_gpu[t, j]
            ref = w_gpu[t, j] * om.swiglu(u2[t:t + 1], lw["w_gate"][e], lw["w_up"][e], lw["w_down"][e])[0]
            assert max_rel(y[slot_gpu[t, j]], ref) <= REL_TOL, (t, j)
    # every wait of the expert kernel saw its input published in time
    assert eng.moe_counters()["spin_timeouts"] == 0
