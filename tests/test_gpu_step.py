"""Whole-loop parity on the tiny workload (1 layer, d 256, V 4096, C 32,
prefix 64, 4 steps): prefill, initial canvas, every denoising step and the
block commit, each compared with the float64 oracle. The oracle is
teacher-forced with the GPU's KV cache and canvas state before each call so a
near-tie decision cannot propagate; every comparison states its band."""
import numpy as np
import pytest
import torch

from block_discrete_diffusion_dg_amd import synth
from block_discrete_diffusion_dg_amd.engine import stats_fields
from oracle import model as om
from oracle import philox as philox_mod
from tests.gpu_util import REL_TOL, make_engine, max_rel, say, tie_gap_ok

pytestmark = pytest.mark.gpu


def _oracle_request(eng, cfg, slot, length):
    req = om.Request(cfg, eng.max_ctx)
    for l in range(cfg.n_layers):
        k, v = eng.cache_rows(slot, l, 0, length)
        req.k[l, :length] = om.f64(k.permute(1, 0, 2).cpu())
        req.v[l, :length] = om.f64(v.permute(1, 0, 2).cpu())
    req.length = length
    return req


@pytest.mark.parametrize("confidence,stop_entropy,candidate",
                         [("prob", 0.0, "argmax"), ("entropy", 1e9, "argmax"), ("prob", 0.0, "sample")])
def test_tiny_block_loop_parity(confidence, stop_entropy, candidate):
    """With entropy confidence and a threshold every mean entropy is under,
    adaptive stopping reduces to "the argmax did not change since the
    previous step": both sides must agree on it wherever the argmax is
    clear of ties."""
    wl = synth.WORKLOADS["tiny"]
    cfg, P, S = wl.model, wl.prefix, wl.n_steps
    C = cfg.canvas
    eng, hw = make_engine(cfg, max_ctx=P + 2 * C)
    prompt = synth.make_prompt(P, cfg.vocab, wl.seed)
    say("[tiny] prefill")
    eng.prefill(0, prompt.cuda())
    torch.cuda.synchronize()
    assert eng.cache_len(0) == P
    ref = om.Request(cfg, eng.max_ctx)
    om.prefill(hw, cfg, ref, prompt.numpy().astype(np.int64))
    gpu_req = _oracle_request(eng, cfg, 0, P)
    assert max_rel(gpu_req.k[:, :P], ref.k[:, :P]) <= REL_TOL
    assert max_rel(gpu_req.v[:, :P], ref.v[:, :P]) <= REL_TOL
    kv_prefix = eng.kv_view()[0, :, :, :, :P].clone()

    x = torch.empty(C, dtype=torch.int32, device="cuda")
    m = torch.empty(C, dtype=torch.uint8, device="cuda")
    seed, block = 1234, 0
    eng.init_canvas([0], x, m, [seed], [block])
    x0, m0 = om.init_canvas(seed, block, 0, C, cfg.vocab)
    assert np.array_equal(x.cpu().numpy(), x0) and not m.cpu().numpy().any()

    a_prev = None
    stop = torch.zeros(1, dtype=torch.int32, device="cuda")
    for s in range(1, S + 1):
        say(f"[tiny] {confidence} step {s}")
        x_in = x.cpu().numpy().astype(np.int64)
        m_in = m.cpu().numpy()
        stats = eng.new_stats(1)
        eng.denoise_step([0], x, m, s, S, [seed], [block], stats, confidence=confidence,
                         stop_entropy=stop_entropy, stop=stop, candidate=candidate)
        torch.cuda.synchronize()
        st = stats_fields(stats)
        keep = {}
        # teacher-forced: the oracle compares with the GPU's previous argmax
        xo, mo = om.denoise_step(hw, cfg, gpu_req, x_in, m_in, s, S, seed, block, 0, keep,
                                 confidence=confidence, stop_entropy=stop_entropy, a_prev=a_prev,
                                 candidate=candidate)
        big = np.abs(keep["logits"]).max()
        assert max_rel(st["max_logit"], keep["M"]) <= REL_TOL
        clear = np.array([tie_gap_ok(keep["logits"][i], 1, 2 * REL_TOL * big) for i in range(C)])
        if candidate == "sample":
            # draws: equal wherever the oracle's two best Gumbel keys are apart
            # by more than the logits' error over tau
            for i in range(C):
                key = keep["logits"][i] / keep["tau"] - np.log(-np.log(
                    philox_mod.gumbel_uniforms(seed, i, s, block, 0, cfg.vocab)))
                ok = tie_gap_ok(key, 1, 2 * REL_TOL * big / keep["tau"])
                clear[i] &= ok
                if ok:
                    assert st["sample"].numpy()[i] == keep["drawn"][0][i], i
        assert np.array_equal(st["argmax"].numpy()[clear], keep["a"][clear])
        assert np.abs(st["entropy"].double().numpy() - keep["H"]).max() <= REL_TOL * big / keep["tau"]
        assert np.abs(st["conf"].double().numpy() - keep["c"]).max() <= REL_TOL * big / keep["tau"] * 4
        stopped = bool(stop.item())
        if clear.all():
            assert stopped == keep["stop"]
        a_prev = st["argmax"].numpy().astype(np.int64)
        k_s = C if stopped else om.commit_count(s, S, C)
        acc = st["accepted"].numpy().astype(bool)
        assert acc.sum() == k_s == m.cpu().numpy().sum()
        if tie_gap_ok(keep["c"], k_s, REL_TOL * big / keep["tau"] * 4) and clear.all():
            assert np.array_equal(acc, keep["accept"])
            assert np.array_equal(x.cpu().numpy(), xo)
        # the KV cache is only read by a denoising step
        assert torch.equal(eng.kv_view()[0, :, :, :, :P], kv_prefix)
        assert eng.cache_len(0) == P
        if stopped:
            break
    assert m.cpu().numpy().all()

    say("[tiny] commit")
    final = x.clone()
    eng.commit_block([0], final)
    torch.cuda.synchronize()
    assert eng.cache_len(0) == P + C
    assert torch.equal(eng.kv_view()[0, :, :, :, :P], kv_prefix)  # committed rows never rewritten
    om.commit_block(hw, cfg, gpu_req, final.cpu().numpy().astype(np.int64))
    after = _oracle_request(eng, cfg, 0, P + C)
    assert max_rel(after.k[:, P:P + C], gpu_req.k[:, P:P + C]) <= REL_TOL
    assert max_rel(after.v[:, P:P + C], gpu_req.v[:, P:P + C]) <= REL_TOL


def test_prefill_chunking_and_commit_are_causally_consistent():
    cfg = synth.TINY
    C = cfg.canvas
    n = 3 * C + 7  # ragged: several chunks of max_rows=C rows plus a tail
    max_ctx = -(-(n + 3 * C) // 32) * 32  # capacity: a multiple of 32 positions
    eng, hw = make_engine(cfg, max_ctx=max_ctx, max_requests=3, max_rows=C)
    ids = synth.make_prompt(n + C, cfg.vocab, 9).cuda()
    eng.prefill(0, ids)                       # whole sequence, chunked by the library
    eng.prefill(1, ids[:n].contiguous())      # prefix only ...
    eng.commit_block([1], ids[n:].contiguous())  # ... then the block as a commit
    torch.cuda.synchronize()
    assert eng.cache_len(0) == eng.cache_len(1) == n + C
    kv = eng.kv_view()
    a = kv[0, :, :, :, :n + C].float().cpu().numpy()
    b = kv[1, :, :, :, :n + C].float().cpu().numpy()
    assert max_rel(b, a) <= REL_TOL
    ref = om.Request(cfg, n + 3 * C)
    om.prefill(hw, cfg, ref, ids.cpu().numpy().astype(np.int64))
    got = _oracle_request(eng, cfg, 0, n + C)
    assert max_rel(got.k[:, :n + C], ref.k[:, :n + C]) <= REL_TOL
    assert max_rel(got.v[:, :n + C], ref.v[:, :n + C]) <= REL_TOL


def test_step_is_deterministic_and_batch_matches_single():
    cfg = synth.TINY
    C = cfg.canvas
    eng, hw = make_engine(cfg, max_ctx=64 + 2 * C, max_requests=2, max_rows=2 * C)
    for slot in (0, 1):
        eng.prefill(slot, synth.make_prompt(64, cfg.vocab, 5 + slot).cuda())
    x = torch.empty(2 * C, dtype=torch.int32, device="cuda")
    m = torch.empty(2 * C, dtype=torch.uint8, device="cuda")
    eng.init_canvas([0, 1], x, m, [1, 2], [0, 0])
    outs = []
    for _ in range(2):
        xx, mm = x.clone(), m.clone()
        st = eng.new_stats(2)
        eng.denoise_step([0, 1], xx, mm, 2, 4, [1, 2], [0, 0], st)
        outs.append((xx.cpu(), mm.cpu(), st.cpu()))
    assert all(torch.equal(a, b) for a, b in zip(outs[0], outs[1]))
    # request 1 alone gives the same statistics (tolerance: its attention split may differ)
    x1, m1 = x[C:].clone(), m[C:].clone()
    st1 = eng.new_stats(1)
    eng.denoise_step([1], x1, m1, 2, 4, [2], [0], st1)
    torch.cuda.synchronize()
    a = stats_fields(outs[0][2][C:])
    b = stats_fields(st1)
    assert max_rel(b["max_logit"], a["max_logit"]) < 1e-4
    assert torch.equal(a["argmax"], b["argmax"])
    assert eng.moe_counters()["spin_timeouts"] == 0


def test_ar_steps_match_the_oracle():
    """AR mode: greedy decode steps of two requests appended to their caches;
    next tokens equal the oracle's argmax wherever its two best logits are
    apart by more than the band, and the appended K/V rows match."""
    cfg = synth.TINY
    P, n_steps = 40, 3
    eng, hw = make_engine(cfg, max_ctx=128, max_requests=2, max_rows=cfg.canvas)
    prompts = [synth.make_prompt(P, cfg.vocab, 21 + r) for r in range(2)]
    for r in range(2):
        eng.prefill(r, prompts[r].cuda())
    tokens = torch.tensor([int(p[-1]) for p in prompts], dtype=torch.int32, device="cuda")
    for step in range(n_steps):
        say(f"[ar] step {step}")
        refs = [_oracle_request(eng, cfg, r, P + step) for r in range(2)]  # teacher-forced caches
        nxt = eng.ar_step([0, 1], tokens)
        torch.cuda.synchronize()
        for r in range(2):
            assert eng.cache_len(r) == P + step + 1
            want, L = om.ar_step(hw, cfg, refs[r], int(tokens[r]))
            if tie_gap_ok(L, 1, 2 * REL_TOL * np.abs(L).max()):
                assert int(nxt[r]) == want, (step, r)
            got = _oracle_request(eng, cfg, r, P + step + 1)
            assert max_rel(got.k[:, P + step], refs[r].k[:, P + step]) <= REL_TOL
            assert max_rel(got.v[:, P + step], refs[r].v[:, P + step]) <= REL_TOL
        tokens = nxt

