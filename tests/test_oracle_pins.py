"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a published known answer, a
closed form, a library routine computing the same mathematical object by
another route, or an invariant the pages state.
"""
import dataclasses

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch
import torch.nn.functional as F

from block_discrete_diffusion_dg_amd import synth
from oracle import fp8
from oracle import model as om
from oracle import metrics
from oracle import philox as philox_mod
from oracle.philox import philox4x32_10, uniform_ids
from tests.conftest import golden

RNG = np.random.default_rng(1234)


# ----------------------------------------------------------------------------- Philox

def test_philox_known_answers():
    for row in golden("philox4x32_10_kat.txt"):
        words = [int(x, 16) for x in row]
        ctr, key, want = words[:4], words[4:6], words[6:]
        got = philox4x32_10(np.array(ctr), np.array(key))
        assert [int(v) for v in got] == want


def test_uniform_ids_power_of_two_is_top_bits():
    ctr = np.stack([np.arange(1000), np.full(1000, 3), np.full(1000, 1), np.zeros(1000)], -1)
    w0 = philox4x32_10(ctr, np.array([7, 0]))[:, 0].astype(np.int64)
    ids = uniform_ids(7, np.arange(1000), 3, 1, 0, 1 << 18)
    assert np.array_equal(ids, w0 >> 14)


def test_uniform_ids_chi_square():
    # The forward process at kappa = 0 leaves every position uniform over the
    # vocabulary (explainer §3.1): re-noised ids must look uniform.
    V = 4096
    ids = np.concatenate([uniform_ids(11, np.arange(256), s, b, 0, V)
                          for s in range(1, 41) for b in range(40)])
    counts = np.bincount(ids, minlength=V)
    chi2 = ((counts - len(ids) / V) ** 2 / (len(ids) / V)).sum()
    assert scipy.stats.chi2.sf(chi2, V - 1) > 1e-4
    assert ids.min() >= 0 and ids.max() < V


def test_uniform_ids_streams_differ():
    a = uniform_ids(5, np.arange(256), 1, 0, 0, 1 << 18)
    for other in [uniform_ids(5, np.arange(256), 2, 0, 0, 1 << 18),
                  uniform_ids(5, np.arange(256), 1, 1, 0, 1 << 18),
                  uniform_ids(5, np.arange(256), 1, 0, 1, 1 << 18),
                  uniform_ids(6, np.arange(256), 1, 0, 0, 1 << 18)]:
        assert np.mean(a == other) < 0.01


# ----------------------------------------------------------------------------- RMSNorm

def test_rms_norm_constant_row_closed_form():
    eps = 1e-6
    for c in [0.02, -3.0, 1e-4]:
        x = np.full((1, 64), c)
        g = RNG.normal(size=64)
        want = c / np.sqrt(c * c + eps) * g
        assert np.allclose(om.rms_norm(x, g, eps), want, rtol=1e-14, atol=0)


def test_rms_norm_matches_torch_and_is_scale_invariant():
    x = RNG.normal(size=(5, 96))
    g = RNG.normal(size=96)
    want = F.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(om.rms_norm(x, g, 1e-6), want, rtol=1e-12, atol=1e-14)
    assert np.allclose(om.rms_norm(1e3 * x, g, 0.0), om.rms_norm(x, g, 0.0), rtol=1e-12)


# ----------------------------------------------------------------------------- RoPE

def test_rope_two_dim_is_rotation_by_position():
    # dh = 2: a single pair with frequency theta^0 = 1: rotation by pos radians.
    x = np.array([[[1.0, 0.0]]] * 4)
    pos = np.array([0, 1, 2, 7])
    out = om.rope(x, pos, 10000.0)[:, 0, :]
    assert np.allclose(out, np.stack([np.cos(pos), np.sin(pos)], -1), atol=1e-15)


def test_rope_preserves_norm_and_is_identity_at_zero():
    x = RNG.normal(size=(6, 3, 128))
    pos = np.arange(6) * 1000
    out = om.rope(x, pos, 10000.0)
    half = 64
    assert np.allclose(out[..., :half] ** 2 + out[..., half:] ** 2,
                       x[..., :half] ** 2 + x[..., half:] ** 2, rtol=1e-12)
    assert np.allclose(om.rope(x, np.zeros(6), 10000.0), x, atol=0)


def test_rope_scores_depend_on_relative_position_only():
    q = RNG.normal(size=(1, 1, 64))
    k = RNG.normal(size=(1, 1, 64))
    base = None
    for shift in [0, 17, 4000]:
        s = float((om.rope(q, [shift + 9], 1e4) * om.rope(k, [shift + 2], 1e4)).sum())
        base = s if base is None else base
        assert abs(s - base) < 1e-9 * max(1.0, abs(base))


def test_rope_angles_hand_values():
    # angle(pos, j) = pos * theta^(-2j/dh), worked by hand at theta = 10000:
    # 10000^(-1/2) = 0.01, 10000^(-1/4) = 0.1, 10000^0 = 1.
    cases = [(3, 1, 4, 0.03), (5, 2, 8, 0.05), (7, 16, 64, 0.07), (9, 1, 8, 0.9),
             (11, 0, 128, 11.0), (2, 48, 128, 2e-3)]
    for pos, j, dh, want in cases:
        got = om.rope_angles(np.array([pos]), dh, 1e4)[0, j]
        assert abs(got - want) <= 1e-12 * max(1.0, want), (pos, j, dh, got, want)


def test_rope_pair_rotates_by_its_own_frequency():
    # a unit vector in pair j (components j and j + dh/2) turns by pos * 0.01
    # for j = dh/4 (theta^(-1/2)); every other pair stays zero.
    dh, j, pos = 16, 4, 250
    x = np.zeros((1, 1, dh))
    x[0, 0, j] = 1.0
    out = om.rope(x, np.array([pos]), 1e4)[0, 0]
    ang = pos * 0.01
    assert abs(out[j] - np.cos(ang)) < 1e-12 and abs(out[j + dh // 2] - np.sin(ang)) < 1e-12
    rest = np.delete(out, [j, j + dh // 2])
    assert np.all(rest == 0.0)


# ----------------------------------------------------------------------------- attention

def _sdpa_reference(q, k, v, n_prefix, causal):
    """torch scaled_dot_product_attention (float64, CPU) with explicit GQA expansion."""
    n, Hq, dh = q.shape
    Hkv = k.shape[1]
    rep = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(rep, 0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(rep, 0)
    mask = None
    if causal:
        nk = k.shape[0]
        mask = torch.arange(nk)[None, :] <= (n_prefix + torch.arange(n))[:, None]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv,P,n", [(4, 2, 7, 5), (2, 2, 0, 6), (8, 2, 33, 16)])
def test_attention_matches_torch_sdpa(causal, Hq, Hkv, P, n):
    dh = 16
    q = RNG.normal(size=(n, Hq, dh))
    k = RNG.normal(size=(P + n, Hkv, dh))
    v = RNG.normal(size=(P + n, Hkv, dh))
    got = om.attention(q, k, v, P, causal)
    assert np.allclose(got, _sdpa_reference(q, k, v, P, causal), rtol=1e-10, atol=1e-12)


def test_attention_rows_sum_to_one_and_equal_scores_average():
    n, P, Hq, Hkv, dh = 5, 9, 4, 2, 8
    q = RNG.normal(size=(n, Hq, dh))
    k = RNG.normal(size=(P + n, Hkv, dh))
    ones = np.ones((P + n, Hkv, dh))
    assert np.allclose(om.attention(q, k, ones, P, False), 1.0, rtol=1e-13)
    v = RNG.normal(size=(P + n, Hkv, dh))
    zero_q = np.zeros_like(q)
    out = om.attention(zero_q, k, v, P, False)
    for h in range(Hq):
        assert np.allclose(out[:, h], v[:, (h * Hkv) // Hq].mean(0), rtol=1e-12)


def test_attention_without_rope_is_permutation_equivariant_over_canvas():
    n, P, H, dh = 6, 4, 2, 8
    q = RNG.normal(size=(n, H, dh))
    kc = RNG.normal(size=(n, H, dh))
    vc = RNG.normal(size=(n, H, dh))
    kp = RNG.normal(size=(P, H, dh))
    vp = RNG.normal(size=(P, H, dh))
    perm = RNG.permutation(n)
    base = om.attention(q, np.concatenate([kp, kc]), np.concatenate([vp, vc]), P, False)
    permuted = om.attention(q[perm], np.concatenate([kp, kc[perm]]),
                            np.concatenate([vp, vc[perm]]), P, False)
    assert np.allclose(permuted, base[perm], rtol=1e-12)


# ----------------------------------------------------------------------------- router

def test_route_matches_stable_argsort_and_softmax():
    z = RNG.normal(size=(64, 16))
    z[3, 5] = z[3, 2]  # a tie: the lower id must come first
    z[3, 2] = z[3].max() + 1.0
    z[3, 5] = z[3, 2]
    idx, w = om.route(z, 4)
    want = np.argsort(-z, axis=1, kind="stable")[:, :4]
    assert np.array_equal(idx, want)
    assert idx[3, 0] == 2 and idx[3, 1] == 5
    sel = np.take_along_axis(z, want, 1)
    assert np.allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-13)
    assert np.allclose(w.sum(1), 1.0)


def test_route_k1_is_argmax_with_weight_one():
    z = RNG.normal(size=(20, 8))
    idx, w = om.route(z, 1)
    assert np.array_equal(idx[:, 0], np.argmax(z, 1))
    assert np.all(w == 1.0)


def test_permutation_matches_stable_argsort():
    n, k, E = 50, 3, 10
    z = RNG.normal(size=(n, E))
    idx, _ = om.route(z, k)
    cnt, off, perm, slot = om.permutation(idx, E)
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(perm, order // k)
    assert np.array_equal(cnt, np.bincount(flat, minlength=E))
    assert cnt.sum() == n * k and off[0] == 0 and off[-1] == n * k
    assert np.array_equal(np.sort(slot.reshape(-1)), np.arange(n * k))
    for t in range(n):
        for j in range(k):
            assert perm[slot[t, j]] == t
            assert off[idx[t, j]] <= slot[t, j] < off[idx[t, j] + 1]


# ----------------------------------------------------------------------------- experts

def _tiny_layer(E, k, d=32, F=16, Fs=24, seed=0):
    cfg = dataclasses.replace(synth.TINY, d_model=d, n_experts=E, top_k=k, d_expert=F,
                              d_shared=Fs, n_q_heads=2, n_kv_heads=1, head_dim=16,
                              weight_std=0.3)
    return cfg, synth.make_layer_weights(cfg, 0, seed, gain_jitter=0.1)


def test_moe_with_all_experts_equals_dense_softmax_mixture():
    E = 6
    cfg, lw = _tiny_layer(E, E)
    u = RNG.normal(size=(9, cfg.d_model))
    z = u @ om.f64(lw["w_router"]).T
    idx, w = om.route(z, E)
    got = om.moe(u, idx, w, lw, E)
    p = scipy.special.softmax(z, axis=1)
    want = om.swiglu(u, lw["ws_gate"], lw["ws_up"], lw["ws_down"])
    for e in range(E):
        want = want + p[:, e:e + 1] * om.swiglu(u, lw["w_gate"][e], lw["w_up"][e], lw["w_down"][e])
    assert np.allclose(got, want, rtol=1e-10, atol=1e-12)


def test_moe_grouped_equals_per_token_sum_and_idle_expert_is_inert():
    E, k = 8, 2
    cfg, lw = _tiny_layer(E, k)
    u = RNG.normal(size=(12, cfg.d_model))
    z = u @ om.f64(lw["w_router"]).T
    z[:, 0] = -1e9  # expert 0 never selected
    idx, w = om.route(z, k)
    got = om.moe(u, idx, w, lw, E)
    per_token = np.stack([
        om.swiglu(u[t:t + 1], lw["ws_gate"], lw["ws_up"], lw["ws_down"])[0]
        + sum(w[t, j] * om.swiglu(u[t:t + 1], lw["w_gate"][idx[t, j]], lw["w_up"][idx[t, j]],
                                  lw["w_down"][idx[t, j]])[0] for j in range(k))
        for t in range(12)])
    assert np.allclose(got, per_token, rtol=1e-12, atol=1e-14)
    lw2 = dict(lw)
    lw2["w_down"] = lw["w_down"].clone()
    lw2["w_down"][0] = 100.0
    assert np.array_equal(om.moe(u, idx, w, lw2, E), got)


def test_swiglu_matches_torch_composition():
    # torch's silu (a library routine: x * sigmoid(x)) gating the gate
    # projection, times the up projection, then the down projection.
    d, F_ = 24, 40
    x = RNG.normal(size=(7, d))
    wg, wu, wd = (RNG.normal(size=s) * 0.3 for s in ((F_, d), (F_, d), (d, F_)))
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    want = (F.silu(t(x) @ t(wg).T) * (t(x) @ t(wu).T)) @ t(wd).T
    assert np.allclose(om.swiglu(x, wg, wu, wd), want.numpy(), rtol=1e-12, atol=1e-14)


def test_swiglu_gate_and_up_are_not_interchangeable():
    # one hidden unit with gate pre-activation a = 20 and up pre-activation
    # b = -20, identity down projection: silu(a) * b = -20 * 20 / (1 + e^-20)
    # (about -400), whereas silu(b) * a would be about -4e-8.
    x = np.array([[1.0, 0.0]])
    wg = np.array([[20.0, 0.0]])
    wu = np.array([[-20.0, 0.0]])
    wd = np.array([[1.0]])
    got = float(om.swiglu(x, wg, wu, wd)[0, 0])
    assert abs(got - (-400.0 / (1.0 + np.exp(-20.0)))) < 1e-9
    # silu's closed forms: silu(0) = 0 and silu(2) = 2 sigmoid(2)
    assert om.silu(np.array([0.0]))[0] == 0.0
    assert abs(om.silu(np.array([2.0]))[0] - 2.0 / (1.0 + np.exp(-2.0))) < 1e-15


# ----------------------------------------------------------------------------- LM head + sampler

def test_row_stats_match_numpy_and_scipy():
    L = RNG.normal(size=(7, 300)) * 3
    L[2, 10] = L[2, 20] = L[2].max() + 1  # tie: first index wins
    held = RNG.integers(0, 300, size=7)
    tau = 0.6
    M, a, logZ, gx = om.row_stats(L, held, tau)
    assert np.array_equal(a, np.argmax(L, 1)) and a[2] == 10
    assert np.array_equal(M, L.max(1))
    assert np.allclose(logZ, scipy.special.logsumexp(L / tau, axis=1) - M / tau, rtol=1e-13)
    c = (gx - M) / tau - logZ
    assert np.allclose(c, scipy.special.log_softmax(L / tau, axis=1)[np.arange(7), held],
                       rtol=1e-12, atol=1e-12)


def test_pages_constants_and_schedule():
    consts = {r[0]: float(r[1]) for r in golden("sampler_constants.txt")}
    cfg = synth.FULL
    assert cfg.tau_first == consts["tau_first"] and cfg.tau_last == consts["tau_last"]
    assert cfg.canvas == consts["canvas"] and cfg.n_experts == consts["n_experts"]
    assert cfg.top_k == consts["top_k"]
    S = int(consts["max_steps"])
    assert om.tau_at(1, S, 0.8, 0.4) == 0.8 and abs(om.tau_at(S, S, 0.8, 0.4) - 0.4) < 1e-15
    taus = [om.tau_at(s, S, 0.8, 0.4) for s in range(1, S + 1)]
    assert np.allclose(np.diff(taus), -0.4 / (S - 1))  # linear descent
    for S in (4, 12, 16, 48):
        ks = [om.commit_count(s, S, 256) for s in range(1, S + 1)]
        assert ks[-1] == 256 and all(b >= a for a, b in zip(ks, ks[1:]))


def test_sampler_invariants_over_a_block():
    V, C, S = 97, 40, 5
    x, m = om.init_canvas(3, 0, 0, C, V)
    assert not m.any() and x.min() >= 0 and x.max() < V
    for s in range(1, S + 1):
        L = RNG.normal(size=(C, V)) * 2
        tau = om.tau_at(s, S, 0.8, 0.4)
        M, a, logZ, gx = om.row_stats(L, x, tau)
        x2, m2, c, acc = om.sample(x, m, M, a, logZ, gx, tau, s, S, 3, 0, 0, V)
        assert x2.min() >= 0 and x2.max() < V
        assert m2.sum() == om.commit_count(s, S, C) == acc.sum()
        # a held token stays unless its position is re-noised
        kept = m.astype(bool) & acc
        assert np.array_equal(x2[kept], x[kept])
        # newly accepted positions take the argmax
        new = ~m.astype(bool) & acc
        assert np.array_equal(x2[new], a[new])
        # accepted = the k_s highest confidences
        thr = np.sort(c)[::-1][m2.sum() - 1]
        assert np.all(c[acc] >= thr) and np.all(c[~acc] <= thr)
        # re-noised positions draw the Philox stream of this step
        noise = uniform_ids(3, np.arange(C), s, 0, 0, V)
        assert np.array_equal(x2[~acc], noise[~acc])
        x, m = x2, m2
    assert m.all()


def test_sampler_float32_precision_agrees_with_float64_off_ties():
    # the float32 schedule is the float64 one to float32 rounding, exactly
    # 0.8 and 0.4 (as float32) at the ends
    for s_, S_ in [(1, 16), (7, 16), (16, 16), (1, 1), (3, 12)]:
        t32 = om.tau_at(s_, S_, 0.8, 0.4, precision="float32")
        assert isinstance(t32, np.float32)
        assert abs(float(t32) - om.tau_at(s_, S_, 0.8, 0.4)) <= 2e-7
    assert om.tau_at(1, 16, 0.8, 0.4, precision="float32") == np.float32(0.8)
    assert om.tau_at(16, 16, 0.8, 0.4, precision="float32") == np.float32(0.4)
    # float32 confidences equal the float64 ones to float32 rounding, and the
    # accepted set is the same wherever the boundary gap exceeds that rounding
    V, C = 211, 48
    for trial in range(20):
        L = RNG.normal(size=(C, V)) * 3
        x = RNG.integers(0, V, size=C)
        m = (RNG.random(C) < 0.4).astype(np.uint8)
        tau = om.tau_at(4, 9, 0.8, 0.4)
        M, a, logZ, gx = om.row_stats(L, x, tau)
        f = lambda v: np.asarray(v, np.float32)
        _, _, c64, acc64 = om.sample(x, m, M, a, logZ, gx, tau, 4, 9, 1, 0, 0, V)
        x32, m32, c32, acc32 = om.sample(x, m, f(M), a, f(logZ), f(gx), om.tau_at(4, 9, 0.8, 0.4, "float32"),
                                         4, 9, 1, 0, 0, V, precision="float32")
        assert c32.dtype == np.float32
        assert np.all(np.abs(c32 - c64) <= 1e-5 * (1 + np.abs(c64)))
        k = om.commit_count(4, 9, C)
        cs = np.sort(c64)[::-1]
        if cs[k - 1] - cs[k] > 1e-4 * (1 + abs(cs[k])):
            assert np.array_equal(acc32, acc64)


# ----------------------------------------------------------------------------- self-conditioning

def test_expected_embedding_closed_forms():
    V, d = 300, 12
    E = RNG.normal(size=(V, d)) * 0.5
    # equal logits: the uniform distribution gives the mean embedding row
    assert np.allclose(om.expected_embedding(np.full((2, V), 0.7), E, chunk=64), E.mean(0)[None].repeat(2, 0),
                       rtol=1e-12, atol=1e-14)
    # one logit far above the rest: a one-hot distribution picks that row
    L = RNG.normal(size=(3, V))
    L[np.arange(3), [5, 77, 299]] += 800.0
    assert np.allclose(om.expected_embedding(L, E, chunk=64), E[[5, 77, 299]], rtol=0, atol=1e-12)
    # two tokens with odds 3 : 1 (temperature 1): 3/4 E_a + 1/4 E_b
    L = np.full((1, V), -1e4)
    L[0, 10], L[0, 200] = np.log(3.0), 0.0
    assert np.allclose(om.expected_embedding(L, E, chunk=64)[0], 0.75 * E[10] + 0.25 * E[200], atol=1e-12)
    # random rows: scipy's softmax times E
    L = RNG.normal(size=(4, V)) * 3
    assert np.allclose(om.expected_embedding(L, E, chunk=64), scipy.special.softmax(L, axis=1) @ E,
                       rtol=1e-12, atol=1e-14)


def test_self_condition_is_the_feed_forward_layer_of_the_expected_embedding():
    V, d, F_ = 200, 16, 24
    E = RNG.normal(size=(V, d)) * 0.3
    sc = {"sc_gate": RNG.normal(size=(F_, d)), "sc_up": RNG.normal(size=(F_, d)), "sc_down": RNG.normal(size=(d, F_))}
    L = RNG.normal(size=(5, V)) * 2
    e = scipy.special.softmax(L, axis=1) @ E
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    want = (F.silu(t(e) @ t(sc["sc_gate"]).T) * (t(e) @ t(sc["sc_up"]).T)) @ t(sc["sc_down"]).T
    assert np.allclose(om.self_condition(L, E, sc), want.numpy(), rtol=1e-11, atol=1e-13)


def test_self_conditioning_in_the_loop():
    # zero layers: logits = RMSNorm(E[x] + s) E^T, with s added only after the first step
    cfg, hw = _tiny_model(n_layers=0)
    sc = synth.make_selfcond_weights(cfg, 64, 0)
    sc = {k: v.float() * 40.0 for k, v in sc.items()}  # large enough to move the logits
    req = om.Request(cfg, 128)
    x, m = om.init_canvas(5, 0, 0, cfg.canvas, cfg.vocab)
    k1, k1_plain = {}, {}
    x1, m1 = om.denoise_step(hw, cfg, req, x, m, 1, 4, 5, 0, 0, keep=k1, sc=sc, sc_prev=None)
    om.denoise_step(hw, cfg, req, x, m, 1, 4, 5, 0, 0, keep=k1_plain)
    assert np.array_equal(k1["logits"], k1_plain["logits"])  # nothing added at the first step
    E = om.f64(hw.embed)
    assert np.allclose(k1["sc"], om.self_condition(k1["logits"], hw.embed, sc), rtol=1e-12, atol=1e-14)
    k2 = {}
    om.denoise_step(hw, cfg, req, x1, m1, 2, 4, 5, 0, 0, keep=k2, sc=sc, sc_prev=k1["sc"])
    g = om.f64(hw.final_norm)
    h_in = torch.from_numpy(E[x1] + k1["sc"])
    hf = F.rms_norm(h_in, (cfg.d_model,), torch.from_numpy(g), eps=cfg.rms_eps).numpy()
    assert np.allclose(k2["logits"], hf @ E.T, rtol=1e-10, atol=1e-12)
    assert np.abs(k2["logits"] - hf @ E.T).max() < 1e-9 < np.abs(k1["sc"]).max()


def test_entropy_closed_forms_and_library():
    tau = 0.7
    # equal logits: the uniform distribution, H = log V
    for V in (5, 97, 4096):
        assert abs(om.row_entropy(np.full((1, V), 3.25), tau)[0] - np.log(V)) < 1e-12
    # two tokens: the binary entropy of p = sigmoid(x / tau)
    for x in (-3.0, 0.1, 2.5):
        p = 1.0 / (1.0 + np.exp(-x / tau))
        want = -(p * np.log(p) + (1 - p) * np.log(1 - p))
        assert abs(om.row_entropy(np.array([[0.0, x]]), tau)[0] - want) < 1e-12
    # k equal maxima far above the rest: H = log k (the rest underflow to p = 0)
    L = np.full((1, 64), -1e4)
    L[0, [3, 17, 40]] = 5.0
    assert abs(om.row_entropy(L, tau)[0] - np.log(3)) < 1e-12
    # random rows: scipy's entropy of the softmax, shift invariance, bounds
    L = RNG.normal(size=(9, 300)) * 2.5
    H = om.row_entropy(L, tau)
    want = scipy.stats.entropy(scipy.special.softmax(L / tau, axis=1), axis=1)
    assert np.allclose(H, want, rtol=1e-12, atol=1e-12)
    assert np.allclose(om.row_entropy(L + 7.0, tau), H, rtol=1e-12)
    assert np.all(H >= 0) and np.all(H <= np.log(300))
    # a lower temperature never raises the entropy (dH/dbeta = -beta Var_p(L) <= 0)
    Hs = np.stack([om.row_entropy(L, t) for t in (2.0, 1.0, 0.8, 0.6, 0.4, 0.2)])
    assert np.all(np.diff(Hs, axis=0) <= 1e-12)


def test_entropy_confidence_and_adaptive_stop():
    V, C, S, s = 53, 24, 6, 2
    L = RNG.normal(size=(C, V)) * 2
    L[5] = L[9]  # equal entropies: the lower position ranks first
    x, m = om.init_canvas(1, 0, 0, C, V)
    m = (np.arange(C) % 3 == 0).astype(np.uint8)
    tau = om.tau_at(s, S, 0.8, 0.4)
    M, a, logZ, gx = om.row_stats(L, x, tau)
    H = om.row_entropy(L, tau)
    x2, m2, c, acc = om.sample(x, m, M, a, logZ, gx, tau, s, S, 1, 0, 0, V, confidence="entropy", H=H)
    k_s = om.commit_count(s, S, C)
    order = sorted(range(C), key=lambda i: (H[i], i))
    assert np.array_equal(np.flatnonzero(acc), np.sort(order[:k_s]))
    assert np.array_equal(c, -H)
    y = np.where(m.astype(bool), x, a)
    assert np.array_equal(x2[acc], y[acc]) and m2.sum() == k_s
    # the stop rule: mean entropy below the threshold and an unchanged argmax
    thr_hi, thr_lo = H.mean() + 1e-9, H.mean() - 1e-9
    assert not om.adaptive_stop(H, a, None, thr_hi)
    assert om.adaptive_stop(H, a, a.copy(), thr_hi)
    assert not om.adaptive_stop(H, a, a.copy(), thr_lo)
    moved = a.copy()
    moved[C - 1] = (moved[C - 1] + 1) % V
    assert not om.adaptive_stop(H, a, moved, thr_hi)
    # a stopped step accepts every position with its candidate
    x3, m3, _, acc3 = om.sample(x, m, M, a, logZ, gx, tau, s, S, 1, 0, 0, V, confidence="entropy",
                                H=H, stop=True)
    assert acc3.all() and m3.all() and np.array_equal(x3, y)


def test_adaptive_stop_in_the_denoising_step():
    cfg, w = _tiny_model(n_layers=1)
    req = om.Request(cfg, 64 + 2 * cfg.canvas)
    om.prefill(w, cfg, req, synth.make_prompt(64, cfg.vocab, 0).numpy())
    x, m = om.init_canvas(0, 0, 0, cfg.canvas, cfg.vocab)
    k1, k2 = {}, {}
    om.denoise_step(w, cfg, req, x, m, 2, 8, 0, 0, 0, keep=k1, stop_entropy=1e9)
    assert not k1["stop"]  # no previous prediction
    # the same canvas again: same argmax, so any threshold above the mean stops it
    x2, m2 = om.denoise_step(w, cfg, req, x, m, 2, 8, 0, 0, 0, keep=k2, stop_entropy=1e9,
                             a_prev=k1["a"])
    assert k2["stop"] and m2.all() and np.array_equal(x2, np.where(m.astype(bool), x, k2["a"]))
    k3 = {}
    om.denoise_step(w, cfg, req, x, m, 2, 8, 0, 0, 0, keep=k3, stop_entropy=k1["H"].mean() * 0.5,
                    a_prev=k1["a"])
    assert not k3["stop"]
    assert np.allclose(k1["H"], om.row_entropy(k1["logits"], k1["tau"]))


def _gumbel_frequencies(L_row, tau, n, seed=7):
    L = np.tile(np.asarray(L_row, np.float64), (n, 1))
    ys, ly = om.gumbel_candidates(L, tau, seed, 3, 1, 0)
    assert np.array_equal(ly, L[np.arange(n), ys])
    return np.bincount(ys, minlength=L.shape[1]) / n


def test_gumbel_candidates_follow_the_tempered_softmax():
    """Gumbel-max: argmax_v (L_v / tau + G_v) is distributed as
    softmax(L / tau); a chi-square test over 20,000 positions."""
    L_row = np.array([0.3, -1.2, 1.1, 0.0, 0.7, -0.4])
    tau = 0.6
    n = 20000
    freq = _gumbel_frequencies(L_row, tau, n)
    p = scipy.special.softmax(L_row / tau)
    chi2 = n * np.sum((freq - p) ** 2 / p)
    assert scipy.stats.chi2.sf(chi2, len(p) - 1) > 1e-3, chi2
    # a vanishing temperature gives the argmax
    assert np.all(om.gumbel_candidates(np.tile(L_row, (50, 1)), 1e-4, 7, 3, 1, 0)[0] == 2)


def test_gumbel_uniforms_lie_on_the_23_bit_grid_inside_the_interval():
    u = philox_mod.gumbel_uniforms(11, 5, 2, 1, 3, 4096)
    assert np.all((u > 0) & (u < 1))
    g = u * (1 << 23) - 0.5
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)  # exact in float32
    assert np.array_equal(g, np.round(g))
    # the four ids that share a counter take its four words; other positions,
    # steps, blocks and requests draw other streams
    assert len(set(np.round(g[[0, 16, 32, 48]]).astype(int))) == 4
    for args in [(11, 6, 2, 1, 3), (11, 5, 3, 1, 3), (11, 5, 2, 2, 3), (11, 5, 2, 1, 4), (12, 5, 2, 1, 3)]:
        assert not np.array_equal(philox_mod.gumbel_uniforms(*args, 4096), u)


def test_sampled_candidates_in_the_sampler():
    V, C, S, s = 40, 16, 4, 2
    L = RNG.normal(size=(C, V)) * 2
    x, _ = om.init_canvas(2, 0, 0, C, V)
    m = (np.arange(C) % 4 == 1).astype(np.uint8)
    tau = om.tau_at(s, S, 0.8, 0.4)
    M, a, logZ, gx = om.row_stats(L, x, tau)
    drawn = om.gumbel_candidates(L, tau, 2, s, 0, 0)
    x2, m2, c, acc = om.sample(x, m, M, a, logZ, gx, tau, s, S, 2, 0, 0, V, drawn=drawn)
    y = np.where(m.astype(bool), x, drawn[0])
    assert np.allclose(c, scipy.special.log_softmax(L / tau, axis=1)[np.arange(C), y], atol=1e-12)
    assert np.array_equal(x2[acc], y[acc])


# ----------------------------------------------------------------------------- FP8 weights

def _torch_e4m3_codes(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_matches_the_format_and_torch():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = fp8.e4m3_decode(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(vals, want)
    assert fp8.e4m3_decode([0x7E])[0] == 448.0 and fp8.e4m3_decode([0x01])[0] == 2.0 ** -9
    assert fp8.e4m3_decode([0x08])[0] == 2.0 ** -6 and fp8.e4m3_decode([0x38])[0] == 1.0
    assert fp8.e4m3_decode([0xB8])[0] == -1.0 and fp8.e4m3_decode([0x07])[0] == 7 * 2.0 ** -9


def test_e4m3_encode_round_trip_ties_and_torch():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)
    # midpoints go to the even mantissa, in the normal and the subnormal range
    assert fp8.e4m3_decode(fp8.e4m3_encode([1 + 1 / 16, 1 + 3 / 16, 2.0 ** -9 * 1.5, 2.0 ** -9 * 0.5,
                                            2.0 ** -9 * 2.5, 416.0])).tolist() == \
        [1.0, 1.25, 2 * 2.0 ** -9, 0.0, 2 * 2.0 ** -9, 416.0]
    assert fp8.e4m3_encode([432.0])[0] == 0x7E  # 432 = midpoint of 416 and 448: even mantissa 6
    # random values across the range, subnormals included: torch's conversion
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-12, 8, 20000))).astype(np.float32)
    v = np.clip(v, -448, 448)
    assert np.array_equal(fp8.e4m3_encode(v), _torch_e4m3_codes(v))


def test_fp8_row_scaling_and_error_bound():
    assert fp8.row_exponent([448.0, 448.0001, 224.0, 449.0, 0.0, 896.0, 1.0]).tolist() == \
        [0, 1, -1, 1, 0, 1, -8]
    W = synth.make_layer_weights(synth.TINY, 0, 4)["w_gate"].double().numpy().reshape(-1, synth.TINY.d_model)
    W[3] = 0.0
    codes, e = fp8.quantize_rows(W)
    amax = np.abs(W).max(1)
    nz = amax > 0
    assert np.all(amax[nz] <= 448 * np.exp2(e[nz])) and np.all(amax[nz] > 448 * np.exp2(e[nz] - 1.0))
    deq = fp8.dequantize_rows(codes, e)
    scaled = np.abs(W) * np.exp2(-e[:, None])
    normal = scaled >= 2.0 ** -6
    err = np.abs(deq - W)
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(W[normal]))  # half an ulp of a 3-bit mantissa
    assert np.all(err[~normal] <= (2.0 ** -10 * np.exp2(e[:, None]) * np.ones_like(W))[~normal])
    assert np.all(deq[3] == 0) and np.all(codes[3] & 0x7F == 0)
    # dequantising the codes reproduces the quantised bank exactly
    assert np.array_equal(fp8.dequantize_bank(W), deq)


# ----------------------------------------------------------------------------- whole step

def _tiny_model(n_layers=1, gain_jitter=0.1, **kw):
    cfg = dataclasses.replace(synth.TINY, n_layers=n_layers, **kw)
    return cfg, synth.ModelWeights(cfg, 0, gain_jitter=gain_jitter)


def test_zero_layer_model_is_normed_embedding_times_embedding():
    cfg, w = _tiny_model(n_layers=0)
    req = om.Request(cfg, 128)
    x, m = om.init_canvas(0, 0, 0, cfg.canvas, cfg.vocab)
    keep = {}
    om.denoise_step(w, cfg, req, x, m, 1, 4, 0, 0, 0, keep=keep)
    E = w.embed.double()
    hf = F.rms_norm(E[torch.from_numpy(x)], (cfg.d_model,), w.final_norm.double(), eps=1e-6)
    assert np.allclose(keep["logits"], (hf @ E.T).numpy(), rtol=1e-10, atol=1e-12)


def test_prefill_then_commit_equals_one_longer_prefill():
    cfg, w = _tiny_model(n_layers=2)
    prompt = synth.make_prompt(48, cfg.vocab, 0).numpy()
    block = synth.make_prompt(cfg.canvas, cfg.vocab, 1).numpy()
    a = om.Request(cfg, 128)
    om.prefill(w, cfg, a, prompt)
    k_before = a.k.copy()
    om.commit_block(w, cfg, a, block)
    # committed rows are never rewritten
    assert np.array_equal(a.k[:, :48], k_before[:, :48])
    b = om.Request(cfg, 128)
    om.prefill(w, cfg, b, np.concatenate([prompt, block]))
    assert a.length == b.length == 48 + cfg.canvas
    assert np.allclose(a.k, b.k, rtol=1e-10, atol=1e-12)
    assert np.allclose(a.v, b.v, rtol=1e-10, atol=1e-12)


def test_denoise_leaves_cache_untouched_and_full_block_loop_runs():
    cfg, w = _tiny_model(n_layers=1)
    req = om.Request(cfg, 64 + 2 * cfg.canvas)
    om.prefill(w, cfg, req, synth.make_prompt(64, cfg.vocab, 0).numpy())
    k0, v0 = req.k.copy(), req.v.copy()
    x, m = om.init_canvas(0, 0, 0, cfg.canvas, cfg.vocab)
    x2, m2 = om.denoise_step(w, cfg, req, x, m, 1, 4, 0, 0, 0)
    assert np.array_equal(req.k, k0) and np.array_equal(req.v, v0) and req.length == 64
    assert m2.sum() == 8
    x_final, m_final, taken = om.generate_block(w, cfg, req, 4, 0, 0, 0)
    assert taken == 4
    assert m_final.all() and req.length == 64 + cfg.canvas


def test_ar_step_equals_a_full_causal_pass():
    """The incremental decode step (cached prefix + one row) against a causal
    pass over the whole sequence from an empty cache: the same K/V rows and
    the same last-row logits, so the same next token."""
    cfg, w = _tiny_model(n_layers=2)
    prompt = synth.make_prompt(40, cfg.vocab, 3).numpy().astype(np.int64)
    req = om.Request(cfg, 64)
    om.prefill(w, cfg, req, prompt)
    tok = int(prompt[-1])
    seq = list(prompt)
    for _ in range(3):
        nxt, L = om.ar_step(w, cfg, req, tok)
        seq.append(tok)
        full = om.Request(cfg, 64)
        h, ks, vs = om.forward_rows(w, cfg, full, np.asarray(seq, np.int64), causal=True)
        L_full = om.logits(h[-1:], w.final_norm, w.embed, cfg)[0]
        assert np.allclose(L, L_full, rtol=1e-9, atol=1e-9)
        assert nxt == int(np.argmax(L_full))
        for l in range(cfg.n_layers):
            assert np.allclose(req.k[l, :len(seq)], ks[l], rtol=1e-9, atol=1e-12)
            assert np.allclose(req.v[l, :len(seq)], vs[l], rtol=1e-9, atol=1e-12)
        assert req.length == len(seq)
        tok = nxt


# ----------------------------------------------------------------------------- metrics

def test_throughput_worked_example():
    vals = {r[0]: float(r[1]) for r in golden("throughput_worked_example.txt")}
    tps = metrics.tokens_per_second(vals["tpf"], vals["t_fwd_ms"] / 1e3)
    assert round(tps) == int(vals["tps"])
    # one block, S steps: TPF = C / S; K blocks add K - 1 commit forwards
    assert metrics.tokens_per_forward(256, 16, 1) == 16.0
    assert abs(metrics.tokens_per_forward(1024, 48, 4) - 1024 / 51) < 1e-12
