"""Host-side layout helpers (no GPU): the V block order of the KV cache and
the fragment-major weight order, checked against the index formulas that
include/dg.h states."""
import numpy as np
import torch

from block_discrete_diffusion_dg_amd.engine import v_from_cache_order, v_to_cache_order


def test_v_cache_order_matches_header_formula():
    heads, n, dh = 2, 96, 16
    v = torch.arange(heads * n * dh, dtype=torch.int64).reshape(heads, n, dh)
    raw = v_to_cache_order(v)
    assert torch.equal(v_from_cache_order(raw), v)
    flat = raw.reshape(heads, -1)
    rng = np.random.default_rng(0)
    for _ in range(200):
        hd, pos, c = int(rng.integers(heads)), int(rng.integers(n)), int(rng.integers(dh))
        b, o = divmod(pos, 32)
        h, rest = divmod(o, 16)
        g, r = divmod(rest, 4)
        idx = 32 * dh * b + (g * dh + c) * 8 + 4 * h + r
        assert flat[hd, idx] == v[hd, pos, c]


def test_v_cache_order_is_a_permutation_within_blocks():
    v = torch.arange(64 * 8).reshape(64, 8)
    raw = v_to_cache_order(v).reshape(-1)
    # block 0 holds exactly positions 0..31, block 1 positions 32..63
    assert sorted(raw[:256].tolist()) == list(range(256))
    assert sorted(raw[256:].tolist()) == list(range(256, 512))
