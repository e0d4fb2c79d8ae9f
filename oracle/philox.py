"""Philox4x32-10 counter-based generator, and the uniform token ids drawn from it.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline may use this module; the product path never does.

The pages say only that low-confidence canvas positions go back to a token
drawn uniformly from the vocabulary (codemajin.net DiffusionGemma explainer,
§3.3; aibars.net news item, "Uniform State Diffusion" paragraph; aiboss88.com
product page, "technical principles": the canvas starts from random
placeholders). The generator that draws them is our reading: Philox4x32 with
10 rounds, as published by Salmon, Moraes, Dror and Shaw ("Parallel random
numbers: as easy as 1, 2, 3", SC'11), restated here from that definition.

Mapping used by both sides of the build:
  key     = (low 32 bits of seed, high 32 bits of seed)
  counter = (position i, step s, block b, request r); s = 0 draws the
            initial canvas
  id      = (word0 * V) >> 32, which is word0 >> (32 - log2 V) when V is a
            power of two.

Gumbel noise for sampling candidates (our reading as well): the uniform of
vocabulary id v at canvas position i is word ((v >> 4) & 3) of
  Philox(key, counter = (v with bits 4 and 5 cleared, i,
                         (block << 16) | step, 0x80000000 | request)),
as u = ((word >> 9) + 1/2) / 2^23, strictly inside (0, 1) and exact in
float32. The top bit of the last counter word keeps these streams apart from
the re-noise draws.
"""
from __future__ import annotations

import numpy as np

_MUL0 = np.uint64(0xD2511F53)
_MUL1 = np.uint64(0xCD9E8D57)
_WEYL0 = 0x9E3779B9
_WEYL1 = 0xBB67AE85
_LO = np.uint64(0xFFFFFFFF)
_SH = np.uint64(32)


def philox4x32_10(counter, key):
    """Apply the 10-round Philox4x32 bijection.

    counter: array [..., 4] of uint32 values; key: array [..., 2] (broadcast).
    Returns uint32 array [..., 4].
    """
    c = np.asarray(counter, dtype=np.uint64) & _LO
    k = np.asarray(key, dtype=np.uint64) & _LO
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0 = np.broadcast_to(k[..., 0], c0.shape).copy()
    k1 = np.broadcast_to(k[..., 1], c0.shape).copy()
    for rnd in range(10):
        if rnd > 0:  # the key is bumped by the Weyl constants between rounds
            k0 = (k0 + np.uint64(_WEYL0)) & _LO
            k1 = (k1 + np.uint64(_WEYL1)) & _LO
        p0 = _MUL0 * c0  # 32x32 -> 64-bit products are exact in uint64
        p1 = _MUL1 * c2
        hi0, lo0 = p0 >> _SH, p0 & _LO
        hi1, lo1 = p1 >> _SH, p1 & _LO
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def seed_key(seed: int):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint64)


def uniform_ids(seed: int, positions, step: int, block: int, request: int,
                vocab: int) -> np.ndarray:
    """Uniform token ids for canvas positions at (step, block, request)."""
    pos = np.asarray(positions, dtype=np.uint64)
    ctr = np.zeros(pos.shape + (4,), dtype=np.uint64)
    ctr[..., 0] = pos
    ctr[..., 1] = np.uint64(step)
    ctr[..., 2] = np.uint64(block)
    ctr[..., 3] = np.uint64(request)
    w0 = philox4x32_10(ctr, seed_key(seed))[..., 0].astype(np.uint64)
    return ((w0 * np.uint64(vocab)) >> _SH).astype(np.int64)


def gumbel_uniforms(seed: int, position: int, step: int, block: int, request: int,
                    vocab: int) -> np.ndarray:
    """The uniforms u_v (float64, exact) of one canvas position, v = 0..V-1."""
    v = np.arange(vocab, dtype=np.uint64)
    ctr = np.zeros((vocab, 4), dtype=np.uint64)
    ctr[:, 0] = v & ~np.uint64(0x30)
    ctr[:, 1] = np.uint64(position)
    ctr[:, 2] = (np.uint64(block) << np.uint64(16)) | np.uint64(step)
    ctr[:, 3] = np.uint64(0x80000000) | np.uint64(request)
    words = philox4x32_10(ctr, seed_key(seed))
    w = words[np.arange(vocab), ((v >> np.uint64(4)) & np.uint64(3)).astype(np.int64)].astype(np.uint64)
    return ((w >> np.uint64(9)).astype(np.float64) + 0.5) / float(1 << 23)
