"""Pins for the oracle's further static primitives: dilated/strided, blockwise and
BigBird-style random blocks ("sparse attention mechanism" glossary, table "Sparse
Attention Patterns"), OR-composed as in "SAS: Sparse Attention Synthesizer", Step 5.

The generator is pinned to its published outputs, the element mask to plain loops over
the definitions and to closed-form row counts, and the attention path to torch's SDPA
with the same mask.
"""
import math

import numpy as np
import pytest
import torch

from oracle import bsfa_oracle as orc
from oracle.bsfa_oracle import MaskSpec


def test_splitmix64_published_sequence():
    """SplitMix64 from state 0 (Steele, Lea and Flood, 2014): the generator adds the
    golden gamma to its state before each output, so output k is splitmix64(k * gamma).
    These are the reference implementation's first four outputs."""
    gamma = 0x9E3779B97F4A7C15
    got = [orc.splitmix64((k * gamma) % (1 << 64)) for k in range(4)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F,
                   0xF88BB8A8724C81EC]


def _allowed_loop(i, j, n, spec):
    """The definition, one pair at a time, in plain Python."""
    if not (0 <= i < n and 0 <= j < n):
        return False
    if spec.causal and j > i:
        return False
    prims = []
    if spec.window > 0:
        prims.append(abs(i - j) < spec.window)
    if spec.dilation > 0:
        hit = (i - j) % spec.dilation == 0
        if spec.dilation_taps > 0:
            hit = hit and abs(i - j) < spec.dilation * spec.dilation_taps
        prims.append(hit)
    if spec.block > 0:
        prims.append(i // spec.block == j // spec.block)
    if spec.random_ppm > 0:
        prims.append(orc.random_block_selected(spec.random_seed, i // 64, j // 64,
                                               spec.random_ppm))
    if not prims:
        return True
    return any(prims) or j < spec.n_global or i < spec.n_global


SPECS = [
    MaskSpec(causal=True, dilation=3, dilation_taps=5),
    MaskSpec(causal=False, dilation=7),
    MaskSpec(causal=True, block=50),
    MaskSpec(causal=False, block=64),
    MaskSpec(causal=True, random_ppm=250_000, random_seed=3),
    MaskSpec(causal=False, window=9, n_global=4, dilation=16, dilation_taps=3, block=40,
             random_ppm=100_000, random_seed=11),
]


@pytest.mark.parametrize("spec", SPECS)
def test_element_mask_matches_definition_loop(spec):
    n = 200
    m = orc.element_mask(range(-2, n + 2), range(-2, n + 2), n, spec)
    for a, i in enumerate(range(-2, n + 2)):
        for b, j in enumerate(range(-2, n + 2)):
            assert m[a, b] == _allowed_loop(i, j, n, spec), (i, j)


def test_closed_form_row_counts():
    n = 500
    rows = np.arange(n)
    # blockwise, causal: row i sees the keys of its block up to itself
    m = orc.element_mask(rows, rows, n, MaskSpec(causal=True, block=37))
    np.testing.assert_array_equal(m.sum(1), rows % 37 + 1)
    # blockwise, both directions: the size of i's block (the last one is short)
    m = orc.element_mask(rows, rows, n, MaskSpec(causal=False, block=37))
    size = np.minimum(37, n - (rows // 37) * 37)
    np.testing.assert_array_equal(m.sum(1), size)
    # dilated with taps, causal: i, i - k, ..., at most `taps` of them
    m = orc.element_mask(rows, rows, n, MaskSpec(causal=True, dilation=6, dilation_taps=4))
    np.testing.assert_array_equal(m.sum(1), np.minimum(rows // 6 + 1, 4))
    # dilated without a limit, both directions: every key of i's residue class mod k
    m = orc.element_mask(rows, rows, n, MaskSpec(causal=False, dilation=6))
    np.testing.assert_array_equal(m.sum(1), (n - 1 - rows % 6) // 6 + 1)


def test_random_block_rate():
    """Over 64 x 64 block pairs the selected share follows the rate (binomial, 5 sigma)."""
    nb = 64
    for ppm in (50_000, 300_000, 700_000):
        hits = sum(orc.random_block_selected(5, t, c, ppm) for t in range(nb) for c in range(nb))
        p = ppm / 1e6
        sigma = math.sqrt(nb * nb * p * (1 - p))
        assert abs(hits - nb * nb * p) < 5 * sigma
    assert not any(orc.random_block_selected(5, t, c, 0) for t in range(8) for c in range(8))
    assert all(orc.random_block_selected(5, t, c, 1_000_000) for t in range(8) for c in range(8))
    # whole blocks: every element of a 64 x 64 block shares the decision
    spec = MaskSpec(causal=False, random_ppm=400_000, random_seed=9)
    m = orc.element_mask(range(256), range(256), 256, spec)
    blocks = m.reshape(4, 64, 4, 64)
    assert np.all(blocks.all(axis=(1, 3)) == blocks.any(axis=(1, 3)))


def test_primitives_or_compose():
    n = 300
    rows = np.arange(n)
    parts = [MaskSpec(causal=True, window=20), MaskSpec(causal=True, dilation=9),
             MaskSpec(causal=True, block=70), MaskSpec(causal=True, random_ppm=200_000)]
    union = MaskSpec(causal=True, window=20, dilation=9, block=70, random_ppm=200_000)
    acc = np.zeros((n, n), dtype=bool)
    for p in parts:
        acc |= orc.element_mask(rows, rows, n, p)
    np.testing.assert_array_equal(orc.element_mask(rows, rows, n, union), acc)


def _sdpa(q, k, v, mask):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=t(mask)).numpy()


@pytest.mark.parametrize("spec", [
    MaskSpec(causal=True, block=48, n_global=8),
    MaskSpec(causal=True, dilation=5, dilation_taps=20, window=16),
    MaskSpec(causal=True, window=32, random_ppm=300_000, random_seed=2),
])
def test_attention_with_pattern_equals_sdpa(spec):
    """Dense path (tau=None) under a pattern equals SDPA with that boolean mask, built
    here from the definition loop."""
    n, d = 257, 8
    rng = np.random.default_rng(17)
    q, k, v = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    mask = np.array([[_allowed_loop(i, j, n, spec) for j in range(n)] for i in range(n)])
    assert mask.any(1).all()  # every row attends to something in these cases
    r = orc.attention(q, k, v, spec, tau=None)
    np.testing.assert_allclose(r.full_out()[:, :, :n], _sdpa(q, k, v, mask), atol=1e-12)
