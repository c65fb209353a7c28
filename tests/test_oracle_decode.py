"""Pins for the oracle's decode step (one new query row per sequence and head against a
key/value cache; "SAS: Sparse Attention Synthesizer", Challenge 2 "KV Cache Management"
and Step 6; the gate of "Block Sparse Flash Attention", "The paper's summary").

The dense path is pinned to torch's fp64 scaled_dot_product_attention over the cached
rows; the gate to closed forms (Q = 0, tau = +inf, a window-cut block whose masked keys
would pass the gate) and to plain loops over the definitions; lengths to their edge
cases.
"""
import math

import numpy as np
import pytest
import torch

from oracle import bsfa_oracle as orc
from oracle.bsfa_oracle import MaskSpec


def _sdpa_row(q_row, k, v, mask_row=None):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    qq = t(q_row)[None, None, None, :]
    kk, vv = t(k)[None, None], t(v)[None, None]
    m = None if mask_row is None else torch.from_numpy(np.asarray(mask_row))[None, None, None]
    return torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m)[0, 0, 0].numpy()


def _inputs(bsz=2, hq=4, hkv=2, lmax=300, d=16, seed=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((bsz, hq, d))
    k = rng.standard_normal((bsz, hkv, lmax, d))
    v = rng.standard_normal((bsz, hkv, lmax, d))
    return q, k, v


def test_dense_decode_equals_sdpa_and_logsumexp():
    q, k, v = _inputs()
    lengths = [300, 171]
    r = orc.decode(q, k, v, lengths, MaskSpec(causal=True), tau=None)
    scale = 1.0 / math.sqrt(q.shape[-1])
    for b, n in enumerate(lengths):
        for h in range(4):
            g = h // 2
            ref = _sdpa_row(q[b, h], k[b, g, :n], v[b, g, :n])
            np.testing.assert_allclose(r.out[b, h], ref, atol=1e-12)
            s = torch.from_numpy(scale * (k[b, g, :n] @ q[b, h]))
            assert abs(r.lse[b, h] - float(torch.logsumexp(s, 0))) < 1e-12


def _allowed(i, j, n, spec):
    if not (0 <= j < n and 0 <= i < n) or (spec.causal and j > i):
        return False
    if not spec.has_pattern:
        return True
    return (abs(i - j) < spec.window if spec.window else False) or j < spec.n_global \
        or i < spec.n_global


def test_window_and_global_decode_equals_masked_sdpa():
    q, k, v = _inputs(lmax=400)
    spec = MaskSpec(causal=True, window=90, n_global=5)
    lengths = [400, 233]
    r = orc.decode(q, k, v, lengths, spec, tau=None)
    for b, n in enumerate(lengths):
        mask = np.array([_allowed(n - 1, j, n, spec) for j in range(n)])
        for h in range(4):
            ref = _sdpa_row(q[b, h], k[b, h // 2, :n], v[b, h // 2, :n], mask)
            np.testing.assert_allclose(r.out[b, h], ref, atol=1e-12)


def test_tau_inf_keeps_forced_blocks_only():
    """tau = +inf: only the block holding the row's own key and the global blocks stay,
    so the result is SDPA over exactly those keys."""
    q, k, v = _inputs(lmax=500)
    spec = MaskSpec(causal=True, n_global=70)
    lengths = [500, 260]
    r = orc.decode(q, k, v, lengths, spec, tau=np.inf)
    for b, n in enumerate(lengths):
        diag = (n - 1) // 64
        keys = [j for j in range(n) if j // 64 == diag or j // 64 <= (70 - 1) // 64]
        for h in range(4):
            ref = _sdpa_row(q[b, h], k[b, h // 2, keys], v[b, h // 2, keys])
            np.testing.assert_allclose(r.out[b, h], ref, atol=1e-12)
            assert r.keep[b, h].sum() == len({j // 64 for j in keys})


def test_zero_query_closed_forms():
    """Q = 0 makes every score and block maximum 0: tau = 0 keeps every allowed block
    (O = mean of the allowed values, LSE = ln of their count); tau = 0.5 keeps only the
    forced block (O = mean of its values)."""
    _, k, v = _inputs(lmax=330)
    q = np.zeros((2, 4, 16))
    lengths = [330, 129]
    spec = MaskSpec(causal=True, window=100)
    r0 = orc.decode(q, k, v, lengths, spec, tau=0.0)
    r1 = orc.decode(q, k, v, lengths, spec, tau=0.5)
    for b, n in enumerate(lengths):
        allowed = [j for j in range(n) if n - 1 - j < 100]
        own = [j for j in allowed if j // 64 == (n - 1) // 64]
        for h in range(4):
            vv = v[b, h // 2]
            np.testing.assert_allclose(r0.out[b, h], vv[allowed].mean(0), atol=1e-12)
            assert abs(r0.lse[b, h] - math.log(len(allowed))) < 1e-12
            np.testing.assert_allclose(r1.out[b, h], vv[own].mean(0), atol=1e-12)


@pytest.mark.parametrize("block_k", [1, 3, 64])
def test_brute_force_loops(block_k):
    """Every step written as plain loops: scores, mask, block maxima, gate, weights."""
    rng = np.random.default_rng(11)
    bsz, hq, hkv, lmax, d = 2, 2, 1, 130, 4
    q = rng.standard_normal((bsz, hq, d))
    k = rng.standard_normal((bsz, hkv, lmax, d))
    v = rng.standard_normal((bsz, hkv, lmax, d))
    lengths = [130, 67]
    spec = MaskSpec(causal=True, window=40, n_global=3)
    tau = [0.2, -0.1]
    r = orc.decode(q, k, v, lengths, spec, tau=tau, block_k=block_k)
    scale = 1.0 / math.sqrt(d)
    for b, n in enumerate(lengths):
        i = n - 1
        for h in range(hq):
            s = {j: scale * sum(q[b, h, x] * k[b, 0, j, x] for x in range(d))
                 for j in range(n) if _allowed(i, j, n, spec)}
            kept = []
            for c in range((n + block_k - 1) // block_k):
                js = [j for j in s if j // block_k == c]
                if not js:
                    continue
                forced = (c * block_k <= i < (c + 1) * block_k) or c * block_k < 3
                if forced or max(s[j] for j in js) >= tau[h]:
                    kept += js
            top = max(s[j] for j in kept)
            w = {j: math.exp(s[j] - top) for j in kept}
            tot = sum(w.values())
            ref = sum(w[j] / tot * v[b, 0, j] for j in kept)
            np.testing.assert_allclose(r.out[b, h], ref, atol=1e-12)
            assert abs(r.lse[b, h] - (top + math.log(tot))) < 1e-12


def test_decode_matches_prefill_row_with_single_row_tiles():
    """The decode step is the prefill rule with a one-row query tile at the newest row."""
    q, k, v = _inputs(bsz=1, lmax=257)
    n = 257
    qf = np.zeros((1, 4, n, 16))
    qf[0, :, n - 1] = q[0]
    spec = MaskSpec(causal=True, window=70, n_global=2)
    tau = [0.1, 0.3, -0.2, 0.0]
    r = orc.decode(q, k, v, [n], spec, tau=tau)
    p = orc.attention(qf, k, v, spec, tau=tau, block_q=1, q_tiles=[n - 1])
    np.testing.assert_allclose(r.out[0], p.out[0, :, 0, 0], atol=1e-12)
    np.testing.assert_array_equal(r.keep[0], p.keep[0, :, 0])


def test_length_edges():
    q, k, v = _inputs(lmax=200)
    r = orc.decode(q, k, v, [0, 999], MaskSpec(causal=True), tau=None)
    assert np.all(r.out[0] == 0) and np.all(r.lse[0] == -np.inf)
    assert not r.allowed[0].any()
    full = orc.decode(q, k, v, [200, 200], MaskSpec(causal=True), tau=None)
    np.testing.assert_array_equal(r.out[1], full.out[1])  # clamped to the cache size
    one = orc.decode(q, k, v, [1, 1], MaskSpec(causal=True), tau=None)
    np.testing.assert_allclose(one.out[:, 0], v[:, 0, 0], atol=1e-15)  # a single key


def test_calibration_hits_target_and_monotone_keep():
    q, k, v = _inputs(bsz=2, lmax=1200, seed=7)
    lengths = [1200, 900]
    spec = MaskSpec(causal=True)
    taus = orc.calibrate_tau_decode(q, k, lengths, spec, 0.5)
    r = orc.decode(q, k, v, lengths, spec, tau=taus)
    eligible = r.allowed & ~r.forced
    for h in range(4):
        skipped = (eligible & ~r.keep[:, h]).sum()
        # numpy's interpolated median: half of the eligible blocks fall strictly below it
        assert abs(skipped - eligible.sum() / 2) <= 1
    lo = orc.decode(q, k, v, lengths, spec, tau=taus - 0.3)
    assert np.all(lo.keep >= r.keep)


@pytest.mark.parametrize("quantile,expected", [(0.5, 2.0), (0.25, 1.0), (0.9, 2.6), (0.0, 1.0)])
def test_calibration_closed_form(quantile, expected):
    """Closed form of the decode threshold: with key block c's largest score c + 1 for
    head 0 (twice that for head 1), the rows at positions 255 and 191 have eligible
    blocks {0, 1, 2} and {0, 1} (their own block is forced), so head 0's pooled maxima
    are [1, 1, 2, 2, 3] and tau is their linear-interpolation quantile."""
    lmax = 256
    rng = np.random.default_rng(5)
    x = np.empty(lmax)
    for c in range(4):
        blk = rng.uniform(-1.0, c + 0.5, 64)
        blk[int(rng.integers(0, 64))] = c + 1.0
        x[c * 64:(c + 1) * 64] = blk
    k = np.zeros((2, 1, lmax, 2))
    k[:, 0, :, 0] = x
    q = np.zeros((2, 2, 2))
    q[:, 0, 0] = 1.0
    q[:, 1, 0] = 2.0
    taus = orc.calibrate_tau_decode(q, k, [256, 192], MaskSpec(causal=True), quantile, scale=1.0)
    np.testing.assert_allclose(taus, [expected, 2.0 * expected], rtol=0, atol=1e-12)


def test_gate_ignores_statically_masked_keys():
    """Closed form: in the block that the window cuts, the keys outside the window score
    high and the keys inside score low, with tau between them. The block's maximum is
    taken over its allowed keys only, so it is skipped. Only the row's own block is kept,
    and its keys all score 0, so O is the mean of their values and LSE = ln(count)."""
    n, d, w = 200, 4, 50  # row 199 sees keys [150, 199]; block 2 holds 128..191
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1.0
    k = np.zeros((1, 1, n, d))
    k[0, 0, 128:150, 0] = 40.0   # masked by the window, scaled scores 20
    k[0, 0, 150:192, 0] = -4.0   # allowed, scaled scores -2
    v = np.random.default_rng(3).standard_normal((1, 1, n, d))
    spec = MaskSpec(causal=True, window=w)
    r = orc.decode(q, k, v, [n], spec, tau=0.0)
    assert r.allowed[0].tolist() == [False, False, True, True]
    assert r.keep[0, 0].tolist() == [False, False, False, True]
    np.testing.assert_allclose(r.out[0, 0], v[0, 0, 192:200].mean(0), atol=1e-12)
    assert abs(r.lse[0, 0] - math.log(8)) < 1e-12
    assert abs(r.tile_max[0, 0, 2] - (-2.0)) < 1e-12
