"""Pins for the fp64 CPU oracle: each test ties it to something other than itself.

- values the pages print (tests/golden/*.json, each with its source),
- library routines (torch's fp64 CPU scaled_dot_product_attention),
- closed forms and invariants of the definition,
- a brute-force pure-Python loop implementation on tiny inputs (ragged N included).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import bsfa_oracle as orc
from oracle.bsfa_oracle import MaskSpec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------------------- pages


def _example_inputs(n, row, weights, d=4):
    """Queries/keys whose scaled scores for ``row`` are ln(weight) on the listed keys
    and -10 elsewhere (scale = 1, so s = q . k)."""
    q = np.zeros((1, 1, n, d))
    k = np.zeros((1, 1, n, d))
    q[0, 0, :, 0] = 1.0
    for j in range(n):
        k[0, 0, j, 0] = math.log(weights[j]) if j in weights else -10.0
    return q, k


def test_worked_sparse_output_example():
    ex = _load("sparse_output_example.json")
    i = ex["query_position"]
    weights = {int(j): w for j, w in ex["weights"].items()}
    n = i + 1
    q, k = _example_inputs(n, i, weights)
    v = np.zeros((1, 1, n, 2))
    v[0, 0, : len(ex["values"])] = ex["values"]
    v[0, 0, i] = [100.0, -100.0]  # the query's own value: outside G, must not leak in
    spec = MaskSpec(causal=True, force_keep_diag=False, force_keep_global=False)
    r = orc.attention(q, k, v, spec, tau=-5.0, block_q=1, block_k=1, scale=1.0)
    out = r.full_out()[0, 0, i]
    np.testing.assert_allclose(out, ex["expected_output"], rtol=0, atol=1e-12)
    kept = sorted(np.nonzero(r.keep[0, 0, i])[0].tolist())
    assert kept == ex["G"]


def test_excluded_index_contributes_nothing():
    ex = _load("excluded_index_example.json")
    i = ex["query_position"]
    g = ex["G"]
    weights = {j: 1.0 / len(g) for j in g}
    n = i + 1
    q, k = _example_inputs(n, i, weights)
    spec = MaskSpec(causal=True, force_keep_diag=False, force_keep_global=False)
    v = _rand((1, 1, n, 3), 7)
    r1 = orc.attention(q, k, v, spec, tau=-5.0, block_q=1, block_k=1, scale=1.0)
    v2 = v.copy()
    v2[0, 0, ex["excluded"]] += 1e6
    r2 = orc.attention(q, k, v2, spec, tau=-5.0, block_q=1, block_k=1, scale=1.0)
    np.testing.assert_array_equal(r1.full_out()[0, 0, i], r2.full_out()[0, 0, i])
    assert not r1.keep[0, 0, i, ex["excluded"]]
    expect = np.mean(v[0, 0, g], axis=0)
    np.testing.assert_allclose(r1.full_out()[0, 0, i], expect, atol=1e-12)


def test_mask_counts_from_pages():
    cases = _load("mask_counts.json")
    c = cases["cases"][0]
    spec = MaskSpec(causal=c["causal"], window=c["window"], n_global=c["n_global"])
    i = c["row_1based"] - 1
    a = orc.element_mask([i], np.arange(c["N"]), c["N"], spec)
    assert int(a.sum()) == c["expected_count"]
    assert sorted(np.nonzero(a[0])[0].tolist()) == [0, i - 2, i - 1, i]
    c = cases["cases"][1]
    spec = MaskSpec(causal=c["causal"], window=c["window"], n_global=c["n_global"])
    a = orc.element_mask(np.arange(c["N"]), np.arange(c["N"]), c["N"], spec)
    assert int(a.sum()) == c["expected_total"]


def test_window_range():
    wr = _load("mask_counts.json")["window_range"]
    n, w = wr["N"], wr["W"]
    spec = MaskSpec(causal=True, window=w)
    a = orc.element_mask(np.arange(n), np.arange(n), n, spec)
    for i in range(n):
        assert np.nonzero(a[i])[0].tolist() == list(range(max(0, i - w + 1), i + 1))


# ------------------------------------------------------------- library cross-checks


def _sdpa(q, k, v, mask=None, scale=None):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)) for x in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [64, 200])
def test_dense_limit_equals_sdpa(causal, n):
    d = 16
    q, k, v = _rand((2, 3, n, d), 1), _rand((2, 3, n, d), 2), _rand((2, 3, n, d), 3)
    spec = MaskSpec(causal=causal)
    for tau in (None, -np.inf):
        r = orc.attention(q, k, v, spec, tau=tau, block_q=64, block_k=64)
        ref = _sdpa(q, k, v, mask=np.tril(np.ones((n, n), bool)) if causal else None)
        got = r.full_out()[:, :, :n]
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_static_masks_equal_sdpa_with_that_mask():
    n, d = 300, 8
    q, k, v = _rand((1, 2, n, d), 4), _rand((1, 2, n, d), 5), _rand((1, 2, n, d), 6)
    spec = MaskSpec(causal=True, window=50, n_global=20)
    ii, jj = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    mask = (jj <= ii) & ((ii - jj < 50) | (jj < 20) | (ii < 20))
    r = orc.attention(q, k, v, spec, tau=None, block_q=64, block_k=64)
    np.testing.assert_allclose(r.full_out()[:, :, :n], _sdpa(q, k, v, mask), atol=1e-12)


def test_tau_plus_inf_keeps_only_diagonal_blocks():
    """tau=+inf with the causal diagonal forced: attention within each 64-token chunk."""
    n, d, blk = 256, 8, 64
    q, k, v = _rand((1, 1, n, d), 8), _rand((1, 1, n, d), 9), _rand((1, 1, n, d), 10)
    r = orc.attention(q, k, v, MaskSpec(causal=True), tau=np.inf)
    ref = np.concatenate(
        [_sdpa(q[:, :, s:s + blk], k[:, :, s:s + blk], v[:, :, s:s + blk],
               np.tril(np.ones((blk, blk), bool))) for s in range(0, n, blk)], axis=2)
    np.testing.assert_allclose(r.full_out(), ref, atol=1e-12)
    assert np.array_equal(r.keep[0, 0], np.eye(n // blk, dtype=bool))


def test_gqa_equals_mha_with_repeated_kv():
    n, d = 128, 8
    q = _rand((1, 4, n, d), 11)
    k, v = _rand((1, 2, n, d), 12), _rand((1, 2, n, d), 13)
    tau = np.array([0.1, 0.3, -0.2, 0.5])
    spec = MaskSpec(causal=True)
    r = orc.attention(q, k, v, spec, tau=tau, block_q=32, block_k=32)
    r2 = orc.attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), spec, tau=tau,
                       block_q=32, block_k=32)
    np.testing.assert_array_equal(r.out, r2.out)
    np.testing.assert_array_equal(r.keep, r2.keep)


# ------------------------------------------------------------ closed forms, invariants


def test_zero_queries_closed_form():
    n, d = 192, 8
    q = np.zeros((1, 1, n, d))
    k, v = _rand((1, 1, n, d), 14), _rand((1, 1, n, d), 15)
    spec = MaskSpec(causal=True)
    r = orc.attention(q, k, v, spec, tau=0.0)
    cnt = np.arange(1, n + 1)
    np.testing.assert_allclose(r.full_out()[0, 0], np.cumsum(v[0, 0], 0) / cnt[:, None], atol=1e-12)
    np.testing.assert_allclose(r.full_lse()[0, 0], np.log(cnt), atol=1e-12)
    assert np.all(r.tile_max[r.keep] == 0.0)
    r = orc.attention(q, k, v, spec, tau=1e-9)  # only forced (diagonal) tiles survive
    assert np.array_equal(r.keep[0, 0], np.eye(3, dtype=bool))
    t = np.arange(n) // 64
    lo = t * 64
    ref = np.stack([v[0, 0, lo[i]:i + 1].mean(0) for i in range(n)])
    np.testing.assert_allclose(r.full_out()[0, 0], ref, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_invariants(seed):
    n, d = 200, 16
    rng = np.random.default_rng(100 + seed)
    q, k = rng.standard_normal((1, 2, n, d)), rng.standard_normal((1, 2, n, d))
    v = rng.standard_normal((1, 2, n, d))
    spec = MaskSpec(causal=True, window=90, n_global=10)
    tau = np.array([0.2, 0.6])
    r = orc.attention(q, k, v, spec, tau=tau, block_q=32, block_k=32)
    # kept weights sum to one: the output for V = 1 is exactly 1 on every row
    r1 = orc.attention(q, k, np.ones_like(v), spec, tau=tau, block_q=32, block_k=32)
    np.testing.assert_allclose(r1.full_out()[:, :, :n], 1.0, atol=1e-12)
    scale = 1.0 / math.sqrt(d)
    nq = r.full_out().shape[2]
    for h in range(2):
        s = scale * q[0, h] @ k[0, h].T
        a = orc.element_mask(np.arange(n), np.arange(n), n, spec)
        keep_el = np.zeros((n, n), bool)
        for ti in range(len(r.q_tiles)):
            for c in range(r.keep.shape[3]):
                keep_el[ti * 32:(ti + 1) * 32, c * 32:(c + 1) * 32] = r.keep[0, h, ti, c]
        member = a & keep_el
        lse = r.full_lse()[0, h, :n]
        out = r.full_out()[0, h, :n]
        for i in range(n):
            idx = np.nonzero(member[i])[0]
            assert idx.size > 0  # the forced diagonal keeps every row non-empty
            top = s[i, idx].max()
            assert top - 1e-12 <= lse[i] <= top + math.log(idx.size) + 1e-12
            lo, hi = v[0, h, idx].min(0), v[0, h, idx].max(0)
            assert np.all(out[i] >= lo - 1e-12) and np.all(out[i] <= hi + 1e-12)
    assert nq >= n


def test_keep_monotone_in_tau():
    n, d = 256, 16
    q, k, v = _rand((1, 1, n, d), 20), _rand((1, 1, n, d), 21), _rand((1, 1, n, d), 22)
    spec = MaskSpec(causal=True)
    taus = [-np.inf, -1.0, 0.0, 0.5, 1.0, 2.0, np.inf]
    keeps = [orc.attention(q, k, v, spec, tau=t, block_q=32, block_k=32).keep for t in taus]
    for a, b in zip(keeps, keeps[1:]):
        assert np.all(b <= a)  # a larger tau never keeps a block a smaller one dropped
    assert keeps[0].sum() > keeps[-1].sum()


def test_nan_tau_keeps_only_forced():
    n, d = 128, 8
    q, k, v = _rand((1, 1, n, d), 23), _rand((1, 1, n, d), 24), _rand((1, 1, n, d), 25)
    r = orc.attention(q, k, v, MaskSpec(causal=True, window=100, n_global=3), tau=np.nan,
                      block_q=32, block_k=32)
    assert np.array_equal(r.keep[0, 0], r.forced)


def test_empty_row_gives_zero_and_minus_inf():
    # Not causal, no forcing, tau=+inf: nothing is kept.
    n, d = 64, 4
    q, k, v = _rand((1, 1, n, d), 26), _rand((1, 1, n, d), 27), _rand((1, 1, n, d), 28)
    spec = MaskSpec(causal=False, force_keep_diag=False, force_keep_global=False)
    r = orc.attention(q, k, v, spec, tau=np.inf, block_q=16, block_k=16)
    assert np.all(r.full_out() == 0.0)
    assert np.all(np.isneginf(r.full_lse()))


# --------------------------------------------------------- brute force on tiny inputs


def _brute(q, k, v, causal, window, n_global, diag, glob, tau, bq, bk, scale):
    """Straight loops over the definition, for one head (no numpy vector tricks)."""
    n, d = len(q), len(q[0])

    def allowed(i, j):
        if causal and j > i:
            return False
        if window > 0 and not (i - window < j < i + window or j < n_global or i < n_global):
            return False
        return True

    s = [[scale * sum(q[i][x] * k[j][x] for x in range(d)) for j in range(n)] for i in range(n)]
    nqt, nkb = -(-n // bq), -(-n // bk)
    keep = {}
    for t in range(nqt):
        for c in range(nkb):
            vals = [s[i][j] for i in range(t * bq, min(n, t * bq + bq))
                    for j in range(c * bk, min(n, c * bk + bk)) if allowed(i, j)]
            if not vals:
                continue
            forced = False
            if diag and any(c * bk <= i < c * bk + bk for i in range(t * bq, min(n, t * bq + bq))):
                forced = True
            if glob and c * bk < n_global:
                forced = True
            keep[(t, c)] = forced or (tau is None) or (max(vals) >= tau)
    out, lse = [], []
    for i in range(n):
        js = [j for j in range(n) if allowed(i, j) and keep.get((i // bq, j // bk), False)]
        if not js:
            out.append([0.0] * len(v[0]))
            lse.append(-math.inf)
            continue
        top = max(s[i][j] for j in js)
        ws = [math.exp(s[i][j] - top) for j in js]
        tot = sum(ws)
        out.append([sum(w * v[j][x] for w, j in zip(ws, js)) / tot for x in range(len(v[0]))])
        lse.append(top + math.log(tot))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize(
    "n,bq,bk,causal,window,n_global,tau",
    [
        (37, 1, 1, True, 0, 0, 0.1),
        (50, 2, 3, True, 9, 4, 0.0),
        (61, 3, 2, False, 7, 0, 0.3),
        (130, 64, 64, True, 0, 0, 0.9),
        (130, 64, 64, True, 40, 5, 0.5),
        (99, 16, 8, False, 0, 0, 0.2),
        (70, 64, 64, False, 0, 0, None),
    ],
)
def test_brute_force_tiny(n, bq, bk, causal, window, n_global, tau):
    d = 5
    rng = np.random.default_rng(n * 7 + bq)
    q, k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((n, 3))
    scale = 1.0 / math.sqrt(d)
    spec = MaskSpec(causal=causal, window=window, n_global=n_global)
    r = orc.attention(q[None, None], k[None, None], v[None, None], spec, tau=tau,
                      block_q=bq, block_k=bk, scale=scale)
    ref_o, ref_l = _brute(q.tolist(), k.tolist(), v.tolist(), causal, window, n_global,
                          True, True, tau, bq, bk, scale)
    np.testing.assert_allclose(r.full_out()[0, 0, :n], ref_o, atol=1e-12)
    np.testing.assert_allclose(r.full_lse()[0, 0, :n], ref_l, atol=1e-12)


def _staircase_inputs():
    """Four 64-token blocks whose keys put every block maximum at a known integer.

    d = 2 and scale 1, query rows of head h are (h + 1, 0), and key j is (x_j, 0) with
    x_j = c + 1 at one key of block c and below c + 0.5 elsewhere. Any query row that
    may attend a whole block c therefore has the block maximum (h + 1) * (c + 1) there:
    on every eligible tile, since the off-diagonal tiles of a causal mask are full."""
    n, nb = 256, 4
    rng = np.random.default_rng(11)
    x = np.empty(n)
    for c in range(nb):
        blk = rng.uniform(-1.0, c + 0.5, 64)
        blk[int(rng.integers(0, 64))] = c + 1.0
        x[c * 64:(c + 1) * 64] = blk
    k = np.zeros((1, 1, n, 2))
    k[0, 0, :, 0] = x
    q = np.zeros((1, 2, n, 2))
    q[0, 0, :, 0] = 1.0
    q[0, 1, :, 0] = 2.0
    return q, k


@pytest.mark.parametrize("causal,diag,quantile,expected", [
    # causal, diagonal forced: eligible (t, c < t) maxima c + 1 = {1, 1, 2, 1, 2, 3}
    (True, True, 0.5, 1.5),   # sorted [1 1 1 2 2 3], position 2.5
    (True, True, 0.4, 1.0),   # position 2.0
    (True, True, 0.9, 2.5),   # position 4.5
    # full mask, diagonal forced: every c three times, [1 1 1 2 2 2 3 3 3 4 4 4]
    (False, True, 0.5, 2.5),  # position 5.5
    (False, True, 0.2, 1.2),  # position 2.2
    # full mask, nothing forced: every c four times
    (False, False, 0.25, 1.75),  # position 3.75
    (False, False, 1.0, 4.0),
])
def test_calibration_closed_form(causal, diag, quantile, expected):
    """tau_h is the linear-interpolation quantile ("Block Sparse Flash Attention",
    threshold calibration) of head h's eligible block maxima, here known exactly. Head 1's
    scores are twice head 0's, so its tau is twice as large: the heads are not pooled."""
    q, k = _staircase_inputs()
    spec = MaskSpec(causal=causal, force_keep_diag=diag)
    tau = orc.calibrate_tau(q, k, spec, quantile, scale=1.0)
    np.testing.assert_allclose(tau, [expected, 2.0 * expected], rtol=0, atol=1e-12)


def test_calibration_hits_target_fraction():
    n, d = 512, 16
    q, k = _rand((1, 2, n, d), 30), _rand((1, 1, n, d), 31)
    spec = MaskSpec(causal=True)
    for target in (0.4, 0.5, 0.6):
        tau = orc.calibrate_tau(q, k, spec, target)
        r = orc.attention(q, k, np.zeros_like(k), spec, tau=tau)
        elig = r.allowed & ~r.forced
        for h in range(2):
            skipped = (~r.keep[0, h] & elig).sum()
            # the quantile sits between two block maxima: off by at most one block
            assert abs(skipped - target * elig.sum()) <= 1.0
