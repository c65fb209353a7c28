"""GPU parity on the edges of the gate: query rows whose kept set is empty, an unforced
diagonal, and a softmax scale other than 1/sqrt(d).

A row with no kept key gets O = 0 and LSE = -inf ("Sparse attention weights assumption",
"Index Set of Non-Zero Attention Weights (G)": only keys in G carry weight, and here G
is empty). With the diagonal and global blocks forced (the defaults) such a row cannot
occur, so these cases switch the forcing off. Each case runs on packs of one, two and
four query heads per KV head (the lock-step kernel's two pack sizes and the
warp-specialised kernel), and compares keep bits, block maxima, O and LSE (-inf rows
included) with the fp64 oracle at the same tolerances as every other parity case.
"""
import numpy as np
import pytest

from block_sparse_flashattention_amd import inputs
from oracle import bsfa_oracle as orc
from tests import parity_helpers as ph

pytestmark = pytest.mark.gpu

NO_FORCE = (("force_keep_diag", 0), ("force_keep_global", 0))
PACKS = [(2, 2), (4, 2), (8, 2)]  # query heads per KV head: 1, 2, 4


def _workload(name, hq, hkv, n, d, causal, extra=NO_FORCE, window=0, n_global=0,
              kind="planted"):
    return inputs.Workload(name, 1, hq, hkv, n, d, causal=causal, window=window,
                           n_global=n_global, kind=kind, planted_frac=0.15,
                           mask_extra=tuple(extra))


def _check_empty_rows(res, lse_rows_expected_empty):
    lse = res.lse.cpu().numpy()
    out = res.out.float().cpu().numpy()
    assert np.isneginf(lse[lse_rows_expected_empty]).all()
    assert (out[lse_rows_expected_empty] == 0).all()


def _oracle_tile_max(w, qb, kb, scale=None):
    q, k, _ = ph.reduced(w, qb, kb, kb, list(range(w.Hq)))
    return orc.attention(q, k, k, ph.oracle_spec(w), tau=None, scale=scale)


@pytest.mark.parametrize("hq,hkv", PACKS)
@pytest.mark.parametrize("d", [64, 128])
def test_tau_plus_inf_nothing_forced_every_row_empty(hq, hkv, d):
    """Non-causal, nothing forced, tau = +inf: every tile is skipped, every row is empty."""
    w = _workload("empty_all", hq, hkv, 300, d, causal=False)
    ph.log(f"case {w.name}: Hq={hq} Hkv={hkv} N={w.N} d={d} non-causal, no forcing, "
           f"tau=+inf, seed=0")
    qb, kb, vb = inputs.generate(w, 0)
    tau = np.full(w.Hq, np.inf, np.float32)
    res = ph.run_gpu(w, qb, kb, vb, tau)
    assert not res.keep.cpu().numpy().any()
    st = res.stats.cpu().numpy()
    assert (st[..., 0] == 0).all() and (st[..., 1] == res.lists.nnz).all()
    _check_empty_rows(res, (slice(None),) * 3)
    ph.compare(w, qb, kb, vb, res, tau)


@pytest.mark.parametrize("hq,hkv", PACKS)
def test_first_tile_keeps_nothing_noncausal(hq, hkv):
    """Non-causal window + globals, nothing forced; per-head tau just above the largest
    block maximum of query tile 0, so tile 0's rows keep nothing and later tiles keep
    the blocks above that level."""
    w = _workload("empty_tile0", hq, hkv, 400, 128, causal=False, window=150, n_global=5,
                  extra=NO_FORCE)
    ph.log(f"case {w.name}: Hq={hq} Hkv={hkv} N={w.N} non-causal window=150 globals=5, "
           f"no forcing, tau above tile 0's maxima, seed=0")
    qb, kb, vb = inputs.generate(w, 0)
    ref = _oracle_tile_max(w, qb, kb)
    tm0 = np.where(ref.allowed[0][None, :], ref.tile_max[0, :, 0, :], -np.inf)
    tau = (tm0.max(axis=1) + 0.05).astype(np.float32)
    res = ph.run_gpu(w, qb, kb, vb, tau)
    rep = ph.compare(w, qb, kb, vb, res, tau)
    _check_empty_rows(res, (0, slice(None), slice(0, 64)))
    assert 0 < rep.kept < rep.total, "some later tiles must keep blocks"


@pytest.mark.parametrize("hq,hkv", PACKS)
def test_causal_diagonal_not_forced_at_quantile(hq, hkv):
    """Causal, neither diagonal nor global blocks forced, tau at the oracle's calibrated
    median (every allowed block is eligible): rows whose blocks all fall below tau are
    empty, e.g. the first tile when its one block is skipped."""
    w = _workload("causal_unforced", hq, hkv, 640, 128, causal=True)
    ph.log(f"case {w.name}: Hq={hq} Hkv={hkv} N={w.N} causal, no forcing, tau at q=0.5 "
           f"(seed 1), eval seed=0")
    tau = ph.oracle_tau(w, 0.5)
    qb, kb, vb = inputs.generate(w, 0)
    res = ph.run_gpu(w, qb, kb, vb, tau)
    rep = ph.compare(w, qb, kb, vb, res, tau)
    assert 0 < rep.kept < rep.total
    lse = res.lse.cpu().numpy()
    ph.log(f"rows with an empty kept set: {int(np.isneginf(lse).sum())} of {lse.size}")


@pytest.mark.parametrize("hq,hkv", PACKS)
def test_causal_diagonal_only_unforced_globals_forced(hq, hkv):
    """Causal with 64 global tokens: the global block stays forced, the diagonal does not.
    At tau = +inf every row keeps exactly the global block."""
    w = _workload("global_only", hq, hkv, 520, 64, causal=True, n_global=64,
                  extra=(("force_keep_diag", 0), ("force_keep_global", 1)))
    ph.log(f"case {w.name}: Hq={hq} Hkv={hkv} N={w.N} d=64 causal globals=64, diagonal "
           f"not forced, tau=+inf, seed=0")
    qb, kb, vb = inputs.generate(w, 0)
    tau = np.full(w.Hq, np.inf, np.float32)
    res = ph.run_gpu(w, qb, kb, vb, tau)
    keep = res.keep.cpu().numpy().astype(bool)
    assert np.array_equal(keep, np.broadcast_to(res.lists.col_host == 0, keep.shape))
    ph.compare(w, qb, kb, vb, res, tau)


@pytest.mark.parametrize("hq,hkv", PACKS)
def test_softmax_scale_not_default(hq, hkv):
    """softmax_scale = 0.05 instead of 1/sqrt(128): the scale enters the gate (block
    maxima in scaled units) and the exponent; tau is calibrated at the same scale."""
    scale = float(np.float32(0.05))
    w = _workload("scale_0p05", hq, hkv, 700, 128, causal=True,
                  extra=(("force_keep_diag", 1), ("force_keep_global", 1)), n_global=3,
                  window=300)
    ph.log(f"case {w.name}: Hq={hq} Hkv={hkv} N={w.N} causal window=300 globals=3, "
           f"scale={scale}, tau at q=0.5, seed=0")
    tau = ph.oracle_tau(w, 0.5, scale=scale)
    qb, kb, vb = inputs.generate(w, 0)
    res = ph.run_gpu(w, qb, kb, vb, tau, scale=scale)
    rep = ph.compare(w, qb, kb, vb, res, tau, scale=scale)
    assert 0 < rep.kept < rep.total
    # the dense path at the same scale
    res = ph.run_gpu(w, qb, kb, vb, None, export=False, scale=scale)
    ph.compare(w, qb, kb, vb, res, None, scale=scale)


@pytest.mark.parametrize("hq,hkv", PACKS)
def test_softmax_scale_with_empty_rows(hq, hkv):
    """A non-default scale together with unforced blocks and a high tau (quantile 0.9):
    many rows keep nothing, the rest keep their few highest blocks."""
    scale = float(np.float32(0.12))
    w = _workload("scale_empty", hq, hkv, 384, 64, causal=False, kind="gaussian")
    ph.log(f"case {w.name}: Hq={hq} Hkv={hkv} N={w.N} d=64 non-causal, no forcing, "
           f"scale={scale}, tau at q=0.9, seed=0")
    tau = ph.oracle_tau(w, 0.9, scale=scale)
    qb, kb, vb = inputs.generate(w, 0)
    res = ph.run_gpu(w, qb, kb, vb, tau, scale=scale)
    rep = ph.compare(w, qb, kb, vb, res, tau, scale=scale)
    assert 0 < rep.kept < rep.total
