"""GPU calibration pass (gate-only kernel pass) against the fp64 oracle's calibration.

The per-head threshold is a quantile of the eligible block maxima (Block Sparse Flash
Attention, "The paper's improvements"). A quantile moves by at most the largest change
of its inputs, so the GPU's thresholds must lie within the block-maximum tolerance
(1e-3) of the oracle's. The gate-only pass (tau = NaN) must export exactly the maxima of
the full pass (tau = -inf), and keep only forced tiles.
"""
import numpy as np
import pytest

from block_sparse_flashattention_amd import inputs
from tests import parity_helpers as ph

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("w", [
    inputs.scaled(inputs.WORKLOADS["gqa_planted_16k"], N=2048, Hq=8, Hkv=2),
    inputs.Workload("cal_window", 1, 4, 2, 1500, 64, causal=True, window=300, n_global=64),
], ids=lambda w: w.name)
def test_gpu_calibration_matches_oracle(w):
    import torch

    import block_sparse_flashattention_amd as bsfa

    quantiles = (0.4, 0.5, 0.6)
    ph.log(f"case calibration {w.name}: Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} seed=1")
    qc, kc, _ = inputs.generate(w, 1)
    q, k = ph.to_dev(qc), ph.to_dev(kc)
    mask = ph.gpu_spec(w)
    taus = bsfa.calibrate_tau(q, k, mask, quantiles)
    torch.cuda.synchronize()
    for qi, qv in enumerate(quantiles):
        ref = ph.oracle_tau(w, qv)
        err = float(np.abs(taus[qi].astype(np.float64) - ref).max())
        ph.log(f"quantile {qv}: max |tau_gpu - tau_oracle| = {err:.2e}")
        assert err <= ph.NEAR_TAU

    # the gate-only pass and the full pass see the same block maxima
    full = bsfa.fwd(q, k, k, mask=mask, tau=torch.full((w.Hq,), -np.inf, device="cuda"),
                    export_tiles=True)
    gate = bsfa.fwd(q, k, k, mask=mask, tau=torch.full((w.Hq,), np.nan, device="cuda"),
                    export_tiles=True)
    torch.cuda.synchronize()
    assert np.array_equal(full.tile_max.cpu().numpy(), gate.tile_max.cpu().numpy())
    forced = (gate.lists.cls_host & 2) != 0
    keep = gate.keep.cpu().numpy().astype(bool)
    assert np.array_equal(keep, np.broadcast_to(forced, keep.shape))
    maxima = bsfa.calibration_maxima(q, k, mask)
    eligible = int((~forced).sum())
    assert [m.size for m in maxima] == [w.B * eligible] * w.Hq


def _np_taus(tmax, keep, quantiles):
    """numpy's linear quantile of each head's eligible maxima (finite, not kept)."""
    out = np.empty((len(quantiles), tmax.shape[1]), dtype=np.float32)
    for h in range(tmax.shape[1]):
        vals = tmax[:, h][(keep[:, h] == 0) & np.isfinite(tmax[:, h])].astype(np.float64)
        out[:, h] = np.quantile(vals, quantiles) if vals.size else -np.inf
    return out


QUANTILES = (0.0, 1e-9, 0.1, 0.25, 0.37, 0.5, 0.6, 0.9, 0.999, 1.0)


@pytest.mark.parametrize("bsz,hq,n,kind", [
    (3, 5, 1000, "normal"),          # several rows per head, forced and -inf blocks
    (2, 4, 777, "ties"),             # values on a coarse grid: long runs of equal keys
    (1, 2, 3_000_000, "normal"),     # one row per head over hundreds of workgroups
    (4, 3, 1, "normal"),             # one block per row
])
def test_gpu_quantile_equals_numpy(bsz, hq, n, kind):
    """bsfa_calibrate_tau against np.quantile on the same fp32 maxima: bit-identical."""
    import torch

    import block_sparse_flashattention_amd as bsfa

    ph.log(f"case gpu quantile: B={bsz} Hq={hq} n_blocks={n} values={kind}")
    rng = np.random.default_rng(17)
    tmax = rng.standard_normal((bsz, hq, n)).astype(np.float32) * 3.0
    if kind == "ties":
        tmax = np.round(tmax * 2.0) / 2.0
    keep = (rng.random((bsz, hq, n)) < 0.1).astype(np.uint8)  # forced blocks
    tmax[rng.random((bsz, hq, n)) < 0.05] = -np.inf               # blocks with no allowed key
    got = bsfa.gpu_quantiles(torch.from_numpy(tmax).cuda(), torch.from_numpy(keep).cuda(),
                             bsz, hq, n, QUANTILES)
    ref = _np_taus(tmax, keep, QUANTILES)
    assert np.array_equal(got, ref), np.abs(got.astype(np.float64) - ref).max()


def test_gpu_quantile_edge_heads():
    """A head with no eligible block (-inf), one with a single one, one with all values
    equal, and one whose values are -0.0 and +0.0 and negatives only."""
    import torch

    import block_sparse_flashattention_amd as bsfa

    n = 300
    tmax = np.random.default_rng(3).standard_normal((2, 4, n)).astype(np.float32)
    keep = np.zeros((2, 4, n), dtype=np.uint8)
    keep[:, 0] = 1                                  # head 0: every block forced
    tmax[:, 1] = -np.inf                            # head 1: a single allowed block
    tmax[1, 1, 17] = 2.5
    tmax[:, 2] = 0.75                               # head 2: all equal
    tmax[:, 3] = -np.abs(tmax[:, 3])                # head 3: non-positive, with signed zeros
    tmax[0, 3, :5] = -0.0
    tmax[1, 3, :5] = 0.0
    got = bsfa.gpu_quantiles(torch.from_numpy(tmax).cuda(), torch.from_numpy(keep).cuda(),
                             2, 4, n, QUANTILES)
    ref = _np_taus(tmax, keep, QUANTILES)
    assert np.all(np.isneginf(got[:, 0]))
    assert np.all(got[:, 1] == 2.5) and np.all(got[:, 2] == 0.75)
    assert np.array_equal(got, ref)


def test_calibrate_tau_equals_numpy_on_the_export():
    """calibrate_tau (gate-only pass, then the GPU quantile) equals np.quantile over the
    maxima the same gate-only pass exports; likewise for decode."""
    import torch

    import block_sparse_flashattention_amd as bsfa

    w = inputs.scaled(inputs.WORKLOADS["gqa_planted_16k"], N=3000, Hq=8, Hkv=2)
    qc, kc, _ = inputs.generate(w, 1)
    q, k = ph.to_dev(qc), ph.to_dev(kc)
    mask = ph.gpu_spec(w)
    qs = (0.3, 0.5, 0.75)
    got = bsfa.calibrate_tau(q, k, mask, qs)
    maxima = bsfa.calibration_maxima(q, k, mask)
    ref = np.stack([np.quantile(m.astype(np.float64), qs) for m in maxima], axis=1)
    assert np.array_equal(got, ref.astype(np.float32))

    dw = inputs.DecodeWorkload("cal_decode", 3, 8, 2, 1500, 128, lengths=(1500, 1001, 64),
                               kind="sink_local")
    dq, dk, _, lengths = inputs.generate_decode(dw, 1)
    lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    got = bsfa.decode_calibrate_tau(ph.to_dev(dq), ph.to_dev(dk), lens, mask, qs)
    maxima = bsfa.decode_calibration_maxima(ph.to_dev(dq), ph.to_dev(dk), lens, mask)
    ref = np.stack([np.quantile(m.astype(np.float64), qs) for m in maxima], axis=1)
    assert np.array_equal(got, ref.astype(np.float32))
    ph.log("calibrate_tau and decode_calibrate_tau: bit-identical to np.quantile on the export")
