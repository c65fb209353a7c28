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
