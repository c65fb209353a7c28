"""GPU decode step (bsfa_decode through the C ABI) against the fp64 oracle's decode.

Cases: dense and gated paths; grouped-query shapes from one to 32 query heads per KV
head; head dims 64 and 128; ragged, empty, single-row and over-long lengths; NaN in the
free cache rows past each length; the further static primitives; the GPU calibration;
and the 64K-row workload of the benchmark at full size.
"""
import numpy as np
import pytest

from block_sparse_flashattention_amd import inputs
from tests import parity_helpers as ph

pytestmark = pytest.mark.gpu

DW = inputs.DecodeWorkload


def _case(w, gated=True, quantile=0.5, poison=True):
    ph.log(f"case decode {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Lmax={w.Lmax} d={w.d} "
           f"lengths={w.lengths} kind={w.kind} gated={gated} seed=0")
    qb, kb, vb, lengths = ph.decode_inputs(w, 0, poison_tail=poison)
    tau = ph.oracle_tau_decode(w, quantile) if gated else None
    res = ph.run_gpu_decode(w, qb, kb, vb, lengths, tau)
    return ph.compare_decode(w, qb, kb, vb, lengths, res, tau)


SHAPES = [
    DW("dec_g4_d128", 3, 8, 2, 1000, 128, lengths=(1000, 517, 65), kind="sink_local"),
    DW("dec_g1_d64", 2, 2, 2, 700, 64, lengths=(700, 64), kind="gaussian", out_f32=True),
    DW("dec_g8_planted", 2, 16, 2, 2048, 128, lengths=(2048, 1999), kind="planted",
       planted_frac=0.1),
    DW("dec_g32", 1, 32, 1, 1200, 128, lengths=(1111,), kind="sink_local"),
    DW("dec_g4_d64", 2, 8, 2, 900, 64, lengths=(900, 333), kind="planted", planted_frac=0.1),
    DW("dec_g8_d64", 2, 16, 2, 700, 64, lengths=(129, 700), kind="sink_local"),
]


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_decode_gated_matches_oracle(w):
    rep = _case(w, gated=True)
    assert 0 < rep.kept < rep.total  # the gate really skipped something


@pytest.mark.parametrize("w", SHAPES[:2], ids=lambda w: w.name)
def test_decode_dense_matches_oracle(w):
    _case(w, gated=False)


def test_decode_length_edges():
    """Length 0 (no keys: O = 0, LSE = -inf), above the cache size (clamped), 1, exactly
    one block, one past a block; NaN in every free cache row."""
    w = DW("dec_edges", 5, 4, 2, 300, 128, lengths=(0, 1000, 1, 64, 65), kind="gaussian",
           out_f32=True)
    _case(w, gated=True)
    _case(w, gated=False)


@pytest.mark.parametrize("extra", [
    dict(window=200, n_global=70),
    dict(dilation=7, dilation_taps=30),
    dict(block=300),
    dict(random_ppm=300_000, random_seed=4, window=64),
], ids=lambda e: "_".join(f"{k}{v}" for k, v in e.items()))
def test_decode_patterns(extra):
    base = {k: extra[k] for k in ("window", "n_global") if k in extra}
    rest = tuple((k, v) for k, v in extra.items() if k not in base)
    w = DW("dec_pattern", 2, 8, 2, 1500, 128, lengths=(1500, 1023), kind="sink_local",
           mask_extra=rest, out_f32=True, **base)
    _case(w, gated=True)


def test_decode_gpu_calibration_matches_oracle():
    import torch

    import block_sparse_flashattention_amd as bsfa

    w = DW("dec_cal", 3, 8, 2, 1800, 128, lengths=(1800, 1301, 700), kind="sink_local")
    ph.log(f"case decode calibration {w.name}: lengths={w.lengths} seed=1")
    qb, kb, _, lengths = inputs.generate_decode(w, 1)
    lens = torch.tensor(lengths, device="cuda")
    taus = bsfa.decode_calibrate_tau(ph.to_dev(qb), ph.to_dev(kb), lens, ph.gpu_spec(w),
                                     (0.4, 0.6))
    for i, qv in enumerate((0.4, 0.6)):
        ref = ph.oracle_tau_decode(w, qv)
        err = float(np.abs(taus[i].astype(np.float64) - ref).max())
        ph.log(f"quantile {qv}: max |tau_gpu - tau_oracle| = {err:.2e}")
        assert err <= ph.NEAR_TAU


def test_decode_full_size_64k():
    """The benchmark's decode workload (4 sequences over a 64K-row cache, 32 query and
    8 KV heads, d = 128) at full size, gated at the calibrated median."""
    import torch

    import block_sparse_flashattention_amd as bsfa

    w = inputs.DECODE_WORKLOADS["decode_sink_local_64k"]
    ph.log(f"case decode full size {w.name}: lengths={w.lengths}")
    qc, kc, _, lc = inputs.generate_decode(w, 1)
    taus = bsfa.decode_calibrate_tau(ph.to_dev(qc), ph.to_dev(kc),
                                     torch.tensor(lc, device="cuda"), ph.gpu_spec(w), 0.5)
    del qc, kc
    qb, kb, vb, lengths = inputs.generate_decode(w, 0)
    res = ph.run_gpu_decode(w, qb, kb, vb, lengths, taus)
    rep = ph.compare_decode(w, qb, kb, vb, lengths, res, taus)
    assert 0.3 < 1 - rep.kept / rep.total < 0.7
