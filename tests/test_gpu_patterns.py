"""GPU parity for the dilated/strided, blockwise and random-block primitives ("sparse
attention mechanism" glossary, table "Sparse Attention Patterns"), alone and OR-composed
with the window and global tokens, on the gated path (tau at the 0.5 quantile) and the
dense path. Sizes span several tiles with a ragged tail.

The output is fp32: these patterns leave rows with a few dozen keys, so |O| reaches
several units, where the bf16 output's half-ulp alone (0.008 to 0.016) would exceed the
1e-2 bound on |dO|. The bf16 output path is covered by the other parity tests."""
import numpy as np
import pytest

from block_sparse_flashattention_amd import inputs
from tests import parity_helpers as ph

pytestmark = pytest.mark.gpu

CASES = [
    # name, N, Hq, Hkv, d, causal, window, n_global, extra mask fields
    ("dilated_taps", 700, 4, 2, 128, True, 0, 0, (("dilation", 5), ("dilation_taps", 30))),
    ("dilated_full", 333, 2, 1, 64, False, 0, 0, (("dilation", 70),)),
    ("dilated_window", 1000, 8, 2, 128, True, 32, 8,
     (("dilation", 64), ("dilation_taps", 6))),
    ("blockwise", 1000, 4, 1, 128, True, 0, 0, (("block", 100),)),
    ("blockwise_global", 450, 2, 2, 64, False, 0, 5, (("block", 64),)),
    ("bigbird", 900, 4, 4, 128, True, 64, 16,
     (("random_ppm", 300_000), ("random_seed", 7))),
    ("all_primitives", 777, 3, 1, 64, False, 40, 3,
     (("dilation", 9), ("dilation_taps", 12), ("block", 150), ("random_ppm", 150_000),
      ("random_seed", 99))),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pattern_parity(case):
    name, n, hq, hkv, d, causal, window, n_global, extra = case
    w = inputs.Workload(f"pattern_{name}", 1, hq, hkv, n, d, causal=causal, window=window,
                        n_global=n_global, kind="planted", planted_frac=0.1,
                        out_f32=True, mask_extra=extra)
    ph.log(f"case {w.name}: N={n} Hq={hq} Hkv={hkv} d={d} causal={causal} window={window} "
           f"n_global={n_global} {dict(extra)} seed=0")
    qb, kb, vb = inputs.generate(w, 0)
    tau = ph.oracle_tau(w, 0.5)
    res = ph.run_gpu(w, qb, kb, vb, tau)
    ph.compare(w, qb, kb, vb, res, tau)
    out = res.out.float().cpu().numpy()
    assert not np.isnan(out).any(), "an output element was never written"
    res = ph.run_gpu(w, qb, kb, vb, None, export=False)
    ph.compare(w, qb, kb, vb, res, None)
