"""GPU parity on seeded random shapes and masks, against the fp64 oracle.

Every head grouping runs here: four heads of one query tile per workgroup (group a
multiple of 4), two heads of two query tiles (even group), one head of four query tiles
(odd group, multi-head attention). These are combined with both head dims, ragged
lengths, batches, causal or not, windows, global tokens and the further primitives
(dilated, blockwise, random blocks). Each case runs the gated path (tau at the 0.5
quantile of the calibration seed) and the dense path. The draws come from a fixed seed,
so the set of cases is the same on every run.

The output is fp32 whenever the mask can leave rows with few keys, where |O| reaches
several units and the bf16 output's half-ulp alone would exceed the 1e-2 bound."""
import numpy as np
import pytest

from block_sparse_flashattention_amd import inputs
from tests import parity_helpers as ph

pytestmark = pytest.mark.gpu


def _draw_cases(n_cases=14, seed=20261203):
    rng = np.random.default_rng(seed)
    groups = [1, 2, 3, 4, 5, 6, 8]
    cases = []
    for i in range(n_cases):
        group = groups[i % len(groups)]  # every grouping at least twice
        hkv = int(rng.integers(1, 3)) if group <= 4 else 1
        b = int(rng.integers(1, 3)) if group * hkv <= 4 else 1
        n = int(rng.integers(1, 1201))
        d = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        window = int(rng.integers(1, 600)) if rng.random() < 0.4 else 0
        n_global = int(rng.integers(1, 100)) if rng.random() < 0.4 else 0
        extra = []
        if rng.random() < 0.3:
            extra += [("dilation", int(rng.integers(2, 80)))]
            if rng.random() < 0.5:
                extra += [("dilation_taps", int(rng.integers(1, 40)))]
        if rng.random() < 0.2:
            extra += [("block", int(rng.integers(8, 300)))]
        if rng.random() < 0.2:
            extra += [("random_ppm", int(rng.integers(50_000, 400_000))),
                      ("random_seed", int(rng.integers(0, 1000)))]
        kind = str(rng.choice(["gaussian", "planted", "sink_local"]))
        out_f32 = bool(extra) or 0 < window < 128 or rng.random() < 0.5
        cases.append((f"r{i:02d}", b, group * hkv, hkv, n, d, causal, window, n_global,
                      tuple(extra), kind, out_f32))
    return cases


CASES = _draw_cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_random_shape_parity(case):
    name, b, hq, hkv, n, d, causal, window, n_global, extra, kind, out_f32 = case
    w = inputs.Workload(f"random_{name}", b, hq, hkv, n, d, causal=causal, window=window,
                        n_global=n_global, kind=kind, planted_frac=0.1, out_f32=out_f32,
                        mask_extra=extra)
    ph.log(f"case {w.name}: B={b} Hq={hq} Hkv={hkv} N={n} d={d} causal={causal} "
           f"window={window} n_global={n_global} {dict(extra)} kind={kind} "
           f"out_f32={out_f32} seed=0")
    qb, kb, vb = inputs.generate(w, 0)
    tau = ph.oracle_tau(w, 0.5)
    res = ph.run_gpu(w, qb, kb, vb, tau)
    ph.compare(w, qb, kb, vb, res, tau)
    out = res.out.float().cpu().numpy()
    assert not np.isnan(out).any(), "an output element was never written"
    st = res.stats.cpu().numpy()
    assert np.all(st.sum(-1) == res.lists.nnz), "kept + skipped must equal the allowed tiles"
    res = ph.run_gpu(w, qb, kb, vb, None, export=False)
    ph.compare(w, qb, kb, vb, res, None)
