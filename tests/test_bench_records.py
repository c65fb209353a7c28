"""bench.py's bookkeeping: a committed HBM counter record is attached to the roofline only
for the workload and tau quantile it was measured on; the FLOP and byte counts behind
the metric follow the tile geometry and the cache rows."""
import json

import numpy as np
import pytest

import bench


def _rec(path):
    with open(path) as f:
        return json.load(f)


def test_prefill_traffic_record_only_for_its_workload():
    rec = _rec(bench.TRAFFIC_FILE)
    name, q = rec["workload_name"], rec["tau_quantile"]
    assert name == "sink_local_64k" and q == 0.5
    assert bench.measured_traffic("gqa_planted_16k", q) is None
    assert bench.measured_traffic(name, 0.4) is None
    got = bench.measured_traffic(name, q)
    if rec["kernel_source_sha256_16"] == bench.kernel_source_hash():
        assert got == rec["hbm_bytes_per_launch"]
    else:
        assert got is None


def test_decode_traffic_record_only_for_its_workload():
    rec = _rec(bench.DECODE_TRAFFIC_FILE)
    name, q = rec["workload_name"], rec["tau_quantile"]
    assert name == "decode_sink_local_64k" and q == 0.5
    assert bench.measured_decode_traffic("sink_local_64k", q) is None
    assert bench.measured_decode_traffic(name, 0.6) is None
    got = bench.measured_decode_traffic(name, q)
    assert got is None or got == rec["hbm_bytes_per_step"]


@pytest.mark.parametrize("name,allowed_all_heads,dense_tflop", [
    ("single_head_1k", 136, 1.43e-4),
    ("static_mask_4k", 7992, 0.01676),
    ("gqa_planted_16k", 1052672, 2.208),
    ("sink_local_64k", 16793600, 35.22),
    ("mha_sink_local_64k", 16793600, 35.22),
    ("gqa70b_planted_128k", 134283264, 281.6),
])
def test_flop_accounting_matches_tile_geometry(name, allowed_all_heads, dense_tflop):
    """bench.py's dense-equivalent FLOP: the host block lists times 4 * 64 * 64 * d per
    allowed tile. Without a window the causal mask allows nqt (nqt + 1) / 2 tiles per head
    (global tokens only force tiles that causality already allows); the windowed 4K mask's
    count comes from the oracle's element mask in tests/test_block_lists.py."""
    from block_sparse_flashattention_amd import binding, inputs

    w = inputs.WORKLOADS[name]
    spec = binding.MaskSpec(causal=w.causal, window=w.window, n_global=w.n_global)
    _, col, _ = binding.build_block_lists(spec, w.N)
    assert col.size * w.B * w.Hq == allowed_all_heads
    if w.causal and not w.window:
        nqt = -(-w.N // 64)
        assert allowed_all_heads == nqt * (nqt + 1) // 2 * w.B * w.Hq
    qk, pv = bench.tile_flops(w.d)
    assert qk == pv == 2 * 64 * 64 * w.d
    got = col.size * w.B * w.Hq * (qk + pv) / 1e12
    assert abs(got - dense_tflop) / dense_tflop < 3e-3


def test_decode_bytes_closed_form():
    """Dense decode step bytes: every valid cached K and V row of every KV head once,
    plus the query rows, O and LSE."""
    from block_sparse_flashattention_amd import inputs

    w = inputs.DECODE_WORKLOADS["decode_sink_local_64k"]
    lengths = list(w.lengths)
    rows = sum(lengths)
    expect = (rows * w.Hkv * w.d * 2 * 2 + w.B * w.Hq * w.d * 2 * 2 + w.B * w.Hq * 4)
    assert bench.decode_bytes(w, lengths) == expect == 872481280
    # keeping nothing but one block per head group leaves K plus that block's V rows
    nkb = -(-w.Lmax // 64)
    keep = np.zeros((w.B, w.Hq, nkb), dtype=bool)
    keep[:, :, 0] = True
    got = bench.decode_bytes(w, lengths, keep)
    assert got == expect - (rows - 64 * w.B) * w.Hkv * w.d * 2


def test_more_than_one_gpu_is_refused():
    """The library has no multi-GPU path: --gpus above 1 exits with a message, before
    anything touches a GPU."""
    import subprocess
    import sys

    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=bench.ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_cpu_baseline_leg_on_a_small_workload():
    """The cpu_baseline leg times the oracle on stratified panels and counts executed FLOP
    as the GPU line does (every allowed tile's QK^T, the kept tiles' P.V)."""
    from block_sparse_flashattention_amd import inputs

    w = inputs.WORKLOADS["single_head_1k"]
    r = bench.cpu_baseline(w, budget_s=0.0)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0.0 and r["cores"] >= 1 and r["elapsed_s"] > 0.0
    assert r["sample"].startswith("2 (query tile, head) panels")
