"""bench.py attaches a committed HBM counter record to its roofline only for the workload
and tau quantile the record was measured on."""
import json

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
