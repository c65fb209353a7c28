"""Benchmark: block-sparse FlashAttention prefill on one MI355X.

Default workload: the long-context sink + local-bias GQA layer (B=1, Hq=32, Hkv=8,
N=65536, d=128, causal, bf16), tau calibrated per head for a 50% skip of eligible
blocks on a separate calibration seed.

A "step" is one forward pass over the whole hot path: every allowed 64x64 tile gets
its exact scores and block maximum, kept tiles get the online softmax and P.V, O and LSE
are written once, and the per-head kept/skipped counters are updated. The static block
lists are built once per (mask, N) and cached, as in deployment; their host build time
is reported separately. Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line (metric, value in executed TFLOP/s, roofline, cpu_baseline, ...).
On the default workload the line also carries, under "decode", the decode step's own
measurement (decode_sink_local_64k: algorithmic GB/s and its HBM roofline), taken after
the prefill timing with the prefill tensors freed; --no-decode leaves it out.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME]
       python bench.py --workload decode_sink_local_64k   (the decode step instead)
       python bench.py --copy-probe        (a plain copy of known size, for counters)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = [os.path.join(ROOT, "block_sparse_flashattention_amd", "csrc", f)
                  for f in ("bsfa_fwd.hip", "bsfa_device.h", "bsfa_host.cpp",
                            "bsfa_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bsfa_fwd_gated_sink_local_64k_traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _record_matches(rec, workload, quantile):
    return rec.get("workload_name") == workload and rec.get("tau_quantile") == quantile


def measured_traffic(workload, quantile):
    """HBM bytes per launch from the committed counter summary, if it was taken on this
    workload and tau quantile and on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    if not _record_matches(rec, workload, quantile):
        return None
    return rec.get("hbm_bytes_per_launch")


DECODE_SOURCES = [os.path.join(ROOT, "block_sparse_flashattention_amd", "csrc", f)
                  for f in ("bsfa_decode.hip", "bsfa_device.h", "bsfa_host.cpp",
                            "bsfa_internal.h")]
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bsfa_decode_sink_local_64k_traffic.json")


def measured_decode_traffic(workload, quantile):
    """HBM bytes per decode step (both kernels) from the committed counter summary, if it
    was taken on this workload and tau quantile and on the current decode source; else
    None."""
    try:
        with open(DECODE_TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    for p in DECODE_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    if rec.get("kernel_source_sha256_16") != h.hexdigest()[:16]:
        return None
    if not _record_matches(rec, workload, quantile):
        return None
    return rec.get("hbm_bytes_per_step")


def tile_flops(d: int):
    qk = 2 * 64 * 64 * d  # S = Q K^T for one 64x64 tile
    pv = 2 * 64 * 64 * d  # O += P V for one kept tile
    return qk, pv


def copy_probe():
    """One plain device copy of known size (for scaling HBM byte counters)."""
    import torch

    nbytes = 1 << 30
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes}))


def cpu_baseline(w, budget_s: float = 20.0):
    """Time the fp64 CPU oracle on a bounded, stratified sample of query tiles."""
    from block_sparse_flashattention_amd import inputs
    from oracle import bsfa_oracle as orc

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    spec = orc.MaskSpec(causal=w.causal, window=w.window, n_global=w.n_global)
    nqt = -(-w.N // 64)
    heads = [(j * w.group + j % w.group) for j in range(w.Hkv)]
    heads = [h for h in heads if h < w.Hq]
    tiles = [int((i + 0.5) * nqt / 16) for i in range(16)]
    groups = sorted({h // w.group for h in heads})
    f64 = lambda bits: inputs.bits_to_f32(bits).astype(np.float64)
    data, cal = {}, {}
    for g in groups:
        data[g] = inputs.generate_group(w, 0, 0, g)
        cal[g] = inputs.generate_group(w, 1, 0, g)
    qk_f, pv_f = tile_flops(w.d)
    done, flop, elapsed = [], 0.0, 0.0
    # thresholds from the oracle's own calibration (same tiles, calibration seed)
    taus = {}
    for h in heads:
        g = h // w.group
        qc = f64(cal[g][0][h - g * w.group])[None, None]
        kc = f64(cal[g][1])[None, None]
        taus[h] = float(orc.calibrate_tau(qc, kc, spec, 0.5, q_tiles=tiles[::4])[0])
    order = [(t, h) for t in tiles for h in heads]
    for t, h in order:
        g = h // w.group
        q = f64(data[g][0][h - g * w.group])[None, None]
        k = f64(data[g][1])[None, None]
        v = f64(data[g][2])[None, None]
        t0 = time.perf_counter()
        r = orc.attention(q, k, v, spec, tau=np.array([taus[h]]), q_tiles=[t])
        elapsed += time.perf_counter() - t0
        allowed = int(r.allowed.sum())
        kept = int(r.keep.sum())
        flop += allowed * qk_f + kept * pv_f
        done.append((t, h))
        if elapsed >= budget_s and len(done) >= 2:
            break
    return {
        "value": flop / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": min(cores, blas_threads),
        "kind": "oracle",
        "sample": (f"{len(done)} (query tile, head) panels of the same workload, stratified "
                   f"over tiles {tiles} x heads {heads}, taus from the oracle's own "
                   f"calibration; executed FLOP counted like the GPU's; "
                   f"{elapsed:.1f} s of fp64 numpy; the matrix products run on "
                   f"{min(cores, blas_threads)} BLAS threads ({cores} cores visible), "
                   f"the rest of the oracle on one"),
        "elapsed_s": elapsed,
    }


def decode_bytes(w, lengths, keep=None):
    """Algorithmic HBM bytes of one decode step: the new query rows, the K rows of every
    allowed block, the V rows of every block some query head of its KV group keeps (all
    allowed blocks on the dense path), O and LSE. ``keep``: bool [B, Hq, nkb] or None."""
    nkb = -(-w.Lmax // 64)
    row = w.d * 2
    total = w.B * w.Hq * w.d * 2 + w.B * w.Hq * w.d * (4 if w.out_f32 else 2) + w.B * w.Hq * 4
    for b in range(w.B):
        n = min(max(int(lengths[b]), 0), w.Lmax)
        rows = np.array([max(0, min(64, n - c * 64)) for c in range(nkb)])
        total += w.Hkv * int(rows.sum()) * row  # K (causal, no pattern: every block < n)
        if keep is None:
            total += w.Hkv * int(rows.sum()) * row
        else:
            kg = keep[b].reshape(w.Hkv, w.group, nkb).any(axis=1)  # [Hkv, nkb]
            total += int((kg * rows[None, :]).sum()) * row
    return total


def cpu_baseline_decode(w, lengths, budget_s: float = 20.0):
    """Time the fp64 CPU oracle's decode step on the same workload (whole sequences,
    one at a time, until the budget is spent)."""
    from block_sparse_flashattention_amd import inputs
    from oracle import bsfa_oracle as orc

    cores = len(os.sched_getaffinity(0))
    spec = orc.MaskSpec(causal=w.causal, window=w.window, n_global=w.n_global)
    f64 = lambda bits: inputs.bits_to_f32(bits).astype(np.float64)
    qc, kc, _, lc = inputs.generate_decode(w, 1)
    taus = orc.calibrate_tau_decode(f64(qc[:1]), f64(kc[:1]), lc[:1], spec, 0.5)
    del qc, kc
    qb, kb, vb, _ = inputs.generate_decode(w, 0)
    done, nbytes, elapsed = 0, 0, 0.0
    for b in range(w.B):
        q, k, v = f64(qb[b:b + 1]), f64(kb[b:b + 1]), f64(vb[b:b + 1])
        t0 = time.perf_counter()
        r = orc.decode(q, k, v, lengths[b:b + 1], spec, tau=taus)
        elapsed += time.perf_counter() - t0
        sub = inputs.scaled(w, B=1, lengths=(int(lengths[b]),))
        nbytes += decode_bytes(sub, lengths[b:b + 1], r.keep)
        done += 1
        if elapsed >= budget_s:
            break
    return {
        "value": nbytes / elapsed / 1e9,
        "unit": "GB/s (algorithmic bytes)",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{done} of {w.B} sequences of the same workload, every head, taus from "
                   f"the oracle's own calibration on sequence 0 of the calibration seed; "
                   f"{elapsed:.1f} s of fp64 numpy"),
        "elapsed_s": elapsed,
    }


def bench_decode(args, w, with_cpu=True):
    """Decode step: one new query row per sequence and head against the cache. Returns the
    JSON record (with the CPU oracle's rate when with_cpu)."""
    import torch

    import block_sparse_flashattention_amd as bsfa
    from block_sparse_flashattention_amd import inputs

    dev = torch.device("cuda:0")
    mask = bsfa.MaskSpec(causal=w.causal, window=w.window, n_global=w.n_global)
    out_dtype = torch.float32 if w.out_f32 else torch.bfloat16

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    t0 = time.perf_counter()
    qc, kc, _, lc = inputs.generate_decode(w, 1)
    taus = bsfa.decode_calibrate_tau(to_dev(qc), to_dev(kc), torch.tensor(lc, device=dev),
                                     mask, args.quantile)
    del qc, kc
    qb, kb, vb, lengths = inputs.generate_decode(w, 0)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    lens = torch.tensor(lengths, device=dev)
    del qb, kb, vb
    torch.cuda.synchronize()
    log(f"[bench] decode inputs resident and tau calibrated in {time.perf_counter() - t0:.1f} s")

    out = torch.empty((w.B, w.Hq, w.d), dtype=out_dtype, device=dev)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(bsfa.decode_workspace_size(w.B, w.Hq, w.Lmax, w.d), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)
    tau_t = torch.tensor(taus, dtype=torch.float32, device=dev)

    def call(tt):
        bsfa.decode(q, k, v, lens, mask=mask, tau=tt, out=out, lse_out=lse, workspace=ws,
                    stream=stream.cuda_stream)

    # A step takes about 0.17 ms, so the HIP events around each call also time the gap
    # between an event and the first kernel. The step time is therefore taken over the
    # timed region: K steps back to back between one pair of events, after a pass with
    # events around each call that gives the per-call median and minimum.
    def timed(tt, label):
        for _ in range(args.warmup):
            call(tt)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for s_, e_ in evs:
            s_.record(stream)
            call(tt)
            e_.record(stream)
        torch.cuda.synchronize()
        ks = [s_.elapsed_time(e_) for s_, e_ in evs]
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        r0.record(stream)
        for _ in range(args.steps):
            call(tt)
        r1.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t_start) / args.steps * 1e3
        kern = r0.elapsed_time(r1) / args.steps
        log(f"[bench] {label}: {wall:.4f} ms/step, kernels {kern:.4f} ms per step over the "
            f"region; per call mean {np.mean(ks):.4f}, min {np.min(ks):.4f}")
        return wall, kern, float(np.mean(ks)), float(np.median(ks)), float(np.min(ks))

    dense_ms, dense_kern, _, _, _ = timed(None, "dense decode (tau=NULL)")
    gated_ms, gated_kern, gated_call, gated_med, gated_min = timed(
        tau_t, f"gated decode tau@q={args.quantile}")
    res = bsfa.decode(q, k, v, lens, mask=mask, tau=tau_t, out=out, lse_out=lse, workspace=ws,
                      stats=True, export_tiles=True)
    torch.cuda.synchronize()
    keep = res.keep.cpu().numpy().astype(bool)
    st = res.stats.cpu().numpy()
    kept, skipped = int(st[..., 0].sum()), int(st[..., 1].sum())
    tmax = res.tile_max.cpu().numpy()
    allowed = tmax > -np.inf
    nkb = keep.shape[2]
    any_keep = keep.reshape(w.B, w.Hkv, w.group, nkb).any(axis=2)
    allowed_g = allowed.reshape(w.B, w.Hkv, w.group, nkb).any(axis=2)
    gated_bytes = decode_bytes(w, lengths, keep)
    dense_bytes = decode_bytes(w, lengths, None)
    value = gated_bytes / (gated_ms / 1e3) / 1e9
    dtraffic = measured_decode_traffic(w.name, args.quantile)
    achieved = gated_bytes / (gated_kern / 1e3) / 1e9
    line = {
        "metric": "BSFA decode step, algorithmic HBM GB/s (one new token per sequence)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(gated_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; no dataset or trained weights)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Lmax": w.Lmax,
                   "lengths": list(map(int, lengths)), "d": w.d, "mask": "causal",
                   "tau_quantile": args.quantile, "block": "1x64"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": dtraffic},
        "hbm_measured_gbs": (None if dtraffic is None
                             else round(dtraffic / (gated_kern / 1e3) / 1e9, 1)),
        "tokens_per_s": round(w.B / (gated_ms / 1e3), 1),
        "dense_path_ms": round(dense_ms, 5),
        "dense_path_gbs": round(dense_bytes / (dense_kern / 1e3) / 1e9, 1),
        "speedup_vs_dense": round(dense_ms / gated_ms, 4),
        "skip_fraction_allowed": round(skipped / max(kept + skipped, 1), 4),
        "v_blocks_skipped_fraction": round(1 - any_keep.sum() / max(allowed_g.sum(), 1), 4),
        "kernel_ms_mean": round(gated_kern, 5),
        "kernel_ms_per_call_mean": round(gated_call, 5),
        "kernel_ms_per_call_median": round(gated_med, 5),
        "kernel_ms_per_call_min": round(gated_min, 5),
        "algorithmic_bytes_per_step": gated_bytes,
        "dense_bytes_per_step": dense_bytes,
    }
    del q, k, v, out, lse, ws
    torch.cuda.empty_cache()
    if with_cpu:
        log("[bench] timing the CPU oracle's decode")
        line["cpu_baseline"] = cpu_baseline_decode(w, lengths, args.cpu_budget)
    return line


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="sink_local_64k")
    ap.add_argument("--quantile", type=float, default=0.5)
    ap.add_argument("--no-sweep", dest="sweep", action="store_false",
                    help="time only --quantile (by default every calibrated quantile of "
                         "the workload and tau=-inf are timed too)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", dest="decode", action="store_false",
                    help="leave the decode step's measurement out of the default line")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return

    import torch

    import block_sparse_flashattention_amd as bsfa
    from block_sparse_flashattention_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload in inputs.DECODE_WORKLOADS:
        line = bench_decode(args, inputs.DECODE_WORKLOADS[args.workload],
                            with_cpu=not args.no_cpu_baseline)
        print(json.dumps(line), flush=True)
        return
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS[args.workload]
    mask = bsfa.MaskSpec(causal=w.causal, window=w.window, n_global=w.n_global)
    out_dtype = torch.float32 if w.out_f32 else torch.bfloat16

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    t0 = time.perf_counter()
    qb, kb, vb = inputs.generate(w, 0)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    del qb, kb, vb
    qc, kc, _ = inputs.generate(w, 1)
    qc_d, kc_d = to_dev(qc), to_dev(kc)
    del qc, kc
    log(f"[bench] inputs generated and resident in {time.perf_counter() - t0:.1f} s")

    t0 = time.perf_counter()
    row_ptr, col, cls = bsfa.build_block_lists(mask, w.N)
    lists_host_s = time.perf_counter() - t0
    lists = bsfa.BlockLists.get(mask, w.N, dev)

    quantiles = sorted(set([args.quantile] + (list(w.tau_quantiles) if args.sweep else [])))
    taus = bsfa.calibrate_tau(qc_d, kc_d, mask, quantiles, lists=lists)
    torch.cuda.synchronize()
    # the whole calibration once more, warm: gate-only pass, GPU quantiles, result copy
    t0 = time.perf_counter()
    taus = bsfa.calibrate_tau(qc_d, kc_d, mask, quantiles, lists=lists)
    calib_total_ms = (time.perf_counter() - t0) * 1e3
    log(f"[bench] calibrated tau for quantiles {quantiles} in {calib_total_ms:.2f} ms")
    # the gate-only calibration pass on its own (tau = NaN: block maxima and their export)
    nan_tau = torch.full((w.Hq,), math.nan, device=dev)
    cal_ms = []
    for it in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        bsfa.fwd(qc_d, kc_d, kc_d, mask=mask, tau=nan_tau, want_lse=False,
                 export_tiles=True, lists=lists)
        e1.record()
        torch.cuda.synchronize()
        if it:
            cal_ms.append(e0.elapsed_time(e1))
    log(f"[bench] gate-only calibration pass: {np.mean(cal_ms):.3f} ms")
    del qc_d, kc_d, nan_tau
    torch.cuda.empty_cache()

    out = torch.empty((w.B, w.Hq, w.N, w.d), dtype=out_dtype, device=dev)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    stats = torch.zeros((w.B, w.Hq, 2), dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(tau_t):
        stats.zero_()
        bsfa.fwd(q, k, v, mask=mask, tau=tau_t, out=out, lse_out=lse, stats_out=stats,
                 lists=lists, stream=stream.cuda_stream)

    def timed(tau_t, label):
        for _ in range(args.warmup):
            step(tau_t)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        t_start = time.perf_counter()
        for s, e in evs:
            stats.zero_()
            s.record(stream)
            bsfa.fwd(q, k, v, mask=mask, tau=tau_t, out=out, lse_out=lse, stats_out=stats,
                     lists=lists, stream=stream.cuda_stream)
            e.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        kern_ms = [s.elapsed_time(e) for s, e in evs]
        st = stats.cpu().numpy()
        log(f"[bench] {label}: {wall / args.steps * 1e3:.3f} ms/step, kernel mean "
            f"{np.mean(kern_ms):.3f} ms (min {np.min(kern_ms):.3f})")
        return (wall / args.steps * 1e3, float(np.mean(kern_ms)), float(np.median(kern_ms)),
                float(np.min(kern_ms)), st)

    qk_f, pv_f = tile_flops(w.d)
    allowed_tiles = lists.nnz * w.B * w.Hq
    forced_tiles = int(((cls & 2) != 0).sum()) * w.B * w.Hq
    dense_flop = allowed_tiles * (qk_f + pv_f)
    alg_bytes = (2 * w.B * w.Hq * w.N * w.d * 2 + 2 * w.B * w.Hkv * w.N * w.d * 2
                 + w.B * w.Hq * w.N * 4) + (2 * w.B * w.Hq * w.N * w.d if w.out_f32 else 0)

    dense_ms, dense_kern, dense_med, dense_min, _ = timed(None, "dense path (tau=NULL)")

    results = {}
    for qi, qv in enumerate(quantiles):
        tau_t = torch.tensor(taus[qi], dtype=torch.float32, device=dev)
        ms, kern, kern_med, kern_min, st = timed(tau_t, f"gated tau@q={qv}")
        kept, skipped = int(st[..., 0].sum()), int(st[..., 1].sum())
        exec_flop = kept * (qk_f + pv_f) + skipped * qk_f
        results[qv] = dict(ms=ms, kernel_ms=kern, kernel_ms_median=kern_med,
                           kernel_ms_min=kern_min, kept=kept,
                           skipped=skipped, exec_flop=exec_flop,
                           skip_eligible=skipped / max(allowed_tiles - forced_tiles, 1),
                           skip_allowed=skipped / max(allowed_tiles, 1))
    gate_ms = None
    if args.sweep:
        gate_ms = timed(torch.full((w.Hq,), -math.inf, device=dev), "gated tau=-inf")[0]

    head = results[args.quantile]
    traffic = measured_traffic(w.name, args.quantile)
    value = head["exec_flop"] / (head["ms"] / 1e3) / 1e12
    achieved = head["exec_flop"] / (head["kernel_ms"] / 1e3) / 1e12
    line = {
        "metric": "BSFA prefill executed TFLOP/s (bf16 MFMA), % of MFMA peak, speedup vs dense path",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; no dataset or trained weights)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "mask": ("causal" if w.causal else "full")
                           + (f"+window{w.window}" if w.window else "")
                           + (f"+global{w.n_global}" if w.n_global else ""),
                   "tau_quantile": args.quantile, "block": "64x64",
                   "out_dtype": "f32" if w.out_f32 else "bf16"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "pct_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "dense_equiv_tflops": round(dense_flop / (head["ms"] / 1e3) / 1e12, 2),
        "dense_path_ms": round(dense_ms, 4),
        "dense_path_tflops": round(dense_flop / (dense_ms / 1e3) / 1e12, 2),
        "speedup_vs_dense": round(dense_ms / head["ms"], 4),
        "skip_fraction_eligible": round(head["skip_eligible"], 4),
        "skip_fraction_allowed": round(head["skip_allowed"], 4),
        "kernel_ms_mean": round(head["kernel_ms"], 4),
        "kernel_ms_median": round(head["kernel_ms_median"], 4),
        "kernel_ms_min": round(head["kernel_ms_min"], 4),
        "dense_kernel_ms_median": round(dense_med, 4),
        "dense_kernel_ms_min": round(dense_min, 4),
        "hbm_algorithmic_gbs": round(alg_bytes / (head["kernel_ms"] / 1e3) / 1e9, 1),
        # HBM bytes the counters measured for one gated launch (null when the committed
        # record does not match this kernel source, workload and quantile) per kernel time
        "hbm_measured_gbs": (None if traffic is None
                             else round(traffic / (head["kernel_ms"] / 1e3) / 1e9, 1)),
        "hbm_peak_gbs": PEAK_HBM_GBS,
        "block_lists_host_ms": round(lists_host_s * 1e3, 2),
        "calibration_pass_ms": round(float(np.mean(cal_ms)), 4),
        "calibration_total_ms": round(calib_total_ms, 3),
        "executed_flop_per_step": head["exec_flop"],
        "dense_flop_per_step": dense_flop,
    }
    if args.sweep:
        line["sweep"] = {str(qv): {"ms": round(r["ms"], 4),
                                   "exec_tflops": round(r["exec_flop"] / (r["ms"] / 1e3) / 1e12, 2),
                                   "speedup_vs_dense": round(dense_ms / r["ms"], 4),
                                   "skip_fraction_eligible": round(r["skip_eligible"], 4)}
                         for qv, r in results.items()}
        line["gated_tau_minus_inf_ms"] = round(gate_ms, 4)
    del q, k, v, out, lse
    torch.cuda.empty_cache()
    if args.decode and w.name == "sink_local_64k":
        log("[bench] the decode step (decode_sink_local_64k)")
        dl = bench_decode(args, inputs.DECODE_WORKLOADS["decode_sink_local_64k"], with_cpu=False)
        line["decode"] = {"workload": dl["config"]["workload"]} | {
            k_: dl[k_] for k_ in ("metric", "value", "unit", "ms_per_step", "kernel_ms_mean",
                                  "roofline", "hbm_measured_gbs", "tokens_per_s",
                                  "dense_path_ms", "speedup_vs_dense", "skip_fraction_allowed",
                                  "v_blocks_skipped_fraction")}
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
