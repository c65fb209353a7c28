"""Shared plumbing for the GPU parity tests: run the HIP path and the CPU oracle on the
same seeded inputs and compare them (keep mask, block maxima, O, LSE)."""
from __future__ import annotations

import math
import sys
from dataclasses import dataclass

import numpy as np

from block_sparse_flashattention_amd import inputs
from oracle import bsfa_oracle as orc

NEAR_TAU = 1e-3  # blocks this close to tau may go either way
O_MAX, O_MEAN, LSE_MAX = 1e-2, 1e-3, 1e-3


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray, device="cuda"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def f64(bits: np.ndarray) -> np.ndarray:
    return inputs.bits_to_f32(bits).astype(np.float64)


def oracle_spec(w: inputs.Workload) -> orc.MaskSpec:
    return orc.MaskSpec(causal=w.causal, window=w.window, n_global=w.n_global)


def gpu_spec(w: inputs.Workload):
    import block_sparse_flashattention_amd as bsfa

    return bsfa.MaskSpec(causal=w.causal, window=w.window, n_global=w.n_global)


def oracle_tau(w: inputs.Workload, quantile: float, q_tiles=None, seed: int = 1) -> np.ndarray:
    """Per-head tau from the oracle's calibration on the calibration seed."""
    qb, kb, _ = inputs.generate(w, seed)
    return orc.calibrate_tau(f64(qb), f64(kb), oracle_spec(w), quantile, q_tiles=q_tiles)


def dense_keep(lists, keep_sparse: np.ndarray, q_tiles) -> np.ndarray:
    """Scatter the GPU's per-entry keep bits [B, Hq, nnz] to [B, Hq, len(q_tiles), nkb]."""
    bsz, hq, _ = keep_sparse.shape
    nkb = lists.n_qtiles
    out = np.zeros((bsz, hq, len(q_tiles), nkb), dtype=keep_sparse.dtype)
    for ti, t in enumerate(q_tiles):
        e0, e1 = lists.row_ptr_host[t], lists.row_ptr_host[t + 1]
        out[:, :, ti, lists.col_host[e0:e1]] = keep_sparse[:, :, e0:e1]
    return out


@dataclass
class Report:
    o_max: float
    o_mean: float
    lse_max: float
    near: int
    kept: int
    total: int
    tmax_err: float


def compare(w: inputs.Workload, qb, kb, vb, res, tau, q_tiles=None, heads=None,
            check_keep=True) -> Report:
    """Compare one GPU result with the oracle on the selected query tiles and heads."""
    spec = oracle_spec(w)
    nqt = -(-w.N // 64)
    q_tiles = list(range(nqt)) if q_tiles is None else list(q_tiles)
    heads = list(range(w.Hq)) if heads is None else list(heads)
    q, k, v = f64(qb), f64(kb), f64(vb)
    near_cnt, tmax_err = 0, 0.0
    override = None
    kept = total = 0
    if tau is not None and res.keep is not None:
        keep_gpu = res.keep.cpu().numpy().astype(bool)
        tmax_gpu = res.tile_max.cpu().numpy().astype(np.float64)
        kd = dense_keep(res.lists, keep_gpu, q_tiles)[:, heads]
        md = dense_keep(res.lists, tmax_gpu, q_tiles)[:, heads]
        ref = orc.attention(q, k, v, spec, tau=tau, q_tiles=q_tiles, heads=heads)
        allowed = ref.allowed[None, None]
        tau_h = np.asarray(tau, dtype=np.float64)[heads][None, :, None, None]
        near = (np.abs(ref.tile_max - tau_h) <= NEAR_TAU) & allowed & ~ref.forced[None, None]
        near_cnt = int(near.sum())
        if near_cnt:
            log(f"near-tau blocks (|M - tau| <= {NEAR_TAU}): {near_cnt}; "
                f"GPU/oracle disagree on {int(((kd != ref.keep) & near).sum())} of them")
        if check_keep:
            mism = (kd != ref.keep) & allowed & ~near
            assert not mism.any(), f"keep mask differs on {int(mism.sum())} non-near tiles"
        tmax_err = float(np.abs(np.where(allowed, md - ref.tile_max, 0.0)).max())
        assert tmax_err <= NEAR_TAU, f"block maxima differ by {tmax_err}"
        override = kd
        kept = int((kd & allowed).sum())
        total = int(np.broadcast_to(allowed, kd.shape).sum())
    ref = orc.attention(q, k, v, spec, tau=tau, q_tiles=q_tiles, heads=heads,
                        keep_override=override)
    out = res.out.float().cpu().numpy()
    lse = res.lse.cpu().numpy()
    o_err, l_err = [], []
    for ti, t in enumerate(q_tiles):
        r0, r1 = t * 64, min(t * 64 + 64, w.N)
        go = out[:, heads, r0:r1]
        ro = ref.out[:, :, ti, : r1 - r0]
        o_err.append(np.abs(go - ro).reshape(-1))
        gl = lse[:, heads, r0:r1]
        rl = ref.lse[:, :, ti, : r1 - r0]
        both_inf = np.isneginf(gl) & np.isneginf(rl)
        l_err.append(np.where(both_inf, 0.0, np.abs(gl - rl)).reshape(-1))
    o_err = np.concatenate(o_err)
    l_err = np.concatenate(l_err)
    rep = Report(float(o_err.max()), float(o_err.mean()), float(l_err.max()), near_cnt,
                 kept, total, tmax_err)
    log(f"{w.name} N={w.N} Hq={w.Hq}: max|dO|={rep.o_max:.3e} mean|dO|={rep.o_mean:.3e} "
        f"max|dLSE|={rep.lse_max:.3e} max|dM|={rep.tmax_err:.2e} near={near_cnt}")
    assert np.isfinite(o_err).all(), "non-finite output"
    assert rep.o_max <= O_MAX and rep.o_mean <= O_MEAN, rep
    assert rep.lse_max <= LSE_MAX, rep
    return rep


def run_gpu(w: inputs.Workload, qb, kb, vb, tau, export=True, stats=True, poison=True):
    import torch

    import block_sparse_flashattention_amd as bsfa

    dev = torch.device("cuda")
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    out_dtype = torch.float32 if w.out_f32 else torch.bfloat16
    out = torch.full((w.B, w.Hq, w.N, w.d), math.nan, dtype=out_dtype, device=dev) if poison else None
    tau_t = None if tau is None else torch.tensor(np.asarray(tau, dtype=np.float32), device=dev)
    res = bsfa.fwd(q, k, v, mask=gpu_spec(w), tau=tau_t, out_dtype=out_dtype, out=out,
                   stats=stats, export_tiles=export and tau is not None)
    torch.cuda.synchronize()
    return res
