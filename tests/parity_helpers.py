"""Shared plumbing for the GPU parity tests: run the HIP path and the CPU oracle on the
same seeded inputs and compare them (keep mask, block maxima, O, LSE).

The oracle runs on reduced fp64 arrays that hold only the compared query heads (each
with its own copy of its KV head), so full-size workloads can be checked on sampled
heads and query tiles.
"""
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
    return orc.MaskSpec(causal=w.causal, window=w.window, n_global=w.n_global,
                        **dict(w.mask_extra))


def gpu_spec(w: inputs.Workload):
    import block_sparse_flashattention_amd as bsfa

    return bsfa.MaskSpec(causal=w.causal, window=w.window, n_global=w.n_global,
                         **dict(w.mask_extra))


def reduced(w: inputs.Workload, qb, kb, vb, heads):
    """fp64 [B, len(heads), N, d] arrays for the listed query heads, K/V per head."""
    groups = [h // w.group for h in heads]
    return f64(qb[:, heads]), f64(kb[:, groups]), f64(vb[:, groups])


def oracle_tau(w: inputs.Workload, quantile: float, q_tiles=None, heads=None,
               seed: int = 1, scale=None) -> np.ndarray:
    """Per-head tau from the oracle's calibration on the calibration seed.

    With ``heads`` given, only those heads are calibrated (their KV groups generated);
    the other entries get the median of the calibrated ones (any value is a valid input:
    those heads are not compared)."""
    heads = list(range(w.Hq)) if heads is None else list(heads)
    groups = sorted({h // w.group for h in heads})
    qb, kb, _ = inputs.generate(w, seed, groups=groups)
    q, k, _ = reduced(w, qb, kb, kb, heads)
    taus = orc.calibrate_tau(q, k, oracle_spec(w), quantile, q_tiles=q_tiles, scale=scale)
    out = np.full(w.Hq, float(np.median(taus)))
    out[heads] = taus
    return out


def dense_grid(lists, per_entry: np.ndarray, q_tiles) -> np.ndarray:
    """Scatter per-CSR-entry values [B, H, nnz] to [B, H, len(q_tiles), nkb]."""
    bsz, nh, _ = per_entry.shape
    nkb = lists.n_qtiles
    out = np.zeros((bsz, nh, len(q_tiles), nkb), dtype=per_entry.dtype)
    for ti, t in enumerate(q_tiles):
        e0, e1 = lists.row_ptr_host[t], lists.row_ptr_host[t + 1]
        out[:, :, ti, lists.col_host[e0:e1]] = per_entry[:, :, e0:e1]
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
            check_keep=True, scale=None) -> Report:
    """Compare one GPU result with the oracle on the selected query tiles and heads.
    ``scale``: the softmax scale both sides use (None: 1/sqrt(d))."""
    spec = oracle_spec(w)
    nqt = -(-w.N // 64)
    q_tiles = list(range(nqt)) if q_tiles is None else list(q_tiles)
    heads = list(range(w.Hq)) if heads is None else list(heads)
    q, k, v = reduced(w, qb, kb, vb, heads)
    tau_r = None if tau is None else np.asarray(tau, dtype=np.float64)[heads]
    near_cnt, tmax_err = 0, 0.0
    override = None
    kept = total = 0
    if tau is not None and res.keep is not None:
        keep_gpu = res.keep[:, heads].cpu().numpy().astype(bool)
        tmax_gpu = res.tile_max[:, heads].cpu().numpy().astype(np.float64)
        kd = dense_grid(res.lists, keep_gpu, q_tiles)
        md = dense_grid(res.lists, tmax_gpu, q_tiles)
        ref = orc.attention(q, k, v, spec, tau=tau_r, q_tiles=q_tiles, scale=scale)
        allowed = ref.allowed[None, None]
        tau_h = tau_r[None, :, None, None]
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
    ref = orc.attention(q, k, v, spec, tau=tau_r, q_tiles=q_tiles, keep_override=override,
                        scale=scale)
    o_err, l_err = [], []
    for ti, t in enumerate(q_tiles):
        r0, r1 = t * 64, min(t * 64 + 64, w.N)
        go = res.out[:, heads, r0:r1].float().cpu().numpy()
        ro = ref.out[:, :, ti, : r1 - r0]
        o_err.append(np.abs(go - ro).reshape(-1))
        gl = res.lse[:, heads, r0:r1].cpu().numpy()
        rl = ref.lse[:, :, ti, : r1 - r0]
        both_inf = np.isneginf(gl) & np.isneginf(rl)
        l_err.append(np.where(both_inf, 0.0, np.abs(gl - rl)).reshape(-1))
    o_err = np.concatenate(o_err)
    l_err = np.concatenate(l_err)
    rep = Report(float(o_err.max()), float(o_err.mean()), float(l_err.max()), near_cnt,
                 kept, total, tmax_err)
    log(f"{w.name} N={w.N} Hq={w.Hq} heads={len(heads)} tiles={len(q_tiles)}: "
        f"max|dO|={rep.o_max:.3e} mean|dO|={rep.o_mean:.3e} max|dLSE|={rep.lse_max:.3e} "
        f"max|dM|={rep.tmax_err:.2e} near={near_cnt} kept={kept}/{total}")
    assert np.isfinite(o_err).all(), "non-finite output"
    assert rep.o_max <= O_MAX and rep.o_mean <= O_MEAN, rep
    assert rep.lse_max <= LSE_MAX, rep
    return rep


def run_gpu(w: inputs.Workload, qb, kb, vb, tau, export=True, stats=True, poison=True,
            scale=None):
    import torch

    import block_sparse_flashattention_amd as bsfa

    dev = torch.device("cuda")
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    out_dtype = torch.float32 if w.out_f32 else torch.bfloat16
    out = torch.full((w.B, w.Hq, w.N, w.d), math.nan, dtype=out_dtype, device=dev) if poison else None
    tau_t = None if tau is None else torch.tensor(np.asarray(tau, dtype=np.float32), device=dev)
    res = bsfa.fwd(q, k, v, mask=gpu_spec(w), tau=tau_t, out_dtype=out_dtype, out=out,
                   stats=stats, export_tiles=export and tau is not None,
                   softmax_scale=0.0 if scale is None else float(scale))
    torch.cuda.synchronize()
    return res


# ---------------------------------------------------------------- decode (one new row)
def decode_inputs(w, seed: int, poison_tail: bool = False):
    """Decode inputs as bf16 bits; with ``poison_tail`` the cache rows at or past each
    sequence's length hold NaN (free slots the kernel must never read)."""
    qb, kb, vb, lengths = inputs.generate_decode(w, seed)
    if poison_tail:
        nan_bits = np.uint16(0x7FC0)
        for b, n in enumerate(lengths):
            n = max(int(n), 0)
            kb[b, :, n:] = nan_bits
            vb[b, :, n:] = nan_bits
    return qb, kb, vb, lengths


def run_gpu_decode(w, qb, kb, vb, lengths, tau, export=True, stats=True):
    import torch

    import block_sparse_flashattention_amd as bsfa

    dev = torch.device("cuda")
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    lens = torch.tensor(np.asarray(lengths, dtype=np.int32), device=dev)
    out_dtype = torch.float32 if w.out_f32 else torch.bfloat16
    out = torch.full((w.B, w.Hq, w.d), math.nan, dtype=out_dtype, device=dev)
    tau_t = None if tau is None else torch.tensor(np.asarray(tau, dtype=np.float32), device=dev)
    res = bsfa.decode(q, k, v, lens, mask=gpu_spec(w), tau=tau_t, out=out, stats=stats,
                      export_tiles=export and tau is not None)
    torch.cuda.synchronize()
    return res


def oracle_tau_decode(w, quantile: float, seed: int = 1) -> np.ndarray:
    qb, kb, _, lengths = inputs.generate_decode(w, seed)
    return orc.calibrate_tau_decode(f64(qb), f64(kb), lengths, oracle_spec(w), quantile)


def compare_decode(w, qb, kb, vb, lengths, res, tau, check_keep=True) -> Report:
    """Compare one GPU decode result with the oracle: keep bits off the near-tau band,
    block maxima, then O and LSE against the oracle run on the GPU's keep bits."""
    spec = oracle_spec(w)
    q, k, v = f64(qb), f64(kb), f64(vb)
    tau_r = None if tau is None else np.asarray(tau, dtype=np.float64)
    override = None
    near_cnt, tmax_err, kept, total = 0, 0.0, 0, 0
    ref = orc.decode(q, k, v, lengths, spec, tau=tau_r)
    allowed = ref.allowed[:, None, :]
    if tau is not None and res.keep is not None:
        keep_gpu = res.keep.cpu().numpy().astype(bool)
        tmax_gpu = res.tile_max.cpu().numpy().astype(np.float64)
        # blocks that are not allowed export -inf and keep 0
        assert np.all(np.isneginf(tmax_gpu[~np.broadcast_to(allowed, tmax_gpu.shape)]))
        assert not keep_gpu[~np.broadcast_to(allowed, keep_gpu.shape)].any()
        near = ((np.abs(ref.tile_max - tau_r[None, :, None]) <= NEAR_TAU) & allowed
                & ~ref.forced[:, None, :])
        near_cnt = int(near.sum())
        if check_keep:
            mism = (keep_gpu != ref.keep) & allowed & ~near
            assert not mism.any(), f"keep bits differ on {int(mism.sum())} non-near blocks"
        with np.errstate(invalid="ignore"):  # -inf - -inf where a block is not allowed
            tmax_err = float(np.abs(np.where(allowed, tmax_gpu - ref.tile_max, 0.0)).max())
        assert tmax_err <= NEAR_TAU, f"block maxima differ by {tmax_err}"
        override = keep_gpu
        kept = int((keep_gpu & allowed).sum())
        total = int(np.broadcast_to(allowed, keep_gpu.shape).sum())
        ref = orc.decode(q, k, v, lengths, spec, tau=tau_r, keep_override=override)
    go = res.out.float().cpu().numpy()
    gl = res.lse.cpu().numpy()
    o_err = np.abs(go - ref.out).reshape(-1)
    both_inf = np.isneginf(gl) & np.isneginf(ref.lse)
    with np.errstate(invalid="ignore"):  # -inf - -inf on rows with no key
        l_err = np.where(both_inf, 0.0, np.abs(gl - ref.lse)).reshape(-1)
    rep = Report(float(o_err.max()), float(o_err.mean()), float(l_err.max()), near_cnt,
                 kept, total, tmax_err)
    log(f"{w.name} Lmax={w.Lmax} lengths={list(lengths)} Hq={w.Hq} Hkv={w.Hkv} d={w.d}: "
        f"max|dO|={rep.o_max:.3e} mean|dO|={rep.o_mean:.3e} max|dLSE|={rep.lse_max:.3e} "
        f"max|dM|={rep.tmax_err:.2e} near={near_cnt} kept={kept}/{total}")
    assert np.isfinite(o_err).all(), "non-finite output"
    assert rep.o_max <= O_MAX and rep.o_mean <= O_MEAN, rep
    assert rep.lse_max <= LSE_MAX, rep
    if res.stats is not None:
        st = res.stats.cpu().numpy()
        n_allowed = ref.allowed.sum(axis=1)[:, None]
        assert np.array_equal(st[..., 0] + st[..., 1], np.broadcast_to(n_allowed, st[..., 0].shape))
        if override is not None:
            assert np.array_equal(st[..., 0], (override & allowed).sum(axis=2))
    return rep
