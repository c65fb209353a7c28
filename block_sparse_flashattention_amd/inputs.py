"""Seeded synthetic inputs for block-sparse attention prefill workloads.

This module only draws random numbers and shapes them into Q, K, V tensors. It holds
no attention arithmetic (no scores, softmax, masks or block rule) and imports numpy
only, so both the GPU path's tests and the CPU oracle can consume the same inputs.

Every tensor is bf16: values are drawn in fp32, rounded once to bf16 with
round-to-nearest-even, and returned as raw uint16 bit patterns (``*_bits``).
``bits_to_f32`` widens them exactly.

Random streams: one ``numpy.random.Generator(PCG64(SeedSequence([seed, tensor, b,
head])))`` per (tensor, batch, head), with tensor ids Q=0, K=1, V=2 and 3 for the choice
of planted blocks. Structure vectors (u_g, c_g, mu_g) use the fixed structure seed
1000, so evaluation data (seed 0) and calibration data (seed 1) share one "model" but
not the tokens.

Workload kinds:

* ``gaussian``: Q, K, V ~ N(0, 1).
* ``planted``: K = N(0,1) + 2.0 u_g on a random fraction of the 64-token key blocks of
  each key/value head g (drawn without replacement from the data seed);
  Q = N(0,1) + 1.5 u_g on all rows; u_g is a unit Gaussian direction per KV head;
  V ~ N(0, 1).
* ``sink_local``: Q = z + mu_g + alpha R(i) c_g and K = z' + alpha R(j) c_g, where R(i)
  rotates the coordinate pairs (2f, 2f+1) by i * theta_f with
  theta_f = 10000^(-2f/d) (a RoPE-style rotation) and alpha = 3, so the score bias
  alpha^2 c^T R(j - i) c decays with the distance |i - j|; mu_g and c_g are unit
  directions. Then K row 0 of head g is shifted by 3 times the mean over rows and group
  heads of the (bf16) Q: an attention sink. V ~ N(0, 1).
"""
from __future__ import annotations

import os
from dataclasses import dataclass, field

import numpy as np

STRUCTURE_SEED = 1000
TID_Q, TID_K, TID_V, TID_BLOCKS = 0, 1, 2, 3
SID_U, SID_C, SID_MU = 10, 11, 12


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool = True
    window: int = 0
    n_global: int = 0
    kind: str = "gaussian"  # gaussian | planted | sink_local
    planted_frac: float = 0.0
    out_f32: bool = False
    # quantiles of the eligible block maxima used to calibrate tau; () = no skipping
    tau_quantiles: tuple = field(default_factory=tuple)
    # further static mask fields as (name, value) pairs: dilation, dilation_taps, block,
    # random_ppm, random_seed
    mask_extra: tuple = field(default_factory=tuple)

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    "single_head_1k": Workload(
        "single_head_1k", 1, 1, 1, 1024, 64, causal=True, kind="gaussian",
        out_f32=True, tau_quantiles=(0.5,)),
    "static_mask_4k": Workload(
        "static_mask_4k", 1, 8, 8, 4096, 128, causal=True, window=1024, n_global=64,
        kind="gaussian"),
    "gqa_planted_16k": Workload(
        "gqa_planted_16k", 1, 32, 8, 16384, 128, causal=True, kind="planted",
        planted_frac=0.10, tau_quantiles=(0.5,)),
    "sink_local_64k": Workload(
        "sink_local_64k", 1, 32, 8, 65536, 128, causal=True, kind="sink_local",
        tau_quantiles=(0.4, 0.5, 0.6)),
    # multi-head attention (one query head per KV head) at the 64K sink/local shape: each
    # workgroup serves four adjacent query tiles of one head
    "mha_sink_local_64k": Workload(
        "mha_sink_local_64k", 1, 32, 32, 65536, 128, causal=True, kind="sink_local",
        tau_quantiles=(0.5,)),
    "gqa70b_planted_128k": Workload(
        "gqa70b_planted_128k", 1, 64, 8, 131072, 128, causal=True, n_global=128,
        kind="planted", planted_frac=0.05, tau_quantiles=(0.5,)),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _unit(key, d: int) -> np.ndarray:
    x = _rng(*key).standard_normal(d)
    return (x / np.linalg.norm(x)).astype(np.float32)


def _rotated(c: np.ndarray, n: int) -> np.ndarray:
    """Rows R(i) c for i = 0..n-1: pair (2f, 2f+1) rotated by i * 10000^(-2f/d)."""
    d = c.size
    f = np.arange(d // 2, dtype=np.float64)
    theta = 10000.0 ** (-2.0 * f / d)
    ang = np.arange(n, dtype=np.float64)[:, None] * theta[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    a, b = c[0::2].astype(np.float64), c[1::2].astype(np.float64)
    out = np.empty((n, d), dtype=np.float32)
    out[:, 0::2] = a * cos - b * sin
    out[:, 1::2] = a * sin + b * cos
    return out


def generate_group(w: Workload, seed: int, b: int, g: int):
    """Q for the query heads of KV head g, and K_g, V_g, as bf16 bits.

    Returns (q_bits [group, N, d], k_bits [N, d], v_bits [N, d]).
    """
    n, d, grp = w.N, w.d, w.group
    heads = range(g * grp, (g + 1) * grp)
    q = np.empty((grp, n, d), dtype=np.float32)
    for i, h in enumerate(heads):
        q[i] = _rng(seed, TID_Q, b, h).standard_normal((n, d), dtype=np.float32)
    k = _rng(seed, TID_K, b, g).standard_normal((n, d), dtype=np.float32)
    v = _rng(seed, TID_V, b, g).standard_normal((n, d), dtype=np.float32)

    if w.kind == "planted":
        u = _unit((STRUCTURE_SEED, SID_U, g), d)
        nblk = (n + 63) // 64
        count = int(round(w.planted_frac * nblk))
        chosen = _rng(seed, TID_BLOCKS, b, g).choice(nblk, size=count, replace=False)
        for blk in chosen:
            k[blk * 64:(blk + 1) * 64] += np.float32(2.0) * u
        q += np.float32(1.5) * u
    elif w.kind == "sink_local":
        alpha = np.float32(3.0)
        c = _unit((STRUCTURE_SEED, SID_C, g), d)
        mu = _unit((STRUCTURE_SEED, SID_MU, g), d)
        rc = alpha * _rotated(c, n)
        q += mu
        q += rc[None]
        k += rc
    elif w.kind != "gaussian":
        raise ValueError(f"unknown workload kind {w.kind!r}")

    q_bits = f32_to_bf16_bits(q)
    if w.kind == "sink_local":
        qmean = bits_to_f32(q_bits).astype(np.float64).mean(axis=(0, 1))
        k[0] += (3.0 * qmean).astype(np.float32)
    return q_bits, f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def generate(w: Workload, seed: int, groups=None):
    """Whole-workload tensors as bf16 bits.

    Returns q_bits [B, Hq, N, d], k_bits [B, Hkv, N, d], v_bits [B, Hkv, N, d]. With
    ``groups`` given, only those KV heads (and their query heads) are generated; the
    other entries are left zero.
    """
    groups = range(w.Hkv) if groups is None else groups
    q = np.zeros((w.B, w.Hq, w.N, w.d), dtype=np.uint16)
    k = np.zeros((w.B, w.Hkv, w.N, w.d), dtype=np.uint16)
    v = np.zeros((w.B, w.Hkv, w.N, w.d), dtype=np.uint16)
    for b in range(w.B):
        for g in groups:
            qg, kg, vg = generate_group(w, seed, b, g)
            q[b, g * w.group:(g + 1) * w.group] = qg
            k[b, g] = kg
            v[b, g] = vg
    return q, k, v


# ---------------------------------------------------------------------------------------
# Decode workloads: one new query row per (sequence, query head) against a key/value cache
# of Lmax rows, of which lengths[b] are valid; the new token is row lengths[b] - 1.
# Streams: tensor ids 5 (new query rows), 6 (K cache), 7 (V cache), 8 (planted blocks).
# The structure vectors are the prefill ones (structure seed 1000), so a decode workload
# of a kind has the same "model" as the prefill workload of that kind:
# * sink_local: q = z + mu_g + alpha R(p) c_g at the row's position p, the cache
#   K_j = z'_j + alpha R(j) c_g; K row 0 is shifted by 3 times the mean of the group's
#   new (bf16) query rows (the attention sink).
# * planted: K = N(0,1) + 2.0 u_g on a random fraction of the 64-token blocks of the
#   cache; q = N(0,1) + 1.5 u_g.
# * gaussian: all N(0, 1).
# ---------------------------------------------------------------------------------------
TID_DQ, TID_DK, TID_DV, TID_DBLOCKS = 5, 6, 7, 8


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Lmax: int
    d: int
    lengths: tuple  # valid cache rows per sequence
    kind: str = "gaussian"
    causal: bool = True
    window: int = 0
    n_global: int = 0
    planted_frac: float = 0.0
    out_f32: bool = False
    tau_quantiles: tuple = field(default_factory=tuple)
    mask_extra: tuple = field(default_factory=tuple)

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv


DECODE_WORKLOADS = {
    # four sequences of ragged lengths over a 64K-row cache, Llama-70B-like GQA heads
    "decode_sink_local_64k": DecodeWorkload(
        "decode_sink_local_64k", 4, 32, 8, 65536, 128,
        lengths=(65536, 57345, 49150, 40961), kind="sink_local", tau_quantiles=(0.5,)),
}


def generate_decode_group(w: DecodeWorkload, seed: int, b: int, g: int, rot=None):
    """New query rows of KV head g's query heads and its caches, as bf16 bits.

    Returns (q_bits [group, d], k_bits [Lmax, d], v_bits [Lmax, d]). ``rot`` may pass
    alpha * R(j) c_g for all cache rows (it depends on g only) to skip recomputing it.
    """
    lmax, d, grp = w.Lmax, w.d, w.group
    p = max(int(w.lengths[b]) - 1, 0)
    heads = range(g * grp, (g + 1) * grp)
    q = np.stack([_rng(seed, TID_DQ, b, h).standard_normal(d, dtype=np.float32)
                  for h in heads])
    k = _rng(seed, TID_DK, b, g).standard_normal((lmax, d), dtype=np.float32)
    v = _rng(seed, TID_DV, b, g).standard_normal((lmax, d), dtype=np.float32)
    if w.kind == "planted":
        u = _unit((STRUCTURE_SEED, SID_U, g), d)
        nblk = (lmax + 63) // 64
        count = int(round(w.planted_frac * nblk))
        chosen = _rng(seed, TID_DBLOCKS, b, g).choice(nblk, size=count, replace=False)
        for blk in chosen:
            k[blk * 64:(blk + 1) * 64] += np.float32(2.0) * u
        q += np.float32(1.5) * u
    elif w.kind == "sink_local":
        alpha = np.float32(3.0)
        c = _unit((STRUCTURE_SEED, SID_C, g), d)
        mu = _unit((STRUCTURE_SEED, SID_MU, g), d)
        rc = alpha * _rotated(c, lmax) if rot is None else rot
        q += mu
        q += rc[p][None]
        k += rc
    elif w.kind != "gaussian":
        raise ValueError(f"unknown workload kind {w.kind!r}")
    q_bits = f32_to_bf16_bits(q)
    if w.kind == "sink_local":
        qmean = bits_to_f32(q_bits).astype(np.float64).mean(axis=0)
        k[0] += (3.0 * qmean).astype(np.float32)
    return q_bits, f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def generate_decode(w: DecodeWorkload, seed: int):
    """Whole decode workload: q_bits [B, Hq, d], k_bits and v_bits [B, Hkv, Lmax, d],
    lengths int32 [B]."""
    from concurrent.futures import ThreadPoolExecutor

    q = np.zeros((w.B, w.Hq, w.d), dtype=np.uint16)
    k = np.zeros((w.B, w.Hkv, w.Lmax, w.d), dtype=np.uint16)
    v = np.zeros((w.B, w.Hkv, w.Lmax, w.d), dtype=np.uint16)
    rots = {}
    if w.kind == "sink_local":
        for g in range(w.Hkv):
            rots[g] = np.float32(3.0) * _rotated(_unit((STRUCTURE_SEED, SID_C, g), w.d), w.Lmax)

    def one(bg):
        b, g = bg
        qg, kg, vg = generate_decode_group(w, seed, b, g, rots.get(g))
        q[b, g * w.group:(g + 1) * w.group] = qg
        k[b, g] = kg
        v[b, g] = vg

    # independent streams per (b, g): the result does not depend on the order
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        list(pool.map(one, [(b, g) for b in range(w.B) for g in range(w.Hkv)]))
    return q, k, v, np.asarray(w.lengths, dtype=np.int32)


def scaled(w, **changes):
    """A copy of a (prefill or decode) workload with some fields replaced (e.g. a
    smaller N for tests)."""
    fields = {f: getattr(w, f) for f in w.__dataclass_fields__}
    fields.update(changes)
    return type(w)(**fields)
