"""Block-sparse FlashAttention (BSFA) prefill: a plain, slow, fp64 CPU reference.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline
leg use this module. It shares no code with the HIP path and imports nothing from it.

Sources (web pages this project is built from; cited by page title and section):

* "Sparse attention weights assumption" (1cademy), section "Sparse Attention Output
  Formula" and "Index Set of Non-Zero Attention Weights (G)": the output of query i is a
  weighted sum of the value vectors v_j over an index set G of the keys j <= i whose
  weights are non-zero; indices outside G contribute nothing, and the worked example
  uses weights that sum to one over G.
* "sparse attention mechanism" (chipfoundryservices glossary), "Standard Attention
  Bottleneck": Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V. "FlashAttention":
  exact attention computed tile by tile with a running softmax (max m, sum l). "Mistral
  sliding window": token i sees keys [max(0, i - W + 1), i]. "Multi-Query and
  Grouped-Query Attention": H query heads share G key/value heads.
* "Block Sparse Flash Attention" (AI Radio episode), "The paper's summary" and
  "The paper's improvements": the query-key scores are computed exactly first; the
  maximum score inside each block is compared with a threshold calibrated per layer and
  head; blocks below it are skipped (their value block is never loaded nor multiplied);
  one calibration on a small data set fixes the thresholds.
* "Sparse attention weights assumption", "Global Tokens in Attention": the first tokens
  are visible to every token. "SAS: Sparse Attention Synthesizer", Step 5 (Logic
  Operators): static primitives are combined with OR.

Readings taken where the pages leave a step open:

* Skipped blocks leave both the softmax numerator and its denominator: the weights of
  the kept keys are renormalised to sum to one (as the worked example's weights do).
* One block maximum per (query tile, key block), taken over the statically allowed
  elements only, on the scaled score s = scale * q . k (natural-log units). A block is
  kept when its maximum is >= tau (a tie keeps; a NaN tau keeps only forced blocks).
* Forced blocks are never skipped: the block holding the diagonal element (i, i) when
  ``force_keep_diag``, and every block holding a global key when ``force_keep_global``.
* The window is |i - j| < W; with the causal mask this is the page's [i - W + 1, i].
  Global tokens act on both sides: keys j < n_global are seen by every query, and
  queries i < n_global see every key; the causal mask still applies (AND).
* The glossary's other static patterns ("sparse attention mechanism", table "Sparse
  Attention Patterns") are read as OR-able primitives:
  - dilated/strided ("every k-th token"): key j is allowed when i - j is a multiple of
    the stride k, and, with w taps, |i - j| < k * w (no limit when w = 0);
  - blockwise ("within fixed-size blocks"): i and j lie in the same block of B tokens,
    floor(i / B) == floor(j / B);
  - BigBird's random part: whole 64-token blocks (query block t, key block c) chosen at
    random with a given rate. The choice is SplitMix64 (Steele, Lea and Flood, "Fast
    splittable pseudorandom number generators", 2014) of a counter built from (seed, t,
    c), keeping the block when the top 32 output bits fall below the rate's threshold.
  With no pattern primitive at all every pair is allowed (then global tokens change
  nothing).
* A query with no kept key gets O = 0 and LSE = -inf.
* The block size is a parameter (64 x 64 on the GPU); block size 1 turns the rule into
  an element-level one, which lets the pages' small worked examples run through it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class MaskSpec:
    """Static sparsity primitives, OR-composed under an optional causal AND."""

    causal: bool = True
    window: int = 0  # 0: no window; else |i - j| < window
    n_global: int = 0  # keys j < n_global and queries i < n_global are global
    force_keep_diag: bool = True
    force_keep_global: bool = True
    dilation: int = 0  # 0: off; else i - j must be a multiple of this stride (>= 2)
    dilation_taps: int = 0  # with a stride: |i - j| < stride * taps (0: no limit)
    block: int = 0  # 0: off; else i and j in the same block of this many tokens
    random_ppm: int = 0  # random 64-token blocks, rate in parts per million (0: off)
    random_seed: int = 0

    @property
    def has_pattern(self) -> bool:
        return (self.window > 0 or self.dilation > 0 or self.block > 0
                or self.random_ppm > 0)


RANDOM_BLOCK = 64  # granularity of the random primitive (tokens)
_M64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """SplitMix64 output for counter x (Steele, Lea and Flood, 2014): add the golden-
    ratio increment, then the variant-13 finaliser of MurmurHash3's mixer."""
    z = (x + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def random_block_selected(seed: int, t: int, c: int, ppm: int) -> bool:
    """Whether the random primitive selects 64-token query block t x key block c.

    Counter = seed * 2^40 + t * 2^20 + c (t, c < 2^20); selected when the top 32 bits of
    SplitMix64(counter) are below floor(ppm * 2^32 / 10^6)."""
    seed, t, c, ppm = int(seed), int(t), int(c), int(ppm)  # exact integer arithmetic
    if ppm <= 0:
        return False
    counter = ((seed & 0xFFFFFF) << 40) | ((t & 0xFFFFF) << 20) | (c & 0xFFFFF)
    threshold = (ppm * (1 << 32)) // 1_000_000
    return (splitmix64(counter) >> 32) < threshold


def element_mask(rows, cols, n: int, spec: MaskSpec) -> np.ndarray:
    """Static mask A(i, j) for query rows ``rows`` and key columns ``cols``.

    A(i, j) = [0 <= i, j < n] and [not causal or j <= i] and pattern(i, j), where the
    pattern is all pairs when no pattern primitive is set, else the OR of
      |i - j| < W (window),  (i - j) % k == 0 with |i - j| < k * taps (dilated),
      i // B == j // B (blockwise),  random 64-token block (i // 64, j // 64),
      j < n_global or i < n_global (global tokens).
    """
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    inside = (i >= 0) & (i < n) & (j >= 0) & (j < n)
    if spec.causal:
        causal_ok = j <= i
    else:
        causal_ok = np.ones(inside.shape, dtype=bool)
    if not spec.has_pattern:
        return inside & causal_ok
    pattern = (j < spec.n_global) | (i < spec.n_global)
    if spec.window > 0:
        pattern = pattern | (np.abs(i - j) < spec.window)
    if spec.dilation > 0:
        dil = (i - j) % spec.dilation == 0
        if spec.dilation_taps > 0:
            dil = dil & (np.abs(i - j) < spec.dilation * spec.dilation_taps)
        pattern = pattern | dil
    if spec.block > 0:
        pattern = pattern | (i // spec.block == j // spec.block)
    if spec.random_ppm > 0:
        # decide each (query block, key block) pair once, then spread it to its elements
        tb, ti = np.unique(np.asarray(rows, dtype=np.int64) // RANDOM_BLOCK,
                           return_inverse=True)
        cb, ci = np.unique(np.asarray(cols, dtype=np.int64) // RANDOM_BLOCK,
                           return_inverse=True)
        sel = np.array([[random_block_selected(spec.random_seed, int(t), int(c),
                                               spec.random_ppm) for c in cb] for t in tb],
                       dtype=bool).reshape(len(tb), len(cb))
        pattern = pattern | sel[ti.reshape(-1)[:, None], ci.reshape(-1)[None, :]]
    return inside & causal_ok & pattern


def scores(q_rows: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """s_ij = scale * sum_k q_ik k_jk in fp64 (Standard Attention Bottleneck)."""
    q64 = np.asarray(q_rows, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    return scale * (q64 @ k64.T)


def tile_grid(n: int, block: int) -> int:
    """Number of blocks of size ``block`` covering n positions (last one may be short)."""
    return (n + block - 1) // block


def tile_max(s_panel: np.ndarray, a_panel: np.ndarray, block_k: int):
    """Per key block: the maximum of s over the allowed elements of the panel.

    Returns (maxima, allowed) with maxima = -inf where a block has no allowed element.
    """
    n_cols = s_panel.shape[1]
    nkb = tile_grid(n_cols, block_k)
    maxima = np.full(nkb, -np.inf)
    allowed = np.zeros(nkb, dtype=bool)
    for c in range(nkb):
        lo, hi = c * block_k, min((c + 1) * block_k, n_cols)
        a = a_panel[:, lo:hi]
        if a.any():
            allowed[c] = True
            maxima[c] = s_panel[:, lo:hi][a].max()
    return maxima, allowed


def forced_tiles(t: int, n: int, spec: MaskSpec, block_q: int, block_k: int) -> np.ndarray:
    """Blocks of query tile t that the rule never skips (diagonal, global keys)."""
    nkb = tile_grid(n, block_k)
    forced = np.zeros(nkb, dtype=bool)
    r0, r1 = t * block_q, min((t + 1) * block_q, n)  # rows [r0, r1)
    for c in range(nkb):
        c0, c1 = c * block_k, min((c + 1) * block_k, n)  # cols [c0, c1)
        holds_diag = max(r0, c0) < min(r1, c1)
        holds_global = c0 < min(spec.n_global, n)
        forced[c] = (spec.force_keep_diag and holds_diag) or (
            spec.force_keep_global and holds_global
        )
    return forced


def keep_tiles(maxima, allowed, forced, tau) -> np.ndarray:
    """BSFA gate: an allowed block is kept if forced or if its maximum >= tau.

    tau=None is the dense path (every allowed block kept).
    """
    if tau is None:
        return allowed.copy()
    with np.errstate(invalid="ignore"):
        return allowed & (forced | (maxima >= tau))


def combine(s_panel, a_panel, keep, v, block_k: int):
    """Renormalised softmax over the kept keys K_i, then O_i = sum_j w_ij v_j.

    K_i = {j : A(i, j) and keep[j // block_k]}; LSE_i = log sum_{j in K_i} exp(s_ij);
    w_ij = exp(s_ij - LSE_i). Rows with an empty K_i give O_i = 0, LSE_i = -inf.
    """
    n_rows, n_cols = s_panel.shape
    col_keep = np.repeat(keep, block_k)[:n_cols]
    member = a_panel & col_keep[None, :]
    v64 = np.asarray(v, dtype=np.float64)
    out = np.zeros((n_rows, v64.shape[1]))
    lse = np.full(n_rows, -np.inf)
    for r in range(n_rows):
        idx = np.nonzero(member[r])[0]
        if idx.size == 0:
            continue
        s = s_panel[r, idx]
        top = s.max()
        w = np.exp(s - top)
        total = w.sum()
        lse[r] = top + math.log(total)
        out[r] = (w / total) @ v64[idx]
    return out, lse


@dataclass
class Result:
    out: np.ndarray  # [B, nH, nT, block_q, dv]; rows >= N are NaN
    lse: np.ndarray  # [B, nH, nT, block_q]
    tile_max: np.ndarray  # [B, nH, nT, nkb]; -inf where not allowed
    keep: np.ndarray  # [B, nH, nT, nkb]
    allowed: np.ndarray  # [nT, nkb]
    forced: np.ndarray  # [nT, nkb]
    heads: list
    q_tiles: list

    def full_out(self) -> np.ndarray:
        """O as [B, nH, N, dv] (all query tiles must have been evaluated)."""
        b, nh, nt, bq, dv = self.out.shape
        return self.out.reshape(b, nh, nt * bq, dv)

    def full_lse(self) -> np.ndarray:
        b, nh, nt, bq = self.lse.shape
        return self.lse.reshape(b, nh, nt * bq)


def attention(
    q,
    k,
    v,
    spec: MaskSpec,
    tau=None,
    block_q: int = 64,
    block_k: int = 64,
    scale: float | None = None,
    keep_override=None,
    q_tiles=None,
    heads=None,
) -> Result:
    """BSFA prefill forward on the CPU in fp64.

    q: [B, Hq, N, d]; k: [B, Hkv, N, d]; v: [B, Hkv, N, dv]; Hq a multiple of Hkv
    (query head h reads key/value head h // (Hq // Hkv)). tau: None (dense path), a
    scalar, or one value per query head. keep_override: optional bool
    [B, nH, nT, nkb] replacing the gate's decisions. q_tiles / heads: optional subsets
    of query tiles and query heads to evaluate (default: all).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    bsz, hq, n, d = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nqt = tile_grid(n, block_q)
    nkb = tile_grid(n, block_k)
    q_tiles = list(range(nqt)) if q_tiles is None else list(q_tiles)
    heads = list(range(hq)) if heads is None else list(heads)
    if tau is None:
        taus = [None] * hq
    else:
        tau_arr = np.broadcast_to(np.asarray(tau, dtype=np.float64), (hq,))
        taus = [float(x) for x in tau_arr]

    dv = v.shape[3]
    out = np.full((bsz, len(heads), len(q_tiles), block_q, dv), np.nan)
    lse = np.full((bsz, len(heads), len(q_tiles), block_q), np.nan)
    tmax = np.full((bsz, len(heads), len(q_tiles), nkb), -np.inf)
    keep = np.zeros((bsz, len(heads), len(q_tiles), nkb), dtype=bool)
    allowed_all = np.zeros((len(q_tiles), nkb), dtype=bool)
    forced_all = np.zeros((len(q_tiles), nkb), dtype=bool)

    cols = np.arange(n)
    for ti, t in enumerate(q_tiles):
        rows = np.arange(t * block_q, min((t + 1) * block_q, n))
        a_panel = element_mask(rows, cols, n, spec)
        forced = forced_tiles(t, n, spec, block_q, block_k)
        forced_all[ti] = forced
        for b in range(bsz):
            for hi, h in enumerate(heads):
                g = h // group
                s_panel = scores(q[b, h, rows], k[b, g], scale)
                m, allowed = tile_max(s_panel, a_panel, block_k)
                allowed_all[ti] = allowed
                if keep_override is not None:
                    kp = np.asarray(keep_override[b, hi, ti], dtype=bool) & allowed
                else:
                    kp = keep_tiles(m, allowed, forced, taus[h])
                o, l = combine(s_panel, a_panel, kp, v[b, g], block_k)
                out[b, hi, ti, : rows.size] = o
                lse[b, hi, ti, : rows.size] = l
                tmax[b, hi, ti] = m
                keep[b, hi, ti] = kp
    return Result(out, lse, tmax, keep, allowed_all, forced_all & allowed_all, heads, q_tiles)


def calibrate_tau(
    q,
    k,
    spec: MaskSpec,
    quantile: float,
    block_q: int = 64,
    block_k: int = 64,
    scale: float | None = None,
    q_tiles=None,
) -> np.ndarray:
    """One-time threshold calibration, one tau per query head.

    tau_h = the ``quantile`` (numpy's default linear interpolation) of the block maxima
    of head h over its eligible blocks (allowed and not forced) on calibration inputs,
    so that about that fraction of the eligible blocks falls below tau_h and is skipped.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    bsz, hq, n, d = q.shape
    group = hq // k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nqt = tile_grid(n, block_q)
    q_tiles = list(range(nqt)) if q_tiles is None else list(q_tiles)
    cols = np.arange(n)
    per_head = [[] for _ in range(hq)]
    for t in q_tiles:
        rows = np.arange(t * block_q, min((t + 1) * block_q, n))
        a_panel = element_mask(rows, cols, n, spec)
        forced = forced_tiles(t, n, spec, block_q, block_k)
        for b in range(bsz):
            for h in range(hq):
                s_panel = scores(q[b, h, rows], k[b, h // group], scale)
                m, allowed = tile_max(s_panel, a_panel, block_k)
                per_head[h].append(m[allowed & ~forced])
    taus = np.empty(hq)
    for h in range(hq):
        vals = np.concatenate(per_head[h]) if per_head[h] else np.empty(0)
        taus[h] = np.quantile(vals, quantile) if vals.size else -np.inf
    return taus


# ---------------------------------------------------------------------------------------
# Decode (token generation): one new query row per sequence and query head against a
# key/value cache.
#
# The pages describe token generation as one new token at a time over a cache of the
# keys and values of all earlier tokens ("SAS: Sparse Attention Synthesizer", Challenge 2
# "KV Cache Management" and Step 6), and the block gate for prefill ("Block Sparse Flash
# Attention", "The paper's summary"). Reading taken for decode:
# the query tile is that single row. Each 64-key block of the cache gets the maximum of
# the row's scaled scores over its allowed keys. The block is kept when forced (it holds
# the row's own key, or a global key) or when that maximum is >= tau_h. The output is
# the renormalised softmax over the kept keys, as in prefill. The row's position is the
# newest token, lengths[b] - 1, and its own key and value are already in the cache.
# Lengths above the cache size count as the cache size. A length <= 0 leaves the row
# with no keys: O = 0, LSE = -inf.
# ---------------------------------------------------------------------------------------


@dataclass
class DecodeResult:
    out: np.ndarray  # [B, Hq, dv]
    lse: np.ndarray  # [B, Hq]
    tile_max: np.ndarray  # [B, Hq, nkb]; -inf where not allowed
    keep: np.ndarray  # [B, Hq, nkb]
    allowed: np.ndarray  # [B, nkb]
    forced: np.ndarray  # [B, nkb]; forced and allowed


def decode(q, k_cache, v_cache, lengths, spec: MaskSpec, tau=None, block_k: int = 64,
           scale: float | None = None, keep_override=None) -> DecodeResult:
    """BSFA decode step on the CPU in fp64.

    q: [B, Hq, d], the newest token's query per sequence and head; k_cache: [B, Hkv,
    Lmax, d]; v_cache: [B, Hkv, Lmax, dv]; lengths: [B] valid cache rows per sequence.
    tau: None (dense path), a scalar, or one value per query head. keep_override:
    optional bool [B, Hq, nkb] replacing the gate's decisions. Blocks are counted over
    the cache size: nkb = ceil(Lmax / block_k).
    """
    q = np.asarray(q)
    k_cache = np.asarray(k_cache)
    v_cache = np.asarray(v_cache)
    bsz, hq, d = q.shape
    hkv, lmax = k_cache.shape[1], k_cache.shape[2]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nkb = tile_grid(lmax, block_k)
    taus = [None] * hq if tau is None else [
        float(x) for x in np.broadcast_to(np.asarray(tau, dtype=np.float64), (hq,))]
    dv = v_cache.shape[3]
    out = np.zeros((bsz, hq, dv))
    lse = np.full((bsz, hq), -np.inf)
    tmax = np.full((bsz, hq, nkb), -np.inf)
    keep = np.zeros((bsz, hq, nkb), dtype=bool)
    allowed_all = np.zeros((bsz, nkb), dtype=bool)
    forced_all = np.zeros((bsz, nkb), dtype=bool)
    for b in range(bsz):
        n = min(int(lengths[b]), lmax)
        if n <= 0:
            continue
        i = n - 1  # the new token's position
        nb = tile_grid(n, block_k)
        a_panel = element_mask([i], np.arange(n), n, spec)
        forced = forced_tiles(i, n, spec, 1, block_k)  # query tile = the single row i
        for h in range(hq):
            g = h // group
            s_panel = scores(q[b, h][None, :], k_cache[b, g, :n], scale)
            m, allowed = tile_max(s_panel, a_panel, block_k)
            if keep_override is not None:
                kp = np.asarray(keep_override[b, h, :nb], dtype=bool) & allowed
            else:
                kp = keep_tiles(m, allowed, forced, taus[h])
            o, l = combine(s_panel, a_panel, kp, v_cache[b, g, :n], block_k)
            out[b, h] = o[0]
            lse[b, h] = l[0]
            tmax[b, h, :nb] = m
            keep[b, h, :nb] = kp
            allowed_all[b, :nb] = allowed
            forced_all[b, :nb] = forced & allowed
    return DecodeResult(out, lse, tmax, keep, allowed_all, forced_all)


def calibrate_tau_decode(q, k_cache, lengths, spec: MaskSpec, quantile: float,
                         block_k: int = 64, scale: float | None = None) -> np.ndarray:
    """Decode thresholds, one per query head: the ``quantile`` (numpy's default linear
    interpolation) of head h's eligible block maxima (allowed, not forced) of the decode
    rows on calibration inputs, as for prefill but with the single-row query tile."""
    r = decode(q, k_cache, v_cache=np.zeros(np.asarray(k_cache).shape[:3] + (1,)),
               lengths=lengths, spec=spec, tau=None, block_k=block_k, scale=scale)
    hq = r.tile_max.shape[1]
    taus = np.empty(hq)
    for h in range(hq):
        eligible = r.allowed & ~r.forced
        vals = r.tile_max[:, h][eligible]
        taus[h] = np.quantile(vals, quantile) if vals.size else -np.inf
    return taus
