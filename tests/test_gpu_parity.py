"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Every case prints its name, shape and seed before touching the GPU. Keep masks must
match exactly except blocks whose maximum lies within 1e-3 of tau (logged); outputs
are compared with the oracle re-run on the GPU's keep mask: max |dO| <= 1e-2,
mean |dO| <= 1e-3, max |dLSE| <= 1e-3.
"""
import numpy as np
import pytest

from block_sparse_flashattention_amd import inputs
from tests import parity_helpers as ph

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS


def _case(w, tau_quantile=None, tau=None, q_tiles=None, heads=None, cal_tiles=None):
    ph.log(f"case {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} "
           f"causal={w.causal} window={w.window} n_global={w.n_global} seed=0")
    if tau_quantile is not None:
        tau = ph.oracle_tau(w, tau_quantile, q_tiles=cal_tiles)
    qb, kb, vb = inputs.generate(w, 0)
    res = ph.run_gpu(w, qb, kb, vb, tau)
    rep = ph.compare(w, qb, kb, vb, res, tau, q_tiles=q_tiles, heads=heads)
    out = res.out.float().cpu().numpy()
    assert not np.isnan(out).any(), "an output element was never written"
    if res.stats is not None:
        st = res.stats.cpu().numpy()
        nnz = res.lists.nnz
        assert np.all(st.sum(-1) == nnz), "kept + skipped must equal the allowed tiles"
        if res.keep is not None:
            assert np.array_equal(st[..., 0], res.keep.cpu().numpy().astype(np.int64).sum(-1))
    return res, rep, (qb, kb, vb), tau


def test_single_head_1k_full():
    w = W["single_head_1k"]
    res, rep, _, tau = _case(w, tau_quantile=0.5)
    skipped = res.stats.cpu().numpy()[0, 0, 1]
    eligible = res.lists.nnz - res.lists.n_qtiles
    ph.log(f"skipped {skipped} of {eligible} eligible tiles")
    assert 0.3 * eligible <= skipped <= 0.7 * eligible


def test_static_mask_4k_dense_and_gated_minus_inf():
    w = W["static_mask_4k"]
    res_dense, _, data, _ = _case(w, tau=None)
    # tau = -inf through the gated kernel keeps everything and must agree bit for bit
    res_gate = ph.run_gpu(w, *data, np.full(w.Hq, -np.inf, np.float32))
    assert np.array_equal(res_dense.out.cpu().view(dtype=__import__("torch").int16).numpy(),
                          res_gate.out.cpu().view(dtype=__import__("torch").int16).numpy())
    assert np.array_equal(res_dense.lse.cpu().numpy(), res_gate.lse.cpu().numpy())
    assert res_gate.keep.cpu().numpy().all()


@pytest.mark.parametrize("n,hq,hkv,d,causal,window,n_global,kind", [
    (1000, 4, 2, 128, True, 0, 0, "planted"),       # ragged tail, 2 heads x 2 query tiles
    (200, 2, 2, 64, False, 90, 7, "gaussian"),      # ragged, non-causal window + globals, MHA
    (640, 8, 2, 128, True, 0, 0, "planted"),        # 4 heads per workgroup
    (520, 8, 2, 64, False, 150, 9, "gaussian"),     # 4 heads per workgroup at d = 64, ragged
    (300, 8, 1, 128, False, 0, 0, "gaussian"),      # two packs share one KV head, no mask
    (777, 3, 1, 64, True, 130, 64, "gaussian"),     # 3 query heads share one KV head
    (64, 1, 1, 128, True, 0, 0, "gaussian"),        # a single tile
    (1, 1, 1, 64, True, 0, 0, "gaussian"),          # a single token
    # MHA: four query tiles per workgroup, 30 tiles (the last workgroup has two), windows
    # so the four tiles' block lists differ
    (1900, 4, 4, 128, True, 300, 64, "sink_local"),
    # 2 heads x 2 query tiles, 23 tiles (the last workgroup has one), non-causal window
    (1470, 6, 3, 64, False, 250, 20, "planted"),
])
def test_small_shapes(n, hq, hkv, d, causal, window, n_global, kind):
    w = inputs.Workload(f"small_{kind}", 1, hq, hkv, n, d, causal=causal, window=window,
                        n_global=n_global, kind=kind, planted_frac=0.1)
    _case(w, tau_quantile=0.5)
    _case(w, tau=None)


def test_batch_and_fp32_output():
    w = inputs.Workload("batch2", 2, 4, 1, 384, 128, causal=True, kind="planted",
                        planted_frac=0.2, out_f32=True)
    _case(w, tau_quantile=0.6)


@pytest.mark.parametrize("b,hq,hkv,n,d", [
    (2, 3, 3, 700, 64),    # one head x four query tiles; 11 tiles, the last workgroup has 3
    (3, 4, 2, 450, 128),   # two heads x two query tiles; 8 tiles
])
def test_member_packs_batch_fp32_output(b, hq, hkv, n, d):
    """Workgroups of query tiles (not only of heads) across a batch, with fp32 output and
    a window, so the members' block lists differ in length and start."""
    w = inputs.Workload(f"members_b{b}", b, hq, hkv, n, d, causal=True, window=200,
                        n_global=10, kind="sink_local", out_f32=True)
    _case(w, tau_quantile=0.5)
    _case(w, tau=None)


def test_batch_of_three_one_row_ragged_tail():
    """Three sequences of N = 129: the last query tile and key block hold one row each."""
    w = inputs.Workload("batch3_n129", 3, 8, 2, 129, 128, causal=True, kind="planted",
                        planted_frac=0.3)
    _case(w, tau_quantile=0.5)
    _case(w, tau=None)


def test_four_heads_d64_long_sampled():
    """The four-head kernel at d = 64 over 128 query tiles, on sampled tiles of all heads."""
    w = inputs.Workload("d64_pack4_8k", 1, 16, 4, 8192, 64, causal=True, window=3000,
                        n_global=64, kind="planted", planted_frac=0.1)
    nqt = w.N // 64
    rng = np.random.default_rng(9)
    tiles = sorted({0, 1, nqt - 1, *rng.choice(nqt, 3, replace=False).tolist()})
    cal = sorted(rng.choice(nqt, 16, replace=False).tolist())
    _case(w, tau_quantile=0.5, q_tiles=tiles, cal_tiles=cal)


def test_four_heads_d64_fp32_output():
    w = inputs.Workload("d64_pack4", 1, 8, 2, 1100, 64, causal=True, kind="planted",
                        planted_frac=0.15, out_f32=True)
    _case(w, tau_quantile=0.5)


def test_tau_nan_and_plus_inf_keep_only_forced():
    w = inputs.Workload("forced_only", 1, 2, 1, 512, 64, causal=True, window=200, n_global=70)
    qb, kb, vb = inputs.generate(w, 0)
    for val in (np.nan, np.inf):
        tau = np.full(w.Hq, val, np.float32)
        res = ph.run_gpu(w, qb, kb, vb, tau)
        forced = (res.lists.cls_host & 2) != 0
        keep = res.keep.cpu().numpy().astype(bool)
        assert np.array_equal(keep, np.broadcast_to(forced, keep.shape))
        ph.compare(w, qb, kb, vb, res, tau)


def test_deterministic_run_to_run():
    w = inputs.scaled(W["gqa_planted_16k"], N=2048)
    qb, kb, vb = inputs.generate(w, 0)
    tau = np.full(w.Hq, 0.5, np.float32)
    a = ph.run_gpu(w, qb, kb, vb, tau)
    b = ph.run_gpu(w, qb, kb, vb, tau)
    assert np.array_equal(a.out.float().cpu().numpy(), b.out.float().cpu().numpy())
    assert np.array_equal(a.lse.cpu().numpy(), b.lse.cpu().numpy())
    assert np.array_equal(a.keep.cpu().numpy(), b.keep.cpu().numpy())


def test_gqa_planted_16k_sampled():
    """Full 16K GQA shape on the GPU; the oracle checks sampled query tiles of all heads."""
    w = W["gqa_planted_16k"]
    nqt = w.N // 64
    rng = np.random.default_rng(5)
    tiles = sorted({0, nqt - 1, *rng.choice(nqt, 3, replace=False).tolist()})
    cal = sorted(rng.choice(nqt, 24, replace=False).tolist())
    res, rep, _, tau = _case(w, tau_quantile=0.5, q_tiles=tiles, cal_tiles=cal)
    st = res.stats.cpu().numpy()[0]
    frac = st[:, 1].sum() / (st.sum() - w.Hq * nqt)
    ph.log(f"eligible skip fraction at the calibrated tau: {frac:.3f}")


def _full_size(name, tiles_of, cal_of, dense_too=False, heads=None, w=None):
    w = W[name] if w is None else w
    nqt = (w.N + 63) // 64
    if heads is None:  # one query head per KV head
        heads = [g * w.group + g % w.group for g in range(w.Hkv)]
    tiles = tiles_of(nqt)
    ph.log(f"case {name} (full size): B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d}; "
           f"oracle on heads {heads}, query tiles {tiles}")
    tau = ph.oracle_tau(w, 0.5, q_tiles=cal_of(nqt), heads=heads)
    qb, kb, vb = inputs.generate(w, 0)
    res = ph.run_gpu(w, qb, kb, vb, tau)
    ph.compare(w, qb, kb, vb, res, tau, q_tiles=tiles, heads=heads)
    st = res.stats.cpu().numpy()
    assert np.all(st.sum(-1) == res.lists.nnz)
    eligible = res.lists.nnz - int(((res.lists.cls_host & 2) != 0).sum())
    frac = st[0, heads, 1].sum() / (len(heads) * eligible)
    ph.log(f"eligible skip fraction on the compared heads: {frac:.3f}")
    if dense_too:
        del res
        res = ph.run_gpu(w, qb, kb, vb, None, export=False)
        ph.compare(w, qb, kb, vb, res, None, q_tiles=tiles, heads=heads)


def test_sink_local_64k_full_size_sampled():
    """The benchmark workload at full size, gated and dense, in bench.py's launch shape."""
    _full_size("sink_local_64k", lambda n: [0, 1, n // 2, n - 2, n - 1],
               lambda n: [n // 4, n // 2, (3 * n) // 4], dense_too=True)


def test_gqa70b_planted_128k_full_size_sampled():
    """The 70B-shaped layer (Hq=64, Hkv=8, N=131072, causal + 128 global tokens)."""
    _full_size("gqa70b_planted_128k", lambda n: [0, n // 2, n - 1],
               lambda n: [n // 3, (2 * n) // 3])


def test_mha_sink_local_64k_full_size_sampled():
    """Multi-head attention at the 64K sink/local shape (Hq = Hkv = 32): workgroups of four
    adjacent query tiles of one head. Tiles 0 and 1 share a workgroup, as do the last two."""
    _full_size("mha_sink_local_64k", lambda n: [0, 1, n // 2 + 1, n - 2, n - 1],
               lambda n: [n // 4, n // 2, (3 * n) // 4], dense_too=True, heads=[0, 13, 31])


@pytest.mark.parametrize("name,heads", [("sink_local_64k", None),
                                        ("mha_sink_local_64k", [0, 13, 31])])
def test_ragged_64k_full_size_sampled(name, heads):
    """The 64K sink/local shapes with N = 65536 - 37: the last query tile has 27 rows and
    the last key block 27 keys, in both head groupings (four heads of a tile; four tiles of
    a head, where the last workgroup's last member has the ragged tile)."""
    w = inputs.scaled(W[name], N=65536 - 37)
    _full_size(name, lambda n: [0, n // 2, n - 3, n - 2, n - 1],
               lambda n: [n // 4, n // 2, (3 * n) // 4], heads=heads, w=w)
