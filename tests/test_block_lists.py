"""The library's analytic block classification against the oracle's element mask."""
import itertools

import numpy as np
import pytest

import block_sparse_flashattention_amd as bsfa
from oracle import bsfa_oracle as orc

SPECS = [
    dict(causal=True, window=0, n_global=0),
    dict(causal=False, window=0, n_global=0),
    dict(causal=True, window=100, n_global=0),
    dict(causal=True, window=64, n_global=64),
    dict(causal=True, window=1024, n_global=64),
    dict(causal=False, window=77, n_global=5),
    dict(causal=True, window=3, n_global=1),
    dict(causal=False, window=200, n_global=130),
    dict(causal=True, window=0, n_global=128),
    # the dilated, blockwise and random primitives, alone and OR-composed
    dict(causal=True, dilation=3, dilation_taps=40),
    dict(causal=False, dilation=70),
    dict(causal=True, dilation=64, dilation_taps=5, n_global=10),
    dict(causal=True, block=100),
    dict(causal=False, block=64, n_global=3),
    dict(causal=True, random_ppm=300_000, random_seed=4),
    dict(causal=False, window=30, dilation=9, dilation_taps=7, block=150,
         random_ppm=100_000, random_seed=123, n_global=2),
]
EXTRA = SPECS[9:]


def _check(spec_kw, n, bq, bk, diag=True, glob=True):
    m = bsfa.MaskSpec(force_keep_diag=diag, force_keep_global=glob, **spec_kw)
    om = orc.MaskSpec(force_keep_diag=diag, force_keep_global=glob, **spec_kw)
    row_ptr, col, cls = bsfa.build_block_lists(m, n, bq, bk)
    nqt, nkb = -(-n // bq), -(-n // bk)
    assert row_ptr.size == nqt + 1 and row_ptr[0] == 0 and row_ptr[-1] == col.size
    a = orc.element_mask(np.arange(nqt * bq), np.arange(nkb * bk), n, om)
    tiles = a.reshape(nqt, bq, nkb, bk)
    any_allowed = tiles.any(axis=(1, 3))
    all_allowed = tiles.all(axis=(1, 3))
    for t in range(nqt):
        cols = col[row_ptr[t]:row_ptr[t + 1]]
        assert np.all(np.diff(cols) > 0)
        assert cols.tolist() == np.nonzero(any_allowed[t])[0].tolist()
        forced = orc.forced_tiles(t, n, om, bq, bk)
        for e, c in zip(range(row_ptr[t], row_ptr[t + 1]), cols):
            assert bool(cls[e] & 1) == (not all_allowed[t, c]), (t, c)
            assert bool(cls[e] & 2) == bool(forced[c]), (t, c)
            if bq == 64 and bk == 64:
                rnd = orc.random_block_selected(om.random_seed, t, c, om.random_ppm)
                assert bool(cls[e] & 4) == rnd, (t, c)


@pytest.mark.parametrize("spec_kw", SPECS)
@pytest.mark.parametrize("n", [1, 63, 64, 65, 200, 640, 1000])
def test_lists_match_element_mask_64(spec_kw, n):
    _check(spec_kw, n, 64, 64)


@pytest.mark.parametrize("spec_kw", SPECS[:6] + EXTRA)
@pytest.mark.parametrize("bq,bk", [(1, 1), (2, 3), (16, 8), (64, 32), (100, 130)])
def test_lists_match_element_mask_other_blocks(spec_kw, bq, bk):
    _check(spec_kw, 197, bq, bk)


def test_invalid_primitive_fields():
    for bad in (dict(dilation=-1), dict(block=-2), dict(dilation_taps=-3),
                dict(random_ppm=-1), dict(random_ppm=1_000_001)):
        with pytest.raises(bsfa.BsfaError):
            bsfa.build_block_lists(bsfa.MaskSpec(**bad), 128)


@pytest.mark.parametrize("diag,glob", list(itertools.product([False, True], repeat=2)))
def test_forcing_flags(diag, glob):
    _check(dict(causal=True, window=150, n_global=70), 500, 64, 64, diag, glob)


def test_long_sequence_counts():
    # causal, 64x64 tiles: allowed tiles per head = nqt (nqt + 1) / 2
    for n in (16384, 65536):
        row_ptr, col, cls = bsfa.build_block_lists(bsfa.MaskSpec(causal=True), n)
        nqt = n // 64
        assert col.size == nqt * (nqt + 1) // 2
        assert int((cls & 2).astype(bool).sum()) == nqt  # the diagonal
        assert int((cls & 1).astype(bool).sum()) == nqt  # only diagonal tiles are partial
    # causal + window 1024 + 64 global tokens at N = 4096
    row_ptr, col, cls = bsfa.build_block_lists(
        bsfa.MaskSpec(causal=True, window=1024, n_global=64), 4096)
    _check(dict(causal=True, window=1024, n_global=64), 4096, 64, 64)
    assert col.size == 999


def test_concurrent_host_calls_agree():
    """bsfa_build_block_lists and the error text are per-call / per-thread: eight threads
    building different lists at once (half of them failing on purpose) each get the lists
    or the error that a serial call gives."""
    from concurrent.futures import ThreadPoolExecutor

    from block_sparse_flashattention_amd import binding

    specs = [bsfa.MaskSpec(causal=True, window=w, n_global=g) for w in (0, 300) for g in (0, 70)]
    sizes = [1000, 4097]
    jobs = [(s, n) for s in specs for n in sizes]
    serial = [binding.build_block_lists(s, n) for s, n in jobs]

    def work(i):
        if i % 2:  # an invalid call in between: its error must stay on this thread
            with pytest.raises(binding.BsfaError):
                binding.build_block_lists(bsfa.MaskSpec(causal=True, window=-1), 100)
        return binding.build_block_lists(*jobs[i % len(jobs)])

    with ThreadPoolExecutor(8) as ex:
        got = list(ex.map(work, range(4 * len(jobs))))
    for i, g in enumerate(got):
        for a, b in zip(g, serial[i % len(jobs)]):
            np.testing.assert_array_equal(a, b)
