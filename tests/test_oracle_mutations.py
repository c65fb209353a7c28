"""Plant plausible mistakes in the CPU oracle and check that some pin catches each one.

Every mutant is applied with monkeypatch (CPU only, undone after the test). The pins
themselves live in test_oracle.py and are re-run here against the mutant.
"""
import math

import numpy as np
import pytest

from oracle import bsfa_oracle as orc
from tests import test_oracle as pins


def _combine_no_renorm(s_panel, a_panel, keep, v, block_k):
    # Mistake: skipped blocks stay in the softmax denominator.
    n_rows, n_cols = s_panel.shape
    col_keep = np.repeat(keep, block_k)[:n_cols]
    member = a_panel & col_keep[None, :]
    out = np.zeros((n_rows, v.shape[1]))
    lse = np.full(n_rows, -np.inf)
    for r in range(n_rows):
        idx = np.nonzero(a_panel[r])[0]
        if idx.size == 0:
            continue
        s = s_panel[r, idx]
        top = s.max()
        w = np.exp(s - top) * member[r, idx]
        total = np.exp(s - top).sum()
        lse[r] = top + math.log(total)
        out[r] = (w / total) @ np.asarray(v, dtype=np.float64)[idx]
    return out, lse


def _tile_max_all_elements(s_panel, a_panel, block_k):
    # Mistake: the block maximum also looks at statically masked elements.
    maxima, allowed = orc.__dict__["_orig_tile_max"](s_panel, a_panel, block_k)
    for c in range(maxima.size):
        if allowed[c]:
            maxima[c] = s_panel[:, c * block_k:(c + 1) * block_k].max()
    return maxima, allowed


def _keep_strict(maxima, allowed, forced, tau):
    # Mistake: a block whose maximum equals tau is skipped.
    if tau is None:
        return allowed.copy()
    return allowed & (forced | (maxima > tau))


def _mask_window_off_by_one(rows, cols, n, spec):
    i = np.asarray(rows)[:, None]
    j = np.asarray(cols)[None, :]
    a = orc.__dict__["_orig_element_mask"](rows, cols, n, spec)
    if spec.window > 0:
        a = a | ((np.abs(i - j) == spec.window) & (j <= i) & (i < n) & (j < n))
    return a


def _scores_unscaled(q_rows, k, scale):
    return np.asarray(q_rows, dtype=np.float64) @ np.asarray(k, dtype=np.float64).T


MUTANTS = {
    "no_renormalisation": ("combine", _combine_no_renorm),
    "max_over_masked": ("tile_max", _tile_max_all_elements),
    "strict_tie": ("keep_tiles", _keep_strict),
    "window_off_by_one": ("element_mask", _mask_window_off_by_one),
    "missing_scale": ("scores", _scores_unscaled),
}

PINS = [
    pins.test_worked_sparse_output_example,
    pins.test_window_range,
    lambda: pins.test_dense_limit_equals_sdpa(True, 200),
    pins.test_static_masks_equal_sdpa_with_that_mask,
    pins.test_zero_queries_closed_form,
    lambda: pins.test_invariants(0),
    lambda: pins.test_brute_force_tiny(130, 64, 64, True, 40, 5, 0.5),
    lambda: pins.test_brute_force_tiny(50, 2, 3, True, 9, 4, 0.0),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(name, monkeypatch):
    fn_name, mutant = MUTANTS[name]
    monkeypatch.setitem(orc.__dict__, "_orig_tile_max", orc.tile_max)
    monkeypatch.setitem(orc.__dict__, "_orig_element_mask", orc.element_mask)
    monkeypatch.setattr(orc, fn_name, mutant)
    caught = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught mutant {name}"
