"""Plant plausible decode mistakes in the CPU oracle and check that some decode pin
catches each one (CPU only; every mutant is undone after its test)."""
import numpy as np
import pytest

from oracle import bsfa_oracle as orc
from tests import test_oracle_decode as pins
from tests.test_oracle_mutations import (_combine_no_renorm, _keep_strict, _scores_unscaled,
                                         _tile_max_all_elements)


def _forced_previous_block(t, n, spec, block_q, block_k):
    # Mistake (single-row tiles): the block before the row's own one is forced instead.
    f = orc.__dict__["_orig_forced_tiles"](t, n, spec, block_q, block_k)
    if block_q == 1:
        own = t // block_k
        f[own] = spec.force_keep_global and own * block_k < min(spec.n_global, n)
        if own > 0:
            f[own - 1] = True
    return f


def _row_is_previous_token(rows, cols, n, spec):
    # Mistake (single-row panels): the new token is taken at position length - 2.
    rows = np.asarray(rows)
    if rows.size == 1 and rows[0] > 0:
        rows = rows - 1
    return orc.__dict__["_orig_element_mask"](rows, cols, n, spec)


def _global_not_forced(t, n, spec, block_q, block_k):
    # Mistake: global blocks go through the gate like any other block.
    f = orc.__dict__["_orig_forced_tiles"](t, n, spec, block_q, block_k)
    if spec.n_global > 0:
        nkb = orc.tile_grid(n, block_k)
        r0, r1 = t * block_q, min((t + 1) * block_q, n)
        for c in range(nkb):
            c0, c1 = c * block_k, min((c + 1) * block_k, n)
            f[c] = spec.force_keep_diag and max(r0, c0) < min(r1, c1)
    return f


MUTANTS = {
    "no_renormalisation": ("combine", _combine_no_renorm),
    "max_over_masked": ("tile_max", _tile_max_all_elements),
    "strict_tie": ("keep_tiles", _keep_strict),
    "missing_scale": ("scores", _scores_unscaled),
    "forced_previous_block": ("forced_tiles", _forced_previous_block),
    "row_is_previous_token": ("element_mask", _row_is_previous_token),
    "global_not_forced": ("forced_tiles", _global_not_forced),
}

PINS = [
    pins.test_dense_decode_equals_sdpa_and_logsumexp,
    pins.test_window_and_global_decode_equals_masked_sdpa,
    pins.test_tau_inf_keeps_forced_blocks_only,
    pins.test_zero_query_closed_forms,
    lambda: pins.test_brute_force_loops(1),
    lambda: pins.test_brute_force_loops(3),
    lambda: pins.test_brute_force_loops(64),
    pins.test_length_edges,
    pins.test_calibration_hits_target_and_monotone_keep,
    pins.test_gate_ignores_statically_masked_keys,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_decode_pin_catches_mutant(name, monkeypatch):
    fn_name, mutant = MUTANTS[name]
    monkeypatch.setitem(orc.__dict__, "_orig_tile_max", orc.tile_max)
    monkeypatch.setitem(orc.__dict__, "_orig_element_mask", orc.element_mask)
    monkeypatch.setitem(orc.__dict__, "_orig_forced_tiles", orc.forced_tiles)
    monkeypatch.setattr(orc, fn_name, mutant)
    caught = []
    for i, pin in enumerate(PINS):
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            caught.append(i)
    assert caught, f"no decode pin caught mutant {name}"


def test_unmutated_pins_pass():
    for pin in PINS:
        pin()
