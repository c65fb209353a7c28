"""Plain fp64 CPU oracle for block-sparse FlashAttention prefill.

Test infrastructure only: tests, the smoke check and the benchmark's CPU-baseline leg
import this package. Product code never does, and this package imports nothing from the
product package.
"""
from .bsfa_oracle import (  # noqa: F401
    MaskSpec,
    element_mask,
    scores,
    tile_grid,
    tile_max,
    forced_tiles,
    keep_tiles,
    combine,
    attention,
    calibrate_tau,
)
