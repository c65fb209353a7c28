"""bsfa_decode_static, the decode step that allocates nothing (its per-split partials
live in the library's fixed device scratch), against bsfa_decode with a caller
workspace: two calls in a row, the second on a smaller input, each bit-identical to
bsfa_decode on the same inputs and within the parity tolerances of the fp64 oracle."""
import math

import numpy as np
import pytest

from block_sparse_flashattention_amd import inputs
from tests import parity_helpers as ph

pytestmark = pytest.mark.gpu

BIG = inputs.DecodeWorkload("static_big", 4, 32, 8, 32768, 128,
                            lengths=(32768, 20001, 9999, 1), kind="sink_local")
SMALL = inputs.DecodeWorkload("static_small", 2, 8, 2, 1000, 64, lengths=(1000, 333),
                              kind="planted", planted_frac=0.2)


def _prepare(dw):
    import torch

    dev = torch.device("cuda")
    qb, kb, vb, lengths = ph.decode_inputs(dw, 0, poison_tail=True)
    tau = ph.oracle_tau_decode(dw, 0.5)
    bufs = dict(
        q=ph.to_dev(qb), k=ph.to_dev(kb), v=ph.to_dev(vb),
        lens=torch.tensor(lengths, dtype=torch.int32, device=dev),
        tau=torch.tensor(tau.astype(np.float32), device=dev),
        out=torch.full((dw.B, dw.Hq, dw.d), math.nan, dtype=torch.bfloat16, device=dev),
        lse=torch.full((dw.B, dw.Hq), math.nan, dtype=torch.float32, device=dev),
        stats=torch.zeros((dw.B, dw.Hq, 2), dtype=torch.int64, device=dev))
    return (qb, kb, vb, lengths, tau), bufs


def test_decode_static_matches_decode_two_calls_in_a_row():
    import torch

    import block_sparse_flashattention_amd as bsfa

    ph.log(f"case decode_static: {BIG} then {SMALL}")
    host_big, big = _prepare(BIG)
    host_small, small = _prepare(SMALL)
    torch.cuda.synchronize()
    got = []
    for dw, b in ((BIG, big), (SMALL, small)):  # back to back on one stream
        got.append(bsfa.decode_static(b["q"], b["k"], b["v"], b["lens"], mask=ph.gpu_spec(dw),
                                      tau=b["tau"], out=b["out"], lse_out=b["lse"],
                                      stats_out=b["stats"]))
    torch.cuda.synchronize()
    for dw, b, r, (qb, kb, vb, lengths, tau) in ((BIG, big, got[0], host_big),
                                                  (SMALL, small, got[1], host_small)):
        ref = bsfa.decode(b["q"], b["k"], b["v"], b["lens"], mask=ph.gpu_spec(dw),
                          tau=b["tau"], stats=True, export_tiles=True)
        torch.cuda.synchronize()
        assert torch.equal(r.out.view(torch.int16), ref.out.view(torch.int16)), dw.name
        assert torch.equal(r.lse, ref.lse) and torch.equal(r.stats, ref.stats), dw.name
        ph.compare_decode(dw, qb, kb, vb, lengths, ref, tau)
        ph.log(f"{dw.name}: decode_static bit-identical to decode")
