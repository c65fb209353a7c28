"""GPU parity with non-contiguous layouts passed through the C ABI's element strides:
tensors stored [B, N, H, d] (sequence-major, as many models keep them) and viewed as
[B, H, N, d]; a decode query and output that are slices of wider tensors."""
import math

import numpy as np
import pytest

from block_sparse_flashattention_amd import inputs
from tests import parity_helpers as ph

pytestmark = pytest.mark.gpu


def _bshd(bits, device="cuda"):
    """[B, H, N, d] bf16 bits -> a [B, H, N, d] view of a [B, N, H, d] device tensor."""
    t = ph.to_dev(np.ascontiguousarray(bits.transpose(0, 2, 1, 3)), device)
    return t.permute(0, 2, 1, 3)


def test_prefill_sequence_major_layout():
    import torch

    import block_sparse_flashattention_amd as bsfa

    w = inputs.Workload("layout_bshd", 2, 8, 2, 700, 128, causal=True, window=300,
                        n_global=16, kind="sink_local")
    ph.log(f"case prefill layout [B, N, H, d]: {w}")
    qb, kb, vb = inputs.generate(w, 0)
    q, k, v = _bshd(qb), _bshd(kb), _bshd(vb)
    assert q.stride() == (w.N * w.Hq * w.d, w.d, w.Hq * w.d, 1)
    out = torch.full((w.B, w.N, w.Hq, w.d), math.nan, dtype=torch.bfloat16,
                     device="cuda").permute(0, 2, 1, 3)
    tau = ph.oracle_tau(w, 0.5)
    res = bsfa.fwd(q, k, v, mask=ph.gpu_spec(w), tau=torch.tensor(tau, dtype=torch.float32),
                   out=out, export_tiles=True)
    torch.cuda.synchronize()
    rep = ph.compare(w, qb, kb, vb, res, tau)
    assert 0 < rep.kept < rep.total
    # the same call on contiguous tensors gives the same bits
    ref = bsfa.fwd(ph.to_dev(qb), ph.to_dev(kb), ph.to_dev(vb), mask=ph.gpu_spec(w),
                   tau=torch.tensor(tau, dtype=torch.float32))
    torch.cuda.synchronize()
    assert torch.equal(ref.out, out.contiguous())


def test_decode_sequence_major_cache_and_sliced_rows():
    import torch

    import block_sparse_flashattention_amd as bsfa

    w = inputs.DecodeWorkload("layout_decode", 3, 8, 2, 900, 128, lengths=(900, 411, 64),
                              kind="sink_local")
    ph.log(f"case decode layout: caches [B, L, Hkv, d], q and out sliced: {w}")
    qb, kb, vb, lengths = ph.decode_inputs(w, 0, poison_tail=True)
    k, v = _bshd(kb), _bshd(vb)
    wide = torch.zeros((w.B, w.Hq, 2 * w.d), dtype=torch.bfloat16, device="cuda")
    wide[..., : w.d] = ph.to_dev(qb)
    q = wide[..., : w.d]  # head stride 2d
    out_wide = torch.full((w.B, w.Hq, 3 * w.d), math.nan, dtype=torch.float32, device="cuda")
    out = out_wide[..., w.d: 2 * w.d]
    lens = torch.tensor(lengths, device="cuda")
    tau = ph.oracle_tau_decode(w, 0.5)
    res = bsfa.decode(q, k, v, lens, mask=ph.gpu_spec(w),
                      tau=torch.tensor(tau, dtype=torch.float32), out=out, stats=True,
                      export_tiles=True)
    torch.cuda.synchronize()
    ph.compare_decode(w, qb, kb, vb, lengths, res, tau)
    # the rest of the wide output buffer is untouched
    assert torch.isnan(out_wide[..., : w.d]).all() and torch.isnan(out_wide[..., 2 * w.d:]).all()
