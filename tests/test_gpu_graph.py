"""HIP graph capture of the hot path: a bsfa.fwd and a bsfa.decode call captured once (with
the counter clear in front of them), then replayed with new inputs copied in between and
eager calls interleaved. Every replay must equal the eager call on the same inputs bit for
bit: the kernels are deterministic and the calls allocate nothing once their buffers are
given."""
import numpy as np
import pytest

from block_sparse_flashattention_amd import inputs
from tests import parity_helpers as ph

pytestmark = pytest.mark.gpu


def _same(a, b):
    import torch

    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_fwd_graph_replays_match_eager():
    import torch

    import block_sparse_flashattention_amd as bsfa

    w = inputs.Workload("graph_fwd", 1, 8, 2, 1000, 128, causal=True, window=400,
                        n_global=16, kind="planted", planted_frac=0.1)
    ph.log(f"case graph capture of bsfa.fwd: {w}")
    dev = torch.device("cuda")
    mask = ph.gpu_spec(w)
    seeds = [0, 2, 3]
    data = [inputs.generate(w, s) for s in seeds]
    q, k, v = (ph.to_dev(x) for x in data[0])
    tau = torch.tensor(ph.oracle_tau(w, 0.5), dtype=torch.float32, device=dev)
    out = torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    stats = torch.zeros((w.B, w.Hq, 2), dtype=torch.int64, device=dev)
    lists = bsfa.BlockLists.get(mask, w.N, dev)
    side = torch.cuda.Stream()

    def call():
        stats.zero_()
        bsfa.fwd(q, k, v, mask=mask, tau=tau, out=out, lse_out=lse, stats_out=stats,
                 lists=lists, stream=side.cuda_stream)

    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call()
    torch.cuda.synchronize()
    for s, (qb, kb, vb) in zip(seeds, data):
        q.copy_(ph.to_dev(qb))
        k.copy_(ph.to_dev(kb))
        v.copy_(ph.to_dev(vb))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = bsfa.fwd(ph.to_dev(qb), ph.to_dev(kb), ph.to_dev(vb), mask=mask, tau=tau,
                       stats=True, lists=lists)
        torch.cuda.synchronize()
        assert _same(out, ref.out), f"seed {s}: O differs"
        assert _same(lse, ref.lse), f"seed {s}: LSE differs"
        assert torch.equal(stats, ref.stats), f"seed {s}: counters differ"
        kept, skipped = stats[0, :, 0].sum().item(), stats[0, :, 1].sum().item()
        assert kept > 0 and skipped > 0
        ph.log(f"replay seed {s}: bit-identical to eager ({kept} kept, {skipped} skipped)")


def test_decode_graph_replays_match_eager():
    import torch

    import block_sparse_flashattention_amd as bsfa

    w = inputs.DecodeWorkload("graph_decode", 3, 8, 2, 900, 128, lengths=(900, 411, 64),
                              kind="sink_local")
    ph.log(f"case graph capture of bsfa.decode: {w}")
    dev = torch.device("cuda")
    mask = ph.gpu_spec(w)
    cases = [inputs.generate_decode(w, s) for s in (0, 2)]
    # the second replay also changes the lengths the kernels read from device memory
    cases.append(cases[0][:3] + (np.array([700, 900, 1], dtype=np.int32),))
    q, k, v = (ph.to_dev(x) for x in cases[0][:3])
    lens = torch.tensor(cases[0][3], dtype=torch.int32, device=dev)
    tau = torch.tensor(ph.oracle_tau_decode(w, 0.5), dtype=torch.float32, device=dev)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    stats = torch.zeros((w.B, w.Hq, 2), dtype=torch.int64, device=dev)
    ws = torch.empty(bsfa.decode_workspace_size(w.B, w.Hq, w.Lmax, w.d), dtype=torch.uint8,
                     device=dev)
    side = torch.cuda.Stream()

    def call():
        stats.zero_()
        bsfa.decode(q, k, v, lens, mask=mask, tau=tau, out=out, lse_out=lse,
                    stats_out=stats, workspace=ws, stream=side.cuda_stream)

    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call()
    torch.cuda.synchronize()
    for i, (qb, kb, vb, lengths) in enumerate(cases):
        q.copy_(ph.to_dev(qb))
        k.copy_(ph.to_dev(kb))
        v.copy_(ph.to_dev(vb))
        lens.copy_(torch.tensor(lengths, dtype=torch.int32))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = bsfa.decode(ph.to_dev(qb), ph.to_dev(kb), ph.to_dev(vb),
                          torch.tensor(lengths, dtype=torch.int32, device=dev), mask=mask,
                          tau=tau, stats=True)
        torch.cuda.synchronize()
        assert _same(out, ref.out), f"case {i}: O differs"
        assert _same(lse, ref.lse), f"case {i}: LSE differs"
        assert torch.equal(stats, ref.stats), f"case {i}: counters differ"
        assert stats[..., 1].sum().item() > 0
        ph.log(f"replay {i} (lengths {list(map(int, lengths))}): bit-identical to eager")
