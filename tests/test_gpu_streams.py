"""The library keeps no per-call state: forward and decode calls queued on two streams at
once, from two host threads, give the same bits as the same calls run one after the
other."""
import threading

import numpy as np
import pytest

from block_sparse_flashattention_amd import inputs
from tests import parity_helpers as ph

pytestmark = pytest.mark.gpu


def test_two_streams_two_threads_match_sequential():
    import torch

    import block_sparse_flashattention_amd as bsfa

    w = inputs.Workload("streams", 1, 8, 2, 1500, 128, causal=True, kind="planted",
                        planted_frac=0.1)
    dw = inputs.DecodeWorkload("streams_decode", 2, 8, 2, 1200, 128, lengths=(1200, 555),
                               kind="sink_local")
    ph.log(f"case two streams: {w} and {dw}")
    dev = torch.device("cuda")
    mask = ph.gpu_spec(w)
    tau = torch.tensor(ph.oracle_tau(w, 0.5), dtype=torch.float32, device=dev)
    dtau = torch.tensor(ph.oracle_tau_decode(dw, 0.5), dtype=torch.float32, device=dev)
    lists = bsfa.BlockLists.get(mask, w.N, dev)
    jobs = []
    for seed in (0, 2):
        q, k, v = (ph.to_dev(x) for x in inputs.generate(w, seed))
        dq, dk, dv, lengths = inputs.generate_decode(dw, seed)
        jobs.append((q, k, v, ph.to_dev(dq), ph.to_dev(dk), ph.to_dev(dv),
                     torch.tensor(lengths, dtype=torch.int32, device=dev)))
    torch.cuda.synchronize()

    def run(job, stream):
        q, k, v, dq, dk, dv, lens = job
        with torch.cuda.stream(stream):
            r = bsfa.fwd(q, k, v, mask=mask, tau=tau, stats=True, lists=lists,
                         stream=stream.cuda_stream)
            d = bsfa.decode(dq, dk, dv, lens, mask=mask, tau=dtau, stream=stream.cuda_stream)
        return r, d

    ref = [run(job, torch.cuda.current_stream()) for job in jobs]
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = [None, None]

    def worker(i):
        got[i] = run(jobs[i], streams[i])

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for i in range(2):
        (r0, d0), (r1, d1) = ref[i], got[i]
        assert torch.equal(r0.out.view(torch.int16), r1.out.view(torch.int16))
        assert torch.equal(r0.lse, r1.lse) and torch.equal(r0.stats, r1.stats)
        assert torch.equal(d0.out.view(torch.int16), d1.out.view(torch.int16))
        assert torch.equal(d0.lse, d1.lse)
    # the two inputs differ, so equal results are not an accident of shared buffers
    assert not torch.equal(ref[0][0].out, ref[1][0].out)
    ph.log("two streams, two threads: bit-identical to sequential calls")


def test_stream_argument_outside_a_stream_context():
    """A call handed a stream other than torch's current one, outside any stream context,
    while the current stream is still busy: the temporaries the call allocates (the
    zeroed counters, the tau copy, the decode and calibration workspaces) are ordered on
    the launch stream, so the results equal those of calls on the current stream."""
    import torch

    import block_sparse_flashattention_amd as bsfa

    w = inputs.Workload("side_stream", 1, 8, 2, 1000, 128, causal=True, kind="planted",
                        planted_frac=0.1)
    dw = inputs.DecodeWorkload("side_stream_decode", 2, 8, 2, 900, 128, lengths=(900, 321),
                               kind="sink_local")
    ph.log(f"case stream argument without context: {w} and {dw}")
    dev = torch.device("cuda")
    mask = ph.gpu_spec(w)
    tau = ph.oracle_tau(w, 0.5).astype(np.float32)
    dtau = ph.oracle_tau_decode(dw, 0.5).astype(np.float32)
    q, k, v = (ph.to_dev(x) for x in inputs.generate(w, 0))
    qc, kc, _ = (ph.to_dev(x) for x in inputs.generate(w, 1))
    dq, dk, dv, lengths = inputs.generate_decode(dw, 0)
    dq, dk, dv = ph.to_dev(dq), ph.to_dev(dk), ph.to_dev(dv)
    lens = torch.tensor(lengths, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    ref = bsfa.fwd(q, k, v, mask=mask, tau=tau, stats=True, export_tiles=True)
    dref = bsfa.decode(dq, dk, dv, lens, mask=mask, tau=dtau, stats=True)
    tref = bsfa.calibrate_tau(qc, kc, mask, 0.5)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(20_000_000)  # keep the current stream busy for a while
    got = bsfa.fwd(q, k, v, mask=mask, tau=tau, stats=True, export_tiles=True,
                   stream=side.cuda_stream)
    dgot = bsfa.decode(dq, dk, dv, lens, mask=mask, tau=dtau, stats=True,
                       stream=side.cuda_stream)
    tgot = bsfa.calibrate_tau(qc, kc, mask, 0.5, stream=side.cuda_stream)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(ref.out.view(torch.int16), got.out.view(torch.int16))
    assert torch.equal(ref.lse, got.lse) and torch.equal(ref.stats, got.stats)
    assert torch.equal(ref.keep, got.keep) and torch.equal(ref.tile_max, got.tile_max)
    assert int(got.stats.sum()) == w.Hq * got.lists.nnz
    assert torch.equal(dref.out.view(torch.int16), dgot.out.view(torch.int16))
    assert torch.equal(dref.lse, dgot.lse) and torch.equal(dref.stats, dgot.stats)
    assert np.array_equal(tref, tgot)
    ph.log("stream argument without context: identical to calls on the current stream")
