"""The C ABI: the library loads on a CPU host, exports every declared symbol, and its
argument checks fail cleanly (these paths return before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_flashattention_amd as bsfa
from block_sparse_flashattention_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "bsfa.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|int32_t|const char\*)\s+(bsfa_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = bsfa.load_library()
    names = _declared()
    assert set(names) >= {"bsfa_build_block_lists", "bsfa_fwd", "bsfa_skip_stats",
                          "bsfa_last_error", "bsfa_abi_version", "bsfa_decode",
                          "bsfa_decode_workspace_size", "bsfa_calibrate_tau",
                          "bsfa_calibrate_workspace_size"}
    for name in names:
        assert hasattr(lib, name), name
    assert lib.bsfa_abi_version() == 5


def test_two_call_sizing_and_too_small():
    lib = bsfa.load_library()
    m = binding._CMask(1, 0, 0, 1, 1)
    nnz = ctypes.c_int64(-1)
    row_ptr = np.zeros(17, np.int32)
    assert lib.bsfa_build_block_lists(ctypes.byref(m), 1024, 64, 64, row_ptr.ctypes.data,
                                      None, None, 0, ctypes.byref(nnz)) == 0
    assert nnz.value == 136 and row_ptr[-1] == 136
    col = np.zeros(10, np.int32)
    cls = np.zeros(10, np.uint8)
    rc = lib.bsfa_build_block_lists(ctypes.byref(m), 1024, 64, 64, row_ptr.ctypes.data,
                                    col.ctypes.data, cls.ctypes.data, 10, ctypes.byref(nnz))
    assert rc == -3 and nnz.value == 136
    assert b"capacity" in lib.bsfa_last_error()


def test_block_list_argument_errors():
    lib = bsfa.load_library()
    m = binding._CMask(1, 0, 0, 1, 1)
    nnz = ctypes.c_int64(0)
    assert lib.bsfa_build_block_lists(None, 64, 64, 64, None, None, None, 0, ctypes.byref(nnz)) == -1
    assert lib.bsfa_build_block_lists(ctypes.byref(m), -1, 64, 64, None, None, None, 0, ctypes.byref(nnz)) == -1
    assert lib.bsfa_build_block_lists(ctypes.byref(m), 64, 0, 64, None, None, None, 0, ctypes.byref(nnz)) == -1
    bad = binding._CMask(1, -5, 0, 1, 1)
    assert lib.bsfa_build_block_lists(ctypes.byref(bad), 64, 64, 64, None, None, None, 0, ctypes.byref(nnz)) == -1
    assert lib.bsfa_last_error() != b""
    # an empty sequence has no tiles
    assert lib.bsfa_build_block_lists(ctypes.byref(m), 0, 64, 64, None, None, None, 0, ctypes.byref(nnz)) == 0
    assert nnz.value == 0


def _fwd_call(lib, **kw):
    args = dict(q=16, k=16, v=16, out=16, lse=None, B=1, Hq=4, Hkv=2, N=128, d=128,
                mask=binding._CMask(1, 0, 0, 1, 1),
                lists=binding._CLists(2, 64, 64, 3, 16, 16, 16),
                tau=None, scale=0.0, out_dtype=0, stats=None, tile_max=None, keep=None)
    skn = kw.pop("skn", 128)
    sqn = kw.pop("sqn", 128)
    args.update(kw)
    s = binding._CStrides(4 * 128 * 128, 128 * 128, sqn)
    sk = binding._CStrides(2 * 128 * 128, 128 * 128, skn)
    return lib.bsfa_fwd(args["q"], args["k"], args["v"], args["out"], args["lse"], args["B"],
                        args["Hq"], args["Hkv"], args["N"], args["d"], ctypes.byref(s),
                        ctypes.byref(sk), ctypes.byref(sk), ctypes.byref(s),
                        ctypes.byref(args["mask"]) if args["mask"] is not None else None,
                        ctypes.byref(args["lists"]) if args["lists"] is not None else None,
                        args["tau"], args["scale"], args["out_dtype"], args["stats"],
                        args["tile_max"], args["keep"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=3), -1),                         # Hq not a multiple of Hkv
    (dict(d=96), -2),                         # unsupported head dim
    (dict(mask=None), -1),
    (dict(lists=None), -1),
    (dict(out_dtype=7), -1),
    (dict(scale=-1.0), -1),
    (dict(scale=float("nan")), -1),
    (dict(tile_max=16), -1),                  # tile_max without keep
    (dict(tile_max=16, keep=16), -1),         # export without tau
    (dict(N=129), -1),                        # lists sized for another N
    (dict(q=None), -1),
    (dict(q=24), -2),                         # misaligned pointer
    (dict(B=-1), -1),
    (dict(sqn=-128), -2),                     # negative stride
    (dict(skn=1 << 24), -2),                  # one head's K/V rows span more than 2^31 bytes
    (dict(B=1 << 23), -2),                    # more than 2^32 work-items in one dispatch
    # one query head per KV head: workgroups of four query tiles count their steps in a
    # bitmap of ceil(N / 64) + 1 bits, at most 524288
    (dict(Hq=2, Hkv=2, N=1 << 25, skn=0,
          lists=binding._CLists(1 << 19, 64, 64, 3, 16, 16, 16)), -2),
])
def test_fwd_argument_errors(kw, code):
    lib = bsfa.load_library()
    assert _fwd_call(lib, **kw) == code
    assert lib.bsfa_last_error() != b""


def test_fwd_empty_inputs_are_a_no_op():
    lib = bsfa.load_library()
    assert _fwd_call(lib, N=0, lists=binding._CLists(0, 64, 64, 0, 16, 16, 16)) == 0
    assert _fwd_call(lib, B=0) == 0
    assert lib.bsfa_last_error() == b""


def test_skip_stats_argument_errors():
    lib = bsfa.load_library()
    assert lib.bsfa_skip_stats(None, 1, 1, 16, 16, None) == -1
    assert lib.bsfa_skip_stats(16, 1, 0, 16, 16, None) == -1


def test_decode_workspace_size():
    # B * Hq * ceil(ceil(max_len / 64) / 4) * (d + 4) * 4 bytes
    assert bsfa.decode_workspace_size(4, 32, 65536, 128) == 4 * 32 * 256 * 132 * 4
    assert bsfa.decode_workspace_size(1, 1, 1, 64) == 68 * 4
    assert bsfa.decode_workspace_size(2, 3, 257, 64) == 2 * 3 * 2 * 68 * 4
    assert bsfa.decode_workspace_size(0, 8, 100, 128) == 0
    lib = bsfa.load_library()
    nb = ctypes.c_int64(0)
    assert lib.bsfa_decode_workspace_size(1, 1, 0, 128, ctypes.byref(nb)) == -1
    assert lib.bsfa_decode_workspace_size(1, 1, 64, 96, ctypes.byref(nb)) == -2
    assert lib.bsfa_decode_workspace_size(1, 1, 64, 128, None) == -1


def _decode_call(lib, **kw):
    args = dict(q=16, k=16, v=16, lengths=16, out=16, lse=None, B=2, Hq=8, Hkv=2, L=1024,
                d=128, mask=binding._CMask(1, 0, 0, 1, 1), tau=None, scale=0.0, out_dtype=0,
                stats=None, tile_max=None, keep=None, ws=16, ws_bytes=1 << 30)
    skn = kw.pop("skn", 128)
    args.update(kw)
    sq = binding._CStrides(8 * 128, 128, 0)
    sk = binding._CStrides(2 * 1024 * 128, 1024 * 128, skn)
    return lib.bsfa_decode(args["q"], args["k"], args["v"], args["lengths"], args["out"],
                           args["lse"], args["B"], args["Hq"], args["Hkv"], args["L"],
                           args["d"], ctypes.byref(sq), ctypes.byref(sk), ctypes.byref(sk),
                           ctypes.byref(sq),
                           ctypes.byref(args["mask"]) if args["mask"] is not None else None,
                           args["tau"], args["scale"], args["out_dtype"], args["stats"],
                           args["tile_max"], args["keep"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=7), -1),                         # Hq not a multiple of Hkv
    (dict(Hq=66, Hkv=2), -2),                 # more than 32 query heads per KV head
    (dict(d=96), -2),
    (dict(L=0), -1),
    (dict(mask=None), -1),
    (dict(out_dtype=5), -1),
    (dict(scale=float("inf")), -1),
    (dict(keep=16), -1),                      # keep without tile_max
    (dict(tile_max=16, keep=16), -1),         # export without tau
    (dict(lengths=None), -1),
    (dict(ws=None), -1),
    (dict(ws=8), -2),                         # misaligned workspace
    (dict(lengths=18), -2),                   # misaligned lengths
    (dict(ws_bytes=1000), -3),                # workspace too small
    (dict(skn=-128), -2),
    (dict(skn=1 << 21), -2),                  # one head's cache rows span 2^31 bytes or more
    (dict(B=1 << 22, ws_bytes=1 << 40), -2),  # more than 2^32 work-items in one dispatch
])
def test_decode_argument_errors(kw, code):
    lib = bsfa.load_library()
    assert _decode_call(lib, **kw) == code
    assert lib.bsfa_last_error() != b""


def test_decode_empty_batch_is_a_no_op():
    lib = bsfa.load_library()
    assert _decode_call(lib, B=0, q=None, out=None) == 0
    assert lib.bsfa_last_error() == b""


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built HIP library every entry point raises: there is no CPU path."""
    import torch

    monkeypatch.setattr(binding, "_LIB", None)
    monkeypatch.setattr(binding, "library_path", lambda: str(tmp_path / "libbsfa.so"))
    x = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16)
    with pytest.raises(binding.BsfaError, match="missing"):
        bsfa.fwd(x, x, x, mask=bsfa.MaskSpec(causal=True))
    with pytest.raises(binding.BsfaError, match="missing"):
        bsfa.decode(x[:, :, 0], x, x, torch.tensor([64]), mask=bsfa.MaskSpec(causal=True))
    with pytest.raises(binding.BsfaError, match="missing"):
        binding.build_block_lists(bsfa.MaskSpec(causal=True), 64)


def test_binding_rejects_host_tensors_before_any_launch():
    """Tensors that are not on the GPU never reach the library: their pointers would be
    invalid device addresses."""
    import torch

    x = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16)
    with pytest.raises(binding.BsfaError, match="is on cpu"):
        bsfa.fwd(x, x, x, mask=bsfa.MaskSpec(causal=True))
    with pytest.raises(binding.BsfaError, match="is on cpu"):
        bsfa.decode(x[:, :, 0], x, x, torch.tensor([64], dtype=torch.int32),
                    mask=bsfa.MaskSpec(causal=True))
    with pytest.raises(binding.BsfaError, match="on the GPU"):
        binding.skip_stats(torch.zeros((1, 1, 2), dtype=torch.int64))


def test_buffer_checks():
    import torch

    t = torch.zeros((2, 3, 5), dtype=torch.float32)
    binding._buffer("lse_out", t, (2, 3, 5), (torch.float32,))
    with pytest.raises(binding.BsfaError, match="shape"):
        binding._buffer("lse_out", t, (2, 3, 6), (torch.float32,))
    with pytest.raises(binding.BsfaError, match="dtype"):
        binding._buffer("lse_out", t, (2, 3, 5), (torch.int64,))
    with pytest.raises(binding.BsfaError, match="contiguous"):
        binding._buffer("lse_out", t.transpose(0, 2).contiguous().transpose(0, 2),
                        (2, 3, 5), (torch.float32,))


def test_block_list_cache_is_bounded(monkeypatch):
    """BlockLists.get keeps the most recently used lists only."""
    calls = []

    class Fake(binding.BlockLists):
        _cache = __import__("collections").OrderedDict()
        CACHE_SIZE = 3

        def __init__(self, mask, n, device):
            calls.append(n)

    spec = bsfa.MaskSpec(causal=True)
    for n in (64, 128, 192, 64, 256, 128):
        Fake.get(spec, n, "cuda:0")
    # 64 was reused before 256 evicted the oldest (128), so 128 is built again
    assert calls == [64, 128, 192, 256, 128]
    assert list(k[1] for k in Fake._cache) == [64, 256, 128]


def _calib_call(lib, **kw):
    args = dict(tm=16, keep=16, B=2, Hq=4, n=100, q=0.5, tau=16, ws=16, ws_bytes=1 << 20)
    args.update(kw)
    return lib.bsfa_calibrate_tau(args["tm"], args["keep"], args["B"], args["Hq"], args["n"],
                                  args["q"], args["tau"], args["ws"], args["ws_bytes"], None)


def test_calibrate_workspace_size():
    lib = bsfa.load_library()
    nb = ctypes.c_int64(0)
    assert lib.bsfa_calibrate_workspace_size(8, ctypes.byref(nb)) == 0
    assert nb.value >= 8 * 256 * 4
    assert lib.bsfa_calibrate_workspace_size(0, ctypes.byref(nb)) == -1
    assert lib.bsfa_calibrate_workspace_size(8, None) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), -1),
    (dict(Hq=0), -1),
    (dict(n=-5), -1),
    (dict(q=-0.1), -1),
    (dict(q=1.5), -1),
    (dict(q=float("nan")), -1),
    (dict(tau=None), -1),
    (dict(ws=None), -1),
    (dict(tm=None), -1),
    (dict(keep=None), -1),
    (dict(ws_bytes=100), -3),                 # workspace too small
    (dict(ws=8), -2),                         # misaligned workspace
    (dict(tm=18), -2),                        # misaligned maxima
    (dict(B=1 << 16, n=1 << 16), -2),         # 2^32 blocks per head
])
def test_calibrate_argument_errors(kw, code):
    lib = bsfa.load_library()
    assert _calib_call(lib, **kw) == code
    assert lib.bsfa_last_error() != b""


def _decode_static_call(lib, **kw):
    args = dict(q=16, k=16, v=16, lengths=16, out=16, lse=None, B=2, Hq=8, Hkv=2, L=1024,
                d=128, mask=binding._CMask(1, 0, 0, 1, 1), tau=None, scale=0.0, out_dtype=0,
                stats=None, tile_max=None, keep=None)
    args.update(kw)
    sq = binding._CStrides(args["Hq"] * args["d"], args["d"], 0)
    sk = binding._CStrides(args["Hkv"] * args["L"] * args["d"], args["L"] * args["d"],
                           args["d"])
    return lib.bsfa_decode_static(
        args["q"], args["k"], args["v"], args["lengths"], args["out"], args["lse"], args["B"],
        args["Hq"], args["Hkv"], args["L"], args["d"], ctypes.byref(sq), ctypes.byref(sk),
        ctypes.byref(sk), ctypes.byref(sq),
        ctypes.byref(args["mask"]) if args["mask"] is not None else None, args["tau"],
        args["scale"], args["out_dtype"], args["stats"], args["tile_max"], args["keep"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=7), -1),
    (dict(d=96), -2),
    (dict(lengths=None), -1),
    (dict(q=8), -2),                          # misaligned
    (dict(tile_max=16, keep=16), -1),         # export without tau
    # 2 * 64 * 512 splits * (128 + 4) * 4 bytes = 34.6 MB of partials > 32 MiB of scratch
    (dict(B=2, Hq=64, Hkv=8, L=131072), -3),
])
def test_decode_static_argument_errors(kw, code):
    """bsfa_decode_static validates like bsfa_decode, and rejects a step whose partials
    exceed its fixed scratch, before any HIP call."""
    lib = bsfa.load_library()
    assert _decode_static_call(lib, **kw) == code
    msg = lib.bsfa_last_error()
    assert msg != b""
    if code == -3:
        assert b"fixed scratch" in msg and str(32 << 20).encode() in msg
    # the largest step that fits: B * Hq * nsplit * (d + 4) * 4 <= 32 MiB
    assert bsfa.decode_workspace_size(2, 64, 122880, 128) <= 32 << 20


def test_decode_static_empty_batch_is_a_no_op():
    lib = bsfa.load_library()
    assert _decode_static_call(lib, B=0, q=None, out=None) == 0
