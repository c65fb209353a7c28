"""Thin Python binding over libbsfa.so (argument marshalling only).

Names follow the C ABI in include/bsfa.h: ``build_block_lists``, ``fwd``,
``skip_stats``. PyTorch supplies device memory and the current stream; every step of the
computation runs in the library's HIP kernels. There is no fallback: if the library is
missing or a call fails, a ``BsfaError`` is raised.
"""
from __future__ import annotations

import collections
import ctypes
import math
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

BSFA_CLS_PARTIAL = 1
BSFA_CLS_FORCED = 2
OUT_BF16, OUT_F32 = 0, 1


class BsfaError(RuntimeError):
    """A libbsfa call returned a non-zero status (message from bsfa_last_error)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"libbsfa status {status}: {message}")
        self.status = status


class _CMask(ctypes.Structure):
    _fields_ = [("causal", ctypes.c_int32), ("window", ctypes.c_int32),
                ("n_global", ctypes.c_int32), ("force_keep_diag", ctypes.c_int32),
                ("force_keep_global", ctypes.c_int32), ("dilation", ctypes.c_int32),
                ("dilation_taps", ctypes.c_int32), ("block", ctypes.c_int32),
                ("random_ppm", ctypes.c_int32), ("random_seed", ctypes.c_int32)]


class _CStrides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("n", ctypes.c_int64)]


class _CLists(ctypes.Structure):
    _fields_ = [("n_qtiles", ctypes.c_int32), ("block_q", ctypes.c_int32),
                ("block_k", ctypes.c_int32), ("nnz", ctypes.c_int64),
                ("row_ptr", ctypes.c_void_p), ("col", ctypes.c_void_p),
                ("cls", ctypes.c_void_p)]


EXPORTED = ("bsfa_build_block_lists", "bsfa_fwd", "bsfa_skip_stats", "bsfa_last_error",
            "bsfa_abi_version", "bsfa_decode", "bsfa_decode_static")


def library_path() -> str:
    return os.path.join(_HERE, "libbsfa.so")


def load_library():
    """Load libbsfa.so (once). Raises BsfaError if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise BsfaError(-4, f"{path} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.bsfa_build_block_lists.argtypes = [
        P(_CMask), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, P(ctypes.c_int64)]
    lib.bsfa_build_block_lists.restype = ctypes.c_int
    lib.bsfa_fwd.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        P(_CStrides), P(_CStrides), P(_CStrides), P(_CStrides), P(_CMask), P(_CLists),
        ctypes.c_void_p, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p]
    lib.bsfa_fwd.restype = ctypes.c_int
    lib.bsfa_decode_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32, P(ctypes.c_int64)]
    lib.bsfa_decode_workspace_size.restype = ctypes.c_int
    lib.bsfa_decode.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, P(_CStrides), P(_CStrides), P(_CStrides), P(_CStrides), P(_CMask),
        ctypes.c_void_p, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.bsfa_decode.restype = ctypes.c_int
    lib.bsfa_decode_static.argtypes = lib.bsfa_decode.argtypes[:-3] + [ctypes.c_void_p]
    lib.bsfa_decode_static.restype = ctypes.c_int
    lib.bsfa_calibrate_workspace_size.argtypes = [ctypes.c_int32, P(ctypes.c_int64)]
    lib.bsfa_calibrate_workspace_size.restype = ctypes.c_int
    lib.bsfa_calibrate_tau.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
        ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.bsfa_calibrate_tau.restype = ctypes.c_int
    lib.bsfa_skip_stats.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.bsfa_skip_stats.restype = ctypes.c_int
    lib.bsfa_last_error.argtypes = []
    lib.bsfa_last_error.restype = ctypes.c_char_p
    lib.bsfa_abi_version.argtypes = []
    lib.bsfa_abi_version.restype = ctypes.c_int32
    _LIB = lib
    return lib


def _check(lib, status: int):
    if status != 0:
        raise BsfaError(status, lib.bsfa_last_error().decode(errors="replace"))


@dataclass(frozen=True)
class MaskSpec:
    """Static pattern: causal AND the OR of the set primitives (window, dilated,
    blockwise, random blocks, global tokens); see include/bsfa.h."""

    causal: bool = True
    window: int = 0
    n_global: int = 0
    force_keep_diag: bool = True
    force_keep_global: bool = True
    dilation: int = 0
    dilation_taps: int = 0
    block: int = 0
    random_ppm: int = 0
    random_seed: int = 0

    def _c(self) -> _CMask:
        return _CMask(int(self.causal), int(self.window), int(self.n_global),
                      int(self.force_keep_diag), int(self.force_keep_global),
                      int(self.dilation), int(self.dilation_taps), int(self.block),
                      int(self.random_ppm), int(self.random_seed))


def build_block_lists(mask: MaskSpec, n: int, block_q: int = 64, block_k: int = 64):
    """Host CSR of allowed tiles: (row_ptr int32 [nqt+1], col int32 [nnz], cls uint8 [nnz])."""
    lib = load_library()
    cm = mask._c()
    nnz = ctypes.c_int64(0)
    nqt = (n + block_q - 1) // block_q
    row_ptr = np.zeros(nqt + 1, dtype=np.int32)
    _check(lib, lib.bsfa_build_block_lists(ctypes.byref(cm), n, block_q, block_k,
                                           row_ptr.ctypes.data, None, None, 0,
                                           ctypes.byref(nnz)))
    col = np.zeros(max(nnz.value, 1), dtype=np.int32)
    cls = np.zeros(max(nnz.value, 1), dtype=np.uint8)
    _check(lib, lib.bsfa_build_block_lists(ctypes.byref(cm), n, block_q, block_k,
                                           row_ptr.ctypes.data, col.ctypes.data,
                                           cls.ctypes.data, col.size, ctypes.byref(nnz)))
    return row_ptr, col[: nnz.value], cls[: nnz.value]


class BlockLists:
    """Device copy of the 64x64 block lists for one (mask, N)."""

    # the most recently used lists, by (mask, N, device); older ones are dropped
    _cache: "collections.OrderedDict" = collections.OrderedDict()
    CACHE_SIZE = 16

    def __init__(self, mask: MaskSpec, n: int, device):
        import torch

        row_ptr, col, cls = build_block_lists(mask, n, 64, 64)
        self.mask, self.n = mask, n
        self.n_qtiles = row_ptr.size - 1
        self.nnz = int(col.size)
        self.row_ptr_host, self.col_host, self.cls_host = row_ptr, col, cls
        self.row_ptr = torch.from_numpy(row_ptr).to(device)
        self.col = torch.from_numpy(col if col.size else np.zeros(1, np.int32)).to(device)
        self.cls = torch.from_numpy(cls if cls.size else np.zeros(1, np.uint8)).to(device)

    @classmethod
    def get(cls, mask: MaskSpec, n: int, device) -> "BlockLists":
        key = (mask, n, str(device))
        if key in cls._cache:
            cls._cache.move_to_end(key)
        else:
            cls._cache[key] = cls(mask, n, device)
            while len(cls._cache) > cls.CACHE_SIZE:
                cls._cache.popitem(last=False)
        return cls._cache[key]

    def _c(self) -> _CLists:
        return _CLists(self.n_qtiles, 64, 64, self.nnz, self.row_ptr.data_ptr(),
                       self.col.data_ptr(), self.cls.data_ptr())


@dataclass
class FwdResult:
    out: object
    lse: object
    stats: object = None  # uint64 view as int64 tensor [B, Hq, 2] {kept, skipped}
    tile_max: object = None  # fp32 [B, Hq, nnz]
    keep: object = None  # uint8 [B, Hq, nnz]
    lists: BlockLists = None


def _on_device(dev, **tensors):
    """Every tensor the kernels touch must live on the GPU that runs them: a host or
    foreign-device pointer would reach the kernel as an invalid address."""
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device != dev):
            raise BsfaError(-1, f"{name} is on {t.device}, the call runs on {dev}")


def _buffer(name, t, shape, dtypes, contiguous=True):
    """A caller-provided output buffer: exact shape, dtype, and (if the kernel indexes it
    densely) contiguous."""
    if tuple(t.shape) != tuple(shape):
        raise BsfaError(-1, f"{name} has shape {tuple(t.shape)}, need {tuple(shape)}")
    if t.dtype not in dtypes:
        raise BsfaError(-2, f"{name} has dtype {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise BsfaError(-2, f"{name} must be contiguous")


def _stream_scope(stream, dev):
    """(context, handle) for a call that launches on ``stream``.

    With no stream the call runs on torch's current stream. With a caller stream (a
    hipStream_t handle) every temporary the call allocates (counters, a tau copy, the
    decode or calibration workspace, outputs not passed in) is allocated and filled with
    that stream current: its zero-fill or copy is queued before the kernel on the same
    stream, and the caching allocator hands the memory out again only to that stream, so
    it cannot be reused while the launch is pending. Inputs the caller passes in must be
    ready on that stream (the caller orders them, as for any stream argument)."""
    import contextlib

    import torch

    if stream is None:
        return contextlib.nullcontext(), torch.cuda.current_stream(dev).cuda_stream
    handle = int(stream)
    default = torch.cuda.default_stream(dev)
    ext = default if handle == default.cuda_stream else torch.cuda.ExternalStream(
        handle, device=dev)
    return torch.cuda.stream(ext), handle


def _strides(t) -> _CStrides:
    s = t.stride()
    if s[3] != 1:
        raise BsfaError(-2, "the head dimension must be contiguous")
    return _CStrides(s[0], s[1], s[2])


def fwd(q, k, v, mask: MaskSpec = MaskSpec(), tau=None, softmax_scale: float = 0.0,
        out_dtype=None, out=None, want_lse: bool = True, stats: bool = False,
        export_tiles: bool = False, lists: BlockLists | None = None, stream=None,
        lse_out=None, stats_out=None) -> FwdResult:
    """Block-sparse attention forward on the GPU, asynchronous on ``stream`` (a
    hipStream_t handle; default torch's current stream).

    q: bf16 [B, Hq, N, d]; k, v: bf16 [B, Hkv, N, d] (CUDA/HIP tensors, last dim
    contiguous). tau: None (dense path) or fp32 tensor [Hq] on the device (or anything
    torch.as_tensor accepts). Returns out [B, Hq, N, d] (bf16 or fp32), lse fp32
    [B, Hq, N], optional per-(b, h) {kept, skipped} counts and per-tile export.
    ``lse_out`` / ``stats_out`` reuse caller buffers (stats are added to stats_out).
    """
    import torch

    lib = load_library()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise BsfaError(-1, "q, k, v must be 4-D [B, H, N, d]")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise BsfaError(-2, "q, k, v must be bfloat16")
    bsz, hq, n, d = q.shape
    hkv = k.shape[1]
    if tuple(k.shape) != (bsz, hkv, n, d) or tuple(v.shape) != (bsz, hkv, n, d):
        raise BsfaError(-1, f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    dev = q.device
    _on_device(dev, q=q, k=k, v=v, out=out, lse_out=lse_out, stats_out=stats_out)
    scope, stream = _stream_scope(stream, dev)
    with scope:
        if out_dtype is None:
            out_dtype = torch.bfloat16
        if out is None:
            out = torch.empty((bsz, hq, n, d), dtype=out_dtype, device=dev)
        _buffer("out", out, (bsz, hq, n, d), (torch.bfloat16, torch.float32), contiguous=False)
        if lse_out is not None:
            _buffer("lse_out", lse_out, (bsz, hq, n), (torch.float32,))
            lse = lse_out
        else:
            lse = torch.empty((bsz, hq, n), dtype=torch.float32, device=dev) if want_lse else None
        if stats_out is not None:
            _buffer("stats_out", stats_out, (bsz, hq, 2), (torch.int64,))
        if lists is None:
            lists = BlockLists.get(mask, n, dev)
        _on_device(dev, lists=lists.row_ptr)
        tau_t = None
        if tau is not None:
            tau_t = torch.as_tensor(tau, dtype=torch.float32, device=dev).reshape(-1)
            if tau_t.numel() == 1 and hq > 1:
                tau_t = tau_t.expand(hq).contiguous()
            if tau_t.numel() != hq:
                raise BsfaError(-1, f"tau needs {hq} values, got {tau_t.numel()}")
            tau_t = tau_t.contiguous()
        if stats_out is not None:
            st = stats_out
        else:
            st = torch.zeros((bsz, hq, 2), dtype=torch.int64, device=dev) if stats else None
        tm = kp = None
        if export_tiles:
            tm = torch.empty((bsz, hq, max(lists.nnz, 1)), dtype=torch.float32, device=dev)
            kp = torch.empty((bsz, hq, max(lists.nnz, 1)), dtype=torch.uint8, device=dev)
        cm = mask._c()
        cl = lists._c()
        sq, sk, sv, so = _strides(q), _strides(k), _strides(v), _strides(out)
        status = lib.bsfa_fwd(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            lse.data_ptr() if lse is not None else None, bsz, hq, hkv, n, d,
            ctypes.byref(sq), ctypes.byref(sk), ctypes.byref(sv), ctypes.byref(so),
            ctypes.byref(cm), ctypes.byref(cl),
            tau_t.data_ptr() if tau_t is not None else None, float(softmax_scale),
            OUT_F32 if out.dtype == torch.float32 else OUT_BF16,
            st.data_ptr() if st is not None else None,
            tm.data_ptr() if tm is not None else None,
            kp.data_ptr() if kp is not None else None, stream)
        _check(lib, status)
        if tm is not None and lists.nnz == 0:
            tm, kp = tm[..., :0], kp[..., :0]
        return FwdResult(out, lse, st, tm, kp, lists)


@dataclass
class DecodeResult:
    out: object  # [B, Hq, d]
    lse: object  # fp32 [B, Hq]
    stats: object = None  # int64 [B, Hq, 2] {kept, skipped} allowed blocks
    tile_max: object = None  # fp32 [B, Hq, nkb]
    keep: object = None  # uint8 [B, Hq, nkb]


def decode_workspace_size(batch: int, hq: int, max_len: int, d: int) -> int:
    """Bytes of scratch ``decode`` needs (bsfa_decode_workspace_size)."""
    lib = load_library()
    nbytes = ctypes.c_int64(0)
    _check(lib, lib.bsfa_decode_workspace_size(batch, hq, max_len, d, ctypes.byref(nbytes)))
    return int(nbytes.value)


def decode(q, k_cache, v_cache, lengths, mask: MaskSpec = MaskSpec(), tau=None,
           softmax_scale: float = 0.0, out_dtype=None, out=None, want_lse: bool = True,
           stats: bool = False, export_tiles: bool = False, workspace=None, stream=None,
           lse_out=None, stats_out=None) -> DecodeResult:
    """One block-sparse decode step on the GPU (bsfa_decode), asynchronous on ``stream``
    (a hipStream_t handle; default torch's current stream).

    q: bf16 [B, Hq, d], the newest token's query per sequence and head; k_cache, v_cache:
    bf16 [B, Hkv, Lmax, d] (last dim contiguous); lengths: int32 [B] on the device, the
    valid cache rows of each sequence (the new token is row lengths[b] - 1). tau: None
    (dense path) or fp32 [Hq]. ``workspace`` is an optional caller buffer of at least
    decode_workspace_size bytes (a uint8 tensor); one is allocated here otherwise.
    """
    return _decode(q, k_cache, v_cache, lengths, mask, tau, softmax_scale, out_dtype, out,
                   want_lse, stats, export_tiles, workspace, stream, lse_out, stats_out,
                   fixed_scratch=False)


def decode_static(q, k_cache, v_cache, lengths, mask: MaskSpec = MaskSpec(), tau=None,
                  softmax_scale: float = 0.0, out_dtype=None, out=None, want_lse: bool = True,
                  stats: bool = False, export_tiles: bool = False, stream=None,
                  lse_out=None, stats_out=None) -> DecodeResult:
    """The decode step through bsfa_decode_static: the library's fixed device scratch
    holds the per-split partials, so the library allocates nothing. Arguments as
    ``decode`` without ``workspace``. Outputs that are not passed in (out, lse_out,
    stats_out) and a tau that is not already an fp32 device tensor are still allocated
    here by torch; a caller that may not allocate passes them all in."""
    return _decode(q, k_cache, v_cache, lengths, mask, tau, softmax_scale, out_dtype, out,
                   want_lse, stats, export_tiles, None, stream, lse_out, stats_out,
                   fixed_scratch=True)


def _decode(q, k_cache, v_cache, lengths, mask, tau, softmax_scale, out_dtype, out,
            want_lse, stats, export_tiles, workspace, stream, lse_out, stats_out,
            fixed_scratch: bool) -> DecodeResult:
    import torch

    lib = load_library()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.dim() != 4:
        raise BsfaError(-1, "q must be [B, Hq, d] and the caches [B, Hkv, Lmax, d]")
    if (q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16
            or v_cache.dtype != torch.bfloat16):
        raise BsfaError(-2, "q, k_cache, v_cache must be bfloat16")
    bsz, hq, d = q.shape
    hkv, lmax = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (bsz, hkv, lmax, d) or tuple(v_cache.shape) != (bsz, hkv, lmax, d):
        raise BsfaError(-1, f"shape mismatch q{tuple(q.shape)} k{tuple(k_cache.shape)} "
                            f"v{tuple(v_cache.shape)}")
    if lengths.dtype != torch.int32 or lengths.numel() != bsz or not lengths.is_contiguous():
        raise BsfaError(-1, "lengths must be a contiguous int32 tensor of B values")
    if q.stride(2) != 1:
        raise BsfaError(-2, "the head dimension of q must be contiguous")
    dev = q.device
    _on_device(dev, q=q, k_cache=k_cache, v_cache=v_cache, lengths=lengths, out=out,
               lse_out=lse_out, stats_out=stats_out, workspace=workspace)
    scope, stream = _stream_scope(stream, dev)
    with scope:
        if out_dtype is None:
            out_dtype = torch.bfloat16
        if out is None:
            out = torch.empty((bsz, hq, d), dtype=out_dtype, device=dev)
        _buffer("out", out, (bsz, hq, d), (torch.bfloat16, torch.float32), contiguous=False)
        if out.stride(2) != 1:
            raise BsfaError(-2, "the head dimension of out must be contiguous")
        if lse_out is not None:
            _buffer("lse_out", lse_out, (bsz, hq), (torch.float32,))
            lse = lse_out
        else:
            lse = torch.empty((bsz, hq), dtype=torch.float32, device=dev) if want_lse else None
        if stats_out is not None:
            _buffer("stats_out", stats_out, (bsz, hq, 2), (torch.int64,))
        tau_t = None
        if tau is not None:
            tau_t = torch.as_tensor(tau, dtype=torch.float32, device=dev).reshape(-1)
            if tau_t.numel() == 1 and hq > 1:
                tau_t = tau_t.expand(hq).contiguous()
            if tau_t.numel() != hq:
                raise BsfaError(-1, f"tau needs {hq} values, got {tau_t.numel()}")
            tau_t = tau_t.contiguous()
        if stats_out is not None:
            st = stats_out
        else:
            st = torch.zeros((bsz, hq, 2), dtype=torch.int64, device=dev) if stats else None
        nkb = -(-lmax // 64)
        tm = kp = None
        if export_tiles:
            tm = torch.empty((bsz, hq, nkb), dtype=torch.float32, device=dev)
            kp = torch.empty((bsz, hq, nkb), dtype=torch.uint8, device=dev)
        if not fixed_scratch:
            need = decode_workspace_size(bsz, hq, lmax, d)
            if workspace is None:
                workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
            elif not workspace.is_contiguous():
                raise BsfaError(-2, "workspace must be contiguous")
        cm = mask._c()
        sq = _CStrides(q.stride(0), q.stride(1), 0)
        so = _CStrides(out.stride(0), out.stride(1), 0)
        sk, sv = _strides(k_cache), _strides(v_cache)
        args = [
            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), lengths.data_ptr(),
            out.data_ptr(), lse.data_ptr() if lse is not None else None, bsz, hq, hkv, lmax, d,
            ctypes.byref(sq), ctypes.byref(sk), ctypes.byref(sv), ctypes.byref(so),
            ctypes.byref(cm), tau_t.data_ptr() if tau_t is not None else None,
            float(softmax_scale), OUT_F32 if out.dtype == torch.float32 else OUT_BF16,
            st.data_ptr() if st is not None else None,
            tm.data_ptr() if tm is not None else None,
            kp.data_ptr() if kp is not None else None]
        if fixed_scratch:
            status = lib.bsfa_decode_static(*args, stream)
        else:
            status = lib.bsfa_decode(*args, workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(), stream)
        _check(lib, status)
        return DecodeResult(out, lse, st, tm, kp)


def decode_calibration_maxima(q, k_cache, lengths, mask: MaskSpec, softmax_scale: float = 0.0,
                              stream=None):
    """Eligible (allowed, not forced) decode block maxima per query head, from one
    gate-only decode pass: with tau = NaN only forced blocks are kept, so the exported
    keep bits mark exactly the forced blocks."""
    import torch

    hq = q.shape[1]
    scope, stream = _stream_scope(stream, q.device)
    with scope:
        res = decode(q, k_cache, k_cache, lengths, mask=mask,
                     tau=torch.full((hq,), math.nan, device=q.device),
                     softmax_scale=softmax_scale, want_lse=False, export_tiles=True,
                     stream=stream)
    torch.cuda.synchronize(q.device)
    tmax = res.tile_max.cpu().numpy()  # [B, Hq, nkb]
    keep = res.keep.cpu().numpy().astype(bool)  # forced blocks only (tau = NaN)
    allowed = tmax > -np.inf  # blocks with no allowed key export -inf
    return [tmax[:, h][allowed[:, h] & ~keep[:, h]].reshape(-1) for h in range(hq)]


def decode_calibrate_tau(q, k_cache, lengths, mask: MaskSpec, quantile,
                         softmax_scale: float = 0.0, stream=None):
    """Per-head decode thresholds: the ``quantile`` of the eligible decode block maxima
    of each query head on calibration inputs (as ``calibrate_tau`` for prefill). One
    gate-only decode pass exports the maxima; ``bsfa_calibrate_tau`` takes the quantile
    on the GPU."""
    import torch

    hq = q.shape[1]
    scope, stream = _stream_scope(stream, q.device)
    with scope:
        res = decode(q, k_cache, k_cache, lengths, mask=mask,
                     tau=torch.full((hq,), math.nan, device=q.device),
                     softmax_scale=softmax_scale, want_lse=False, export_tiles=True,
                     stream=stream)
        nkb = -(-k_cache.shape[2] // 64)
        return gpu_quantiles(res.tile_max, res.keep, q.shape[0], hq, nkb, quantile, stream)


def calibrate_workspace_size(hq: int) -> int:
    """Bytes of scratch ``gpu_quantiles`` needs (bsfa_calibrate_workspace_size)."""
    lib = load_library()
    nbytes = ctypes.c_int64(0)
    _check(lib, lib.bsfa_calibrate_workspace_size(hq, ctypes.byref(nbytes)))
    return int(nbytes.value)


def gpu_quantiles(tile_max, keep, bsz: int, hq: int, n_blocks: int, quantile, stream=None):
    """Per-head quantiles of the eligible exported block maxima, on the GPU
    (bsfa_calibrate_tau): tile_max fp32 and keep uint8, both [B, Hq, n_blocks] on the
    device. A scalar ``quantile`` returns fp32 [Hq]; a sequence returns fp32
    [len(quantile), Hq]. Heads with no eligible block get -inf."""
    import torch

    lib = load_library()
    dev = tile_max.device
    _on_device(dev, tile_max=tile_max, keep=keep)
    if n_blocks:
        _buffer("tile_max", tile_max, (bsz, hq, n_blocks), (torch.float32,))
        _buffer("keep", keep, (bsz, hq, n_blocks), (torch.uint8,))
    qs = np.atleast_1d(np.asarray(quantile, dtype=np.float64))
    scope, stream = _stream_scope(stream, dev)
    with scope:
        taus = torch.empty((qs.size, hq), dtype=torch.float32, device=dev)
        ws = torch.empty(calibrate_workspace_size(hq), dtype=torch.uint8, device=dev)
        for i, qv in enumerate(qs):
            _check(lib, lib.bsfa_calibrate_tau(tile_max.data_ptr(), keep.data_ptr(), bsz, hq,
                                               n_blocks, float(qv), taus[i].data_ptr(),
                                               ws.data_ptr(), ws.numel(), stream))
    torch.cuda.synchronize(dev)  # the launches may sit on a stream other than torch's
    out = taus.cpu().numpy()
    return out[0] if np.ndim(quantile) == 0 else out


def skip_stats(stats_tensor, stream=None):
    """{kept, skipped} tile counts per (b, h) as two uint64 numpy arrays [B, Hq]."""
    import torch

    lib = load_library()
    if not stats_tensor.is_cuda:
        raise BsfaError(-1, "stats_tensor must be on the GPU")
    bsz, hq, _ = stats_tensor.shape
    _buffer("stats_tensor", stats_tensor, (bsz, hq, 2), (torch.int64,))
    kept = np.zeros((bsz, hq), dtype=np.uint64)
    skipped = np.zeros((bsz, hq), dtype=np.uint64)
    if stream is None:
        stream = torch.cuda.current_stream(stats_tensor.device).cuda_stream
    _check(lib, lib.bsfa_skip_stats(stats_tensor.data_ptr(), bsz, hq, kept.ctypes.data,
                                    skipped.ctypes.data, stream))
    return kept, skipped


def calibration_maxima(q, k, mask: MaskSpec, softmax_scale: float = 0.0, lists=None,
                       stream=None):
    """Block maxima of every eligible (allowed, not forced) tile, per query head.

    One gate-only pass of the kernel: tau = NaN keeps forced tiles only, so every other
    tile costs its S = scale * Q K^T, its block maximum and the export, with no softmax,
    P.V or V load. Returns a list of Hq fp32 arrays, each [B * eligible tiles] (the
    per-head histogram input of the calibration in Block Sparse Flash Attention, "The
    paper's improvements")."""
    import torch

    hq = q.shape[1]
    scope, stream = _stream_scope(stream, q.device)
    with scope:
        res = fwd(q, k, k, mask=mask, tau=torch.full((hq,), math.nan, device=q.device),
                  softmax_scale=softmax_scale, want_lse=False, export_tiles=True, lists=lists,
                  stream=stream)
    torch.cuda.synchronize(q.device)  # the launch may sit on a stream other than torch's
    tmax = res.tile_max.cpu().numpy()  # [B, Hq, nnz]
    eligible = (res.lists.cls_host & BSFA_CLS_FORCED) == 0
    return [tmax[:, h, :][:, eligible].reshape(-1) for h in range(hq)]


def calibrate_tau(q, k, mask: MaskSpec, quantile, softmax_scale: float = 0.0, lists=None,
                  stream=None):
    """One-time per-head threshold calibration (Block Sparse Flash Attention, "The
    paper's improvements": thresholds learned once per layer and head on a small data set).

    tau_h = the ``quantile`` of the eligible block maxima of query head h on calibration
    inputs q, k, with numpy's linear interpolation. One gate-only pass of the kernel
    exports the maxima and ``bsfa_calibrate_tau`` takes the quantile on the GPU; nothing
    is copied to the host but the result. ``quantile`` may be a scalar (returns fp32
    [Hq]) or a sequence (returns fp32 [len(quantile), Hq])."""
    import torch

    hq = q.shape[1]
    scope, stream = _stream_scope(stream, q.device)
    with scope:
        res = fwd(q, k, k, mask=mask, tau=torch.full((hq,), math.nan, device=q.device),
                  softmax_scale=softmax_scale, want_lse=False, export_tiles=True, lists=lists,
                  stream=stream)
        return gpu_quantiles(res.tile_max, res.keep, q.shape[0], hq, res.lists.nnz,
                             quantile, stream)