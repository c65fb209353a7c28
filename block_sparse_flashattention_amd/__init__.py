"""Block-sparse FlashAttention prefill and decode for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libbsfa.so`` (hand-written HIP kernels); the
Python layer only marshals arguments. Importing this package loads nothing: the binding
module is imported on first attribute access, and the library on the first call into
it, which raises if the library is missing.

Usage (bf16 CUDA tensors; q [B, Hq, N, d], k and v [B, Hkv, N, d], d = 64 or 128)::

    import block_sparse_flashattention_amd as bsfa
    mask = bsfa.MaskSpec(causal=True, window=0, n_global=0)
    # per-head thresholds: a quantile of the block maxima on calibration inputs
    tau = bsfa.calibrate_tau(q_cal, k_cal, mask, 0.5)
    res = bsfa.fwd(q, k, v, mask=mask, tau=tau, stats=True)  # tau=None: dense path
    res.out, res.lse, bsfa.skip_stats(res.stats)
    # one decode step: q [B, Hq, d] against caches [B, Hkv, Lmax, d], lengths int32 [B]
    dtau = bsfa.decode_calibrate_tau(q_cal1, k_cache_cal, lengths_cal, mask, 0.5)
    step = bsfa.decode(q1, k_cache, v_cache, lengths, mask=mask, tau=dtau)
    step.out, step.lse

Calls are asynchronous on the current stream (or ``stream=``). With every output buffer
passed in (``out=``, ``lse_out=``, ``stats_out=``, ``lists=``, ``workspace=``) they
allocate nothing and can be captured in a HIP graph. ``decode_static`` is the decode
step for callers that cannot provide a workspace either: the library's fixed device
scratch (32 MiB per GPU) holds the partials; calls that overlap on one GPU race.
"""
_BINDING_NAMES = {
    "MaskSpec", "BlockLists", "BsfaError", "build_block_lists", "fwd", "skip_stats",
    "library_path", "load_library", "calibrate_tau", "calibration_maxima",
    "decode", "decode_workspace_size", "decode_calibrate_tau", "decode_calibration_maxima",
    "gpu_quantiles", "calibrate_workspace_size", "decode_static",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
