"""Block-sparse FlashAttention prefill and decode for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libbsfa.so`` (hand-written HIP kernels); the
Python layer only marshals arguments. Importing this package loads nothing: the binding
module is imported on first attribute access, and the library on the first call into
it, which raises if the library is missing.
"""
_BINDING_NAMES = {
    "MaskSpec", "BlockLists", "BsfaError", "build_block_lists", "fwd", "skip_stats",
    "library_path", "load_library", "calibrate_tau", "calibration_maxima",
    "decode", "decode_workspace_size", "decode_calibrate_tau", "decode_calibration_maxima",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
