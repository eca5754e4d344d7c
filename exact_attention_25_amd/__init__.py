"""Exact attention (FlashAttention forward and recompute backward) for MI355X.

The compute lives in ``libfa.so`` (hand-written HIP for gfx950 behind a C
ABI, declared in ``include/fa.h``).  ``binding`` marshals torch tensors into
that ABI.  The binding is imported lazily so that ``inputs`` and
``workloads`` can be used without the library; any use of the compute entry
points loads ``libfa.so`` and raises if it is missing -- there is no
fallback implementation.
"""

_BINDING_NAMES = ("fwd", "bwd", "fwd_splitkv", "fwd_masked", "bwd_masked", "mask_tiles", "fwd_dropout",
                  "bwd_dropout", "dropout_mask", "fa_fwd", "fa_bwd", "fa_fwd_ex", "fa_bwd_ex", "fa_bwd_noalloc",
                  "fa_dropout_mask", "fa_mask_tiles", "fa_mask_tiles_bytes", "options", "FaOptions",
                  "bwd_workspace_bytes", "fwd_ex_workspace_bytes", "bwd_ex_workspace_bytes", "splitkv_num_splits",
                  "fwd_kernel_name", "status_str", "load_library", "FaError", "library_path")


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    if name == "attention":  # differentiable attention over fwd / bwd
        from .autograd import attention
        return attention
    raise AttributeError(name)
