"""Exact IO-aware attention for MI355X (gfx950).

The compute path is the C-ABI library ``libmiattn.so`` (hand-written HIP
kernels); this package is its thin Python binding plus the seeded synthetic
inputs and the work accounting used by the tests and the benchmark.
"""
from . import accounting, inputs  # noqa: F401

_BINDING_NAMES = ("attn_fwd", "attn_decode", "attn_decode_multi", "attn_bwd", "prepare_fwd",
                  "prepare_decode", "prepare_decode_multi", "prepare_bwd", "attn_decode_paged",
                  "prepare_decode_paged",
                  "attn_decode_multi_workspace_bytes", "attn_fwd_workspace_bytes", "attn_decode_workspace_bytes",
                  "attn_bwd_workspace_bytes",
                  "attn_status_str", "library", "MiattnError", "fixed_max_decisions", "attn_decode_noalloc")


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
