"""Batch-invariant selected-token logprob on MI355X (gfx950).

The computation runs in the HIP library ``librlk.so`` built from ``csrc/``;
this package is a thin binding over its C ABI (torch supplies device memory
and streams).  The library is loaded on first use and a missing or unloadable
library raises: there is no CPU fallback.
"""
from ._binding import (  # noqa: F401
    LinearLogprob,
    RlkError,
    SelectedLogprob,
    build_info,
    library_path,
    linear_logp,
    linear_logp_backward,
    linear_logp_param_grads,
    linear_logp_param_grads_workspace_size,
    linear_logp_noalloc,
    linear_logp_with_logits,
    linear_logp_workspace_size,
    load_library,
    log_softmax,
    logp_backward,
    logp_entropy,
    logp_selected,
    token_losses,
)

__all__ = [
    "LinearLogprob", "RlkError", "SelectedLogprob", "build_info", "library_path", "linear_logp",
    "linear_logp_backward", "linear_logp_param_grads", "linear_logp_param_grads_workspace_size",
    "linear_logp_noalloc", "linear_logp_with_logits", "linear_logp_workspace_size", "load_library", "log_softmax", "logp_backward", "logp_entropy",
    "logp_selected", "token_losses",
]
