"""fp64 CPU oracle (test infrastructure only; see logprob_oracle)."""
from .logprob_oracle import (  # noqa: F401
    LN2,
    bf16_to_f64,
    entropy,
    entropy_from_f64,
    log_softmax,
    log_softmax_from_f64,
    linear_logits,
    linear_logp,
    linear_logp_backward,
    logp_backward,
    logp_backward_from_f64,
    logp_selected,
    logsumexp_rows,
    selected_logp_from_f64,
    token_losses,
)
