"""LM-head variant: logits = h W^T, then the fused loss, then the gradients of
h and W.  TEST INFRASTRUCTURE ONLY (see package docstring).
"""

import numpy as np

from .loss import loss_fwd_bwd


def lmhead_fwd_bwd(h, W, target, mask, old_logp, adv_tok, scale,
                   eps_low=0.2, eps_high=0.2, **terms):
    """Token-level GRPO loss through a linear LM head, plainly.

    ``h`` [n_tok, H] hidden states, ``W`` [V, H] LM-head weight (both read as
    float64).  z = h W^T is the logit matrix; the loss and dz = dL/dz follow
    ``loss_fwd_bwd``; then dh = dz W and dW = dz^T h (the chain rule through
    z = h W^T).  The gradient of a chunk is added to the gradients of earlier
    chunks by the caller ([P1] "The hard part: deferred normalization": the
    sum over chunks of the chunk gradients is the gradient of the step).
    Masked tokens ([P4] figure: pad rows are masked) contribute nothing.

    ``terms`` are passed to ``loss_fwd_bwd`` (row weights, entropy bonus, KL).

    Returns the ``loss_fwd_bwd`` dict plus ``dh`` [n_tok, H] and ``dW`` [V, H].
    """
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    z = h @ W.T
    out = loss_fwd_bwd(z, target, mask, old_logp, adv_tok, scale, eps_low, eps_high, want_dz=True, **terms)
    dz = out["dz"]
    out["dh"] = dz @ W
    out["dW"] = dz.T @ h
    return out
