"""Step accumulator: token-weighted roll-up, deferred divisor and the
poisoned-window countdown.  TEST INFRASTRUCTURE ONLY (see package docstring).
"""

import math

ACC_OK = "OK"
ACC_NONFINITE = "NONFINITE"
ACC_SKIPPED = "SKIPPED"
ACC_STATE = "STATE"      # a completed window was not finalized before the next add

_KEYS = ("loss_sum", "entropy_sum", "kl_sum", "obj_sum", "n_valid", "n_clipped", "n_valid_rows")
_FLOAT_KEYS = ("loss_sum", "entropy_sum", "kl_sum", "obj_sum")


class Accumulator:
    """One optimizer-step window of ``n_micro`` chunk calls.

    [P1] "The hard part: deferred normalization": chunk divisors add up and
    the gradient is scaled once, by 1/max(sum of divisors, 1), at the step.
    [P1] "Metric roll-up: token-weighted, not averaged": the step loss is
    sum(loss_i * denom_i) / sum(denom_i) = sum(loss_sum_i) / sum(denom_i);
    counts sum.
    [P1] "The poisoned-window countdown": a non-finite chunk at position j of
    the window discards the window (sums reset) and the next n_micro - 1 - j
    calls are swallowed before a fresh window starts.  [P1] invariant 4: the
    whole mini-batch is abandoned, not only the chunk.

    Reading: a chunk is non-finite when any valid token was (n_nonfinite > 0)
    or one of its loss, entropy, KL or objective sums is not finite.  With an
    empty step (sum of divisors 0) the loss is 0 and the gradient scale is 1.
    Stats dicts without ``kl_sum`` / ``obj_sum`` count them as 0.
    """

    def __init__(self, n_micro):
        if n_micro < 1:
            raise ValueError("n_micro must be >= 1")
        self.n_micro = n_micro
        self.pos = 0
        self.skip = 0
        self.sums = {k: 0 for k in _KEYS}
        self.done = None

    def add(self, stats):
        if self.done is not None:
            return ACC_STATE
        if self.skip > 0:
            self.skip -= 1
            return ACC_SKIPPED
        bad = stats["n_nonfinite"] > 0 or not all(math.isfinite(stats.get(k, 0.0)) for k in _FLOAT_KEYS)
        if bad:
            self.skip = self.n_micro - 1 - self.pos
            self.pos = 0
            self.sums = {k: 0 for k in _KEYS}
            return ACC_NONFINITE
        for k in _KEYS:
            self.sums[k] += stats.get(k, 0)
        self.pos += 1
        if self.pos == self.n_micro:
            self.done = dict(self.sums)
            self.pos = 0
            self.sums = {k: 0 for k in _KEYS}
        return ACC_OK

    def finalize(self):
        """Close a completed window.  Returns ``None`` when no window is complete,
        else a dict with the step loss, counts, mean entropy and KL per valid
        token, the gradient scale 1/max(N, 1) and ``obj_sum``, the window's sum
        of the chunks' objective shares (the step objective itself when the
        chunks carried the normalisation; times grad_scale in the deferred
        token-mean mode)."""
        if self.done is None:
            return None
        d = self.done
        self.done = None
        denom = max(d["n_valid"], 1)
        return {"loss": d["loss_sum"] / denom, "n_valid": d["n_valid"],
                "n_valid_rows": d["n_valid_rows"], "n_clipped": d["n_clipped"],
                "entropy": d["entropy_sum"] / denom, "kl": d["kl_sum"] / denom,
                "obj_sum": d["obj_sum"], "grad_scale": 1.0 / denom}
