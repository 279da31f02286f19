"""Frozen pi_old across a window of optimizer steps: the ahead-pass gate,
the old-log-prob cache keyed by call order, and the one-shot determinism
probe.  TEST INFRASTRUCTURE ONLY (see package docstring).

[P1] "pi_old must be frozen across the window -- the ahead pass":
* with n_mini > 1 and pi_old recomputed from the current policy, every
  ratio is 1 and the clip never binds; the fix walks the whole (mini, micro)
  product once before training, records pi_old per chunk, and replays the
  records during training;
* the pass is needed when n_mini > 1 and the loss does not use the rollout's
  own log-probs, and the objective consumes old log-probs; n_mini = 1 skips it;
* records are keyed by call order: both walks visit the chunks in the same
  order, so chunk k of the training walk pairs with chunk k of the ahead walk;
* the determinism probe re-scores the first ahead chunk of a run and
  compares it with the record; it gates on the fraction of tokens whose
  log-prob moved past a per-token bound, under the tolerance the model
  declares, strict default 0.05 nats on any token; it runs once per run.

Readings: a token "moved past" the bound when |a - b| > bound or either value
is not finite; the difference and the comparison are taken in float32, the
precision of the recorded log-probs; a tolerance is (bound, largest allowed
moved fraction), the strict gate being (0.05, 0).  A replay whose token count
differs from the paired record means the two walks diverged: an error.
"""

import numpy as np

from .loss import logprob_fwd

PROBE_STRICT_BOUND = 0.05
PROBE_STRICT_FRACTION = 0.0


class CacheError(Exception):
    """Misuse of the cache; ``kind`` is EINVAL, ECAPACITY or ESTATE."""

    def __init__(self, kind, msg):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind


def needs_ahead_pass(n_mini, use_rollout_logprobs, consumes_old_logprobs):
    """The gate of the ahead pass (see the module docstring)."""
    return n_mini > 1 and not use_rollout_logprobs and bool(consumes_old_logprobs)


class OldLogprobCache:
    """Per-chunk pi_old records of one collected batch, keyed by call order.

    ``record`` runs the forward-only log-prob pass on a chunk and stores it
    as record k (k = calls recorded so far); ``replay`` hands out record k
    for the k-th training call.  ``capacity`` bounds the total stored tokens.
    """

    def __init__(self, n_calls, capacity):
        if n_calls < 1 or capacity < 0:
            raise CacheError("EINVAL", "n_calls >= 1 and capacity >= 0")
        self.n_calls = n_calls
        self.capacity = capacity
        self.reset()

    def reset(self):
        self.records = []
        self.used = 0
        self.replayed = 0

    def record(self, logits, target, mask):
        if self.replayed > 0:
            raise CacheError("ESTATE", "record after replay started: reset for the next batch")
        if len(self.records) >= self.n_calls:
            raise CacheError("ESTATE", "every call of the walk is recorded")
        n = len(target)
        if self.used + n > self.capacity:
            raise CacheError("ECAPACITY", "cache buffer too small")
        lp = logprob_fwd(logits, target, mask)["logp"].astype(np.float32)
        self.records.append(lp)
        self.used += n
        return len(self.records) - 1

    def rewind(self):
        """Start the next inner epoch's replay from call 0 ([P1] "What's not
        done", item 2: inner epochs reuse the frozen pi_old unchanged); only
        after a complete walk was recorded and replayed."""
        if not (len(self.records) == self.n_calls and self.replayed == self.n_calls):
            raise CacheError("ESTATE", "rewind needs a complete recorded and replayed walk")
        self.replayed = 0

    def replay(self, n_tok):
        k = self.replayed
        if k >= len(self.records):
            raise CacheError("ESTATE", "replay of a call that was not recorded")
        if len(self.records[k]) != n_tok:
            raise CacheError("EINVAL", "the training walk diverged from the ahead walk (token count)")
        self.replayed += 1
        return self.records[k]


def gather(src, idx):
    """dst[k] = src[idx[k]]: the per-token (or per-row) values of a chunk whose
    rows sit anywhere in the batch ([P1] "The core idea": the driver passes
    indices only and the chunk is resolved from them)."""
    return [src[i] for i in idx]


def chunk_token_sources(src_row_off, rows):
    """Batch token index of every token of a chunk made of ``rows`` (in
    order): row r's tokens src_row_off[r] .. src_row_off[r+1]-1, rows end to
    end."""
    out = []
    for r in rows:
        out.extend(range(src_row_off[r], src_row_off[r + 1]))
    return out


def probe_compare(recorded, rescored, mask, bound):
    """(n_valid, n_moved, max_abs) over the valid tokens: |a - b| in float32,
    moved when it exceeds ``bound`` (float32) or is not finite; max_abs is the
    largest difference (infinite if any is not finite)."""
    a = np.asarray(recorded, dtype=np.float32)
    b = np.asarray(rescored, dtype=np.float32)
    bnd = np.float32(bound)
    n_valid = n_moved = 0
    max_abs = 0.0
    for t in range(len(a)):
        if not mask[t]:
            continue
        n_valid += 1
        with np.errstate(invalid="ignore", over="ignore"):
            d = np.float32(abs(np.float32(a[t] - b[t])))
        if not (d <= bnd):
            n_moved += 1
        max_abs = max(max_abs, float(d) if np.isfinite(d) else float("inf"))
    return n_valid, n_moved, max_abs


class Probe:
    """The one-shot determinism screen of a run."""

    def __init__(self, bound=PROBE_STRICT_BOUND, max_fraction=PROBE_STRICT_FRACTION):
        if not (bound >= 0 and 0 <= max_fraction <= 1):
            raise CacheError("EINVAL", "bound >= 0 and 0 <= max_fraction <= 1")
        self.bound = bound
        self.max_fraction = max_fraction
        self.done = False
        self.passed = None

    def due(self):
        return not self.done

    def finish(self, n_valid, n_moved):
        if self.done:
            raise CacheError("ESTATE", "the probe runs once per run")
        self.done = True
        self.passed = n_moved <= self.max_fraction * n_valid
        return self.passed
