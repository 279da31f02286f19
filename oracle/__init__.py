"""CPU oracle for the token-level GRPO loss path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the package
``grpo_token_level_amd``, its C-ABI library or its kernels) may import, call
or link anything in this directory.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.

The oracle is plain, slow and written to be checked by eye against the pages
it follows.  Floating point is float64 throughout (logits are read as their
exact bf16 / fp32 values); plans and indices are Python integers.  It shares
no code, table or constant with the HIP path.

Sources (cited by title and section in every function):

* [P1] "Sizing mini-batches and micro-batches" -- the cosmos-framework
  post-training how-to on batching.
* [P2] "03 Data Protocol and Batch Lifecycle" -- verl source reading, field
  lifecycle of one GRPO update.
* [P3] "22 - mini-batch, micro-batch and dynamic batch size" -- verl article on
  the three batch levels, loss normalisation and the aggregation modes.
* [P4] "How a context-compaction step fits a variable number of rows into one
  batch" -- NeMo-RL context-compaction explainer.

Where the pages leave a step open, the reading taken is stated in the
function's docstring (and listed with the rest of the design notes).

Parity status: every public function here is pinned by ``tests/test_oracle_*``
against worked examples, closed forms, brute force or finite differences,
except the balance quality of ``plan_dynamic`` (its feasibility and
determinism are pinned; that its greedy order is the "right" partition is
parity unpinned, because the pages name no algorithm).
"""

from .plans import (PlanError, plan_fixed, chunk_rows, train_calls,
                    plan_dynamic, plan_compaction, compaction_micro_chunks,
                    splitmix64_stream, fisher_yates, plan_epochs, epoch_chunk_rows,
                    epoch_train_calls)
from .advantage import group_advantage, rows_advantage
from .loss import (round_to_bf16, token_forward, surrogate, loss_fwd_bwd,
                   logprob_fwd, chunk_stats, row_stats, valid_count, kl_term,
                   KL_K1, KL_K2, KL_K3, STAT_KEYS)
from .agg import (AGG_TOKEN_MEAN, AGG_SEQ_MEAN_TOKEN_SUM, AGG_SEQ_MEAN_TOKEN_MEAN,
                  row_valid_counts, count_rows, agg_loss, row_weights)
from .accum import Accumulator, ACC_OK, ACC_NONFINITE, ACC_SKIPPED
from .lmhead import lmhead_fwd_bwd
from .cache import (CacheError, needs_ahead_pass, OldLogprobCache, probe_compare, Probe,
                    PROBE_STRICT_BOUND, PROBE_STRICT_FRACTION, gather, chunk_token_sources)

__all__ = [
    "PlanError", "plan_fixed", "chunk_rows", "train_calls", "plan_dynamic",
    "plan_compaction", "compaction_micro_chunks", "group_advantage",
    "rows_advantage", "round_to_bf16", "token_forward", "surrogate",
    "loss_fwd_bwd", "logprob_fwd", "chunk_stats", "row_stats", "valid_count",
    "Accumulator", "ACC_OK", "ACC_NONFINITE", "ACC_SKIPPED", "lmhead_fwd_bwd",
    "kl_term", "KL_K1", "KL_K2", "KL_K3", "STAT_KEYS", "AGG_TOKEN_MEAN",
    "AGG_SEQ_MEAN_TOKEN_SUM", "AGG_SEQ_MEAN_TOKEN_MEAN", "row_valid_counts",
    "count_rows", "agg_loss", "row_weights", "CacheError", "needs_ahead_pass",
    "OldLogprobCache", "probe_compare", "Probe", "PROBE_STRICT_BOUND", "PROBE_STRICT_FRACTION",
    "splitmix64_stream", "fisher_yates", "plan_epochs", "epoch_chunk_rows", "epoch_train_calls",
    "gather", "chunk_token_sources",
]
