"""Group-relative advantages.  TEST INFRASTRUCTURE ONLY (see package docstring)."""

import math

import numpy as np


def group_advantage(rewards, group_size, eps=1e-6, norm_by_std=True):
    """One advantage per rollout, relative to its group of ``group_size``.

    [P2] "Field Lineage" (reward, log-prob and advantage): the trainer turns
    trajectory-level rewards into advantages once, over the padded batch.
    [P4] "Why the row count does not change the math", item 2: the advantage
    is computed once per rollout.

    The pages give no formula.  Reading taken: for each group of G consecutive
    rollouts, A = (r - mean) / (std + eps) with the unbiased (G-1) standard
    deviation; ``norm_by_std=False`` gives A = r - mean; a group of one rollout
    has A = 0.  Sums run in index order in float64.
    """
    r = [float(x) for x in rewards]
    n = len(r)
    if group_size <= 0 or n % group_size != 0:
        raise ValueError("rewards must hold a whole number of groups")
    out = np.zeros(n, dtype=np.float64)
    G = group_size
    for g in range(n // G):
        seg = r[g * G:(g + 1) * G]
        if G == 1:
            out[g * G] = 0.0
            continue
        total = 0.0
        for x in seg:
            total += x
        mean = total / G
        sq = 0.0
        for x in seg:
            sq += (x - mean) * (x - mean)
        std = math.sqrt(sq / (G - 1))
        for k, x in enumerate(seg):
            out[g * G + k] = (x - mean) / (std + eps) if norm_by_std else (x - mean)
    return out


def rows_advantage(adv_rollout, row_rollout):
    """Copy each rollout's advantage to every one of its rows; pads get 0.

    [P4] "Why the row count does not change the math", item 2, and the figure's
    pad-row rule (reward 0, masked).  [P2] "Field Lineage": the scalar
    advantage is broadcast over the rollout's tokens.  A row whose rollout
    index is negative is a pad.
    """
    out = np.zeros(len(row_rollout), dtype=np.float64)
    for i, r in enumerate(row_rollout):
        out[i] = 0.0 if r < 0 else float(adv_rollout[r])
    return out
