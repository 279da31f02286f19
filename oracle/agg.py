"""Loss-aggregation modes: how per-token losses of a mini-batch become one
number, and the per-row weights that give each token its share of the
gradient.  TEST INFRASTRUCTURE ONLY (see package docstring).

[P3] section 5 ("global token normalisation"): the token mean divides by the
mini-batch's global valid-token count, the sequence-level modes divide by the
global batch size (a count of sequences), and the policy, entropy and KL
losses all pass through the same aggregation.

Readings (the pages name the modes but print no formula):
* token-mean:           L = sum_t l_t / max(N, 1)
* seq-mean-token-sum:   L = sum_r (sum_{t in r} l_t) / max(B, 1)
* seq-mean-token-mean:  L = sum_r (sum_{t in r} l_t / L_r) / max(B, 1)
with N the valid tokens, L_r the valid tokens of row r, and B the rows that
hold at least one valid token (so masked padding rows, [P4] "Why the row count
does not change the math", do not count).  Sums run over valid tokens only.
"""

AGG_TOKEN_MEAN = 0
AGG_SEQ_MEAN_TOKEN_SUM = 1
AGG_SEQ_MEAN_TOKEN_MEAN = 2


def row_valid_counts(mask, row_off):
    """L_r for every row r (tokens row_off[r] .. row_off[r+1])."""
    out = []
    for r in range(len(row_off) - 1):
        n = 0
        for t in range(row_off[r], row_off[r + 1]):
            n += 1 if mask[t] else 0
        out.append(n)
    return out


def count_rows(mask, row_off):
    """B: the rows holding at least one valid token."""
    return sum(1 for n in row_valid_counts(mask, row_off) if n > 0)


def agg_loss(values, mask, row_off, mode, n_tok, n_seq):
    """The aggregated loss of per-token ``values`` by its definition (see the
    module docstring); ``n_tok`` = N and ``n_seq`` = B of the whole
    mini-batch, which may span several chunks."""
    if mode == AGG_TOKEN_MEAN:
        tot = 0.0
        for t in range(row_off[0], row_off[-1]):
            if mask[t]:
                tot += float(values[t])
        return tot / max(n_tok, 1)
    tot = 0.0
    for r in range(len(row_off) - 1):
        row_sum, L = 0.0, 0
        for t in range(row_off[r], row_off[r + 1]):
            if mask[t]:
                row_sum += float(values[t])
                L += 1
        if L == 0:
            continue
        tot += row_sum if mode == AGG_SEQ_MEAN_TOKEN_SUM else row_sum / L
    if mode not in (AGG_SEQ_MEAN_TOKEN_SUM, AGG_SEQ_MEAN_TOKEN_MEAN):
        raise ValueError(f"unknown aggregation mode {mode}")
    return tot / max(n_seq, 1)


def row_weights(mask, row_off, mode, n_seq):
    """w_r such that agg_loss = sum over valid tokens of w_row(t) * l_t * c,
    where c = 1/max(N, 1) for token-mean (applied as the step's scale) and 1
    otherwise: token-mean 1; seq-mean-token-sum 1/max(B, 1);
    seq-mean-token-mean 1/(max(B, 1) * L_r), 0 for a row without valid
    tokens."""
    Bd = max(n_seq, 1)
    out = []
    for L in row_valid_counts(mask, row_off):
        if mode == AGG_TOKEN_MEAN:
            out.append(1.0)
        elif mode == AGG_SEQ_MEAN_TOKEN_SUM:
            out.append(1.0 / Bd)
        elif mode == AGG_SEQ_MEAN_TOKEN_MEAN:
            out.append(1.0 / (Bd * L) if L > 0 else 0.0)
        else:
            raise ValueError(f"unknown aggregation mode {mode}")
    return out
