"""Per-token log-softmax statistics, the clipped GRPO surrogate, its gradient
with respect to the logits, and the row / chunk roll-ups.

TEST INFRASTRUCTURE ONLY (see package docstring).  float64 throughout; one
token row at a time so that each line can be checked against the definition.
"""

import math

import numpy as np


# --------------------------------------------------------------------------
# bf16 rounding (used only to express "the oracle rounded once to the output
# dtype" when a kernel stores bf16)
# --------------------------------------------------------------------------

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_to_bf16(x):
    """Round float64 values once, to nearest-even, onto the bf16 grid.

    bf16 keeps 8 significant bits and fp32's exponent range (normal minimum
    2^-126, subnormal quantum 2^-133).  Rounding straight from float64 avoids
    the double rounding of going through float32.  Non-finite values pass
    through; finite values past the largest bf16 become infinities.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x)
    xf = x[fin]
    _, e = np.frexp(xf)                  # xf = m * 2^e with 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133).astype(np.float64)
    scale = np.exp2(q)
    r = np.rint(xf / scale) * scale      # np.rint rounds halves to even
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


# --------------------------------------------------------------------------
# one token
# --------------------------------------------------------------------------

def token_forward(z, y):
    """Log-softmax statistics of one logit row ``z`` (float64 [V]) for target y.

    [P1] "The problem": the loss needs the log-softmax over the completion
    logits.  [P2] "Field Lineage" (reward, log-prob and advantage): the
    recompute yields per-token log-probs and an entropy.

    Returns ``(lse, logp, H, p)`` with lse = log sum_v exp(z_v), logp = z_y - lse,
    p_v = exp(z_v - lse) and H = -sum_v p_v (z_v - lse) (terms with p_v = 0 count
    as 0).  A target outside [0, V) gives logp = NaN.
    """
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z)
    s = np.sum(np.exp(z - m))
    lse = m + math.log(s)
    p = np.exp(z - lse)
    with np.errstate(invalid="ignore"):
        terms = np.where(p > 0.0, p * (z - lse), 0.0)
    H = -float(np.sum(terms))
    if 0 <= y < z.shape[0]:
        logp = float(z[y]) - lse
    else:
        logp = float("nan")
    return float(lse), logp, H, p


def surrogate(logp, old_logp, A, eps_low, eps_high):
    """Clipped surrogate for one token.

    [P1] "pi_old must be frozen across the window": the ratio is
    exp(logp - old_logp) and the epsilon-clip bounds it (pi_old = the rollout
    policy).  [P1] "The hard part: deferred normalization": the loss is a
    token mean.

    Reading (the pages name the clip but print no formula): symmetric or
    asymmetric PPO clip, l = -min(rho*A, clip(rho, 1-eps_low, 1+eps_high)*A).  The
    gradient gate g is 0 exactly where the clipped branch is the smaller one
    and the clip binds, i.e. (A > 0 and rho > 1+eps_high) or (A < 0 and
    rho < 1-eps_low); on the interval's edges g = 1.

    Returns ``(l, g, rho)``.
    """
    with np.errstate(over="ignore", invalid="ignore"):
        rho = float(np.exp(np.float64(logp) - np.float64(old_logp)))
    s1 = rho * A
    s2 = min(max(rho, 1.0 - eps_low), 1.0 + eps_high) * A
    l = -min(s1, s2)
    g = 0 if ((A > 0 and rho > 1.0 + eps_high) or (A < 0 and rho < 1.0 - eps_low)) else 1
    return l, g, rho


KL_K1, KL_K2, KL_K3 = 1, 2, 3


def kl_term(logp, ref_logp, kind):
    """Per-token estimate of KL(current || reference) from the sampled
    token's two log-probs, and its derivative with respect to logp.

    [P2] "Field Lineage": the reference worker writes ref_log_prob next to the
    old log-probs.  [P3] section 5: the KL loss is aggregated like the policy
    loss.

    Reading (the pages name a KL loss but print no estimator): with
    d = ref_logp - logp,
      k1: KL = -d,             dKL/dlogp = 1
      k2: KL = d^2 / 2,        dKL/dlogp = -d
      k3: KL = e^d - d - 1,    dKL/dlogp = 1 - e^d
    with no clamp (an overflow makes the token non-finite, as for the ratio).
    Returns ``(KL, dKL/dlogp)``.
    """
    d = float(ref_logp) - float(logp)
    if kind == KL_K1:
        return -d, 1.0
    if kind == KL_K2:
        return 0.5 * d * d, -d
    if kind == KL_K3:
        with np.errstate(over="ignore"):
            ed = float(np.exp(np.float64(d)))
        return ed - d - 1.0, 1.0 - ed
    raise ValueError(f"unknown KL estimator {kind}")


def loss_fwd_bwd(logits, target, mask, old_logp, adv_tok, scale,
                 eps_low=0.2, eps_high=0.2, want_dz=True, w_tok=None,
                 ent_coef=0.0, kl_coef=0.0, ref_logp=None, kl_type=KL_K3):
    """Fused forward and backward of the token-level GRPO loss over one chunk.

    ``logits`` [n_tok, V] (read as float64), ``target`` [n_tok] int,
    ``mask`` [n_tok] (1 = policy token), ``old_logp`` [n_tok],
    ``adv_tok`` [n_tok] the advantage of each token's row, ``scale`` the factor
    applied to the gradient (1/max(N,1) for a step of N valid tokens, or 1 to
    leave the division for the optimizer step).

    [P1] "The hard part: deferred normalization": the loss is the sum of the
    per-token losses over valid tokens divided by N; the gradient of a chunk
    is linear in its tokens.  [P2] "Field Lineage" (response mask semantics):
    only mask-1 tokens carry loss; the advantage is broadcast and multiplied
    by the mask.  [P4] "Why the row count does not change the math", item 1:
    pads have no valid tokens and add nothing.

    Per valid token: lse, logp, H (``token_forward``); l, g, rho
    (``surrogate``); coef = scale * A * rho * g; dz_v = coef * (p_v - [v == y]),
    which is d(scale * l)/dz_v.  Masked tokens: every output 0 and dz = 0.

    Extra terms ([P3] section 5: the policy, entropy and KL losses share one
    aggregation).  ``w_tok`` [n_tok] (default 1) multiplies each token's
    factor, s_t = scale * w_tok[t] (the aggregation-mode weight of the token's
    row, ``agg.row_weights``).  The token's objective is
      obj_t = s_t * (l_t - ent_coef * H_t + kl_coef * KL_t)
    (entropy as a bonus, KL from ``kl_term`` against ``ref_logp``), and dz is
    its gradient:
      dz_v = coef_t (p_v - [v == y]) + ent_coef s_t p_v (z_v - lse + H_t),
      coef_t = s_t (A rho g - kl_coef dKL/dlogp),
    using dlogp/dz_v = [v == y] - p_v and dH/dz_v = -p_v (z_v - lse + H).

    Returns a dict of float64 arrays: ``logp``, ``lse``, ``entropy``,
    ``loss_tok``, ``kl``, ``obj``, ``coef``, ``clipped`` (bool, g == 0),
    ``valid`` (bool), ``nonfinite`` (bool) and ``dz`` ([n_tok, V] or None).
    """
    logits = np.asarray(logits)
    n, V = logits.shape
    out = {k: np.zeros(n, dtype=np.float64) for k in ("logp", "lse", "entropy", "loss_tok", "kl", "obj", "coef")}
    out["clipped"] = np.zeros(n, dtype=bool)
    out["valid"] = np.zeros(n, dtype=bool)
    out["nonfinite"] = np.zeros(n, dtype=bool)
    dz = np.zeros((n, V), dtype=np.float64) if want_dz else None
    for t in range(n):
        if not mask[t]:
            continue
        out["valid"][t] = True
        z = logits[t].astype(np.float64)
        y = int(target[t])
        lse, logp, H, p = token_forward(z, y)
        A = float(adv_tok[t])
        l, g, rho = surrogate(logp, float(old_logp[t]), A, eps_low, eps_high)
        s = scale * (1.0 if w_tok is None else float(w_tok[t]))
        kl, dkl = (0.0, 0.0) if ref_logp is None else kl_term(logp, float(ref_logp[t]), kl_type)
        coef = s * (A * rho * g - kl_coef * dkl)
        out["logp"][t] = logp
        out["lse"][t] = lse
        out["entropy"][t] = H
        out["loss_tok"][t] = l
        out["kl"][t] = kl
        out["obj"][t] = s * (l - ent_coef * H + kl_coef * kl)
        out["coef"][t] = coef
        out["clipped"][t] = (g == 0)
        out["nonfinite"][t] = not (math.isfinite(logp) and math.isfinite(l) and math.isfinite(H)
                                   and math.isfinite(kl))
        if want_dz:
            row = coef * p
            if ent_coef != 0.0:
                with np.errstate(invalid="ignore"):
                    row = row + np.where(p > 0.0, ent_coef * s * p * (z - lse + H), 0.0)
            if 0 <= y < V:
                row[y] -= coef
            dz[t] = row
    out["dz"] = dz
    return out


def logprob_fwd(logits, target, mask):
    """Forward-only recompute of the per-token log-prob, logsumexp and entropy.

    [P1] "pi_old must be frozen across the window": the ahead pass walks the
    chunks once without gradients and records pi_old per chunk.  [P2] "Field
    Lineage": the normal-mode recompute yields old log-probs plus entropy.
    Masked tokens give zeros.
    """
    logits = np.asarray(logits)
    n = logits.shape[0]
    logp = np.zeros(n)
    lse = np.zeros(n)
    ent = np.zeros(n)
    for t in range(n):
        if not mask[t]:
            continue
        a, b, c, _ = token_forward(logits[t].astype(np.float64), int(target[t]))
        lse[t], logp[t], ent[t] = a, b, c
    return {"logp": logp, "lse": lse, "entropy": ent}


# --------------------------------------------------------------------------
# roll-ups
# --------------------------------------------------------------------------

def valid_count(mask):
    """N = number of mask-1 tokens (an integer).

    [P1] "The hard part: deferred normalization": N counts the masked
    completion positions.  [P3] section 5: the token mean uses the summed
    loss-mask count.  [P4] "Why the row count does not change the math",
    item 1: padding counts 0.
    """
    n = 0
    for m in mask:
        n += 1 if m else 0
    return n


STAT_KEYS = ("loss_sum", "entropy_sum", "kl_sum", "obj_sum", "n_valid", "n_clipped", "n_nonfinite",
             "n_valid_rows")


def _stats_over(out, idx):
    s = {k: 0.0 if k.endswith("_sum") else 0 for k in STAT_KEYS}
    for t in idx:
        if not out["valid"][t]:
            continue
        s["loss_sum"] += float(out["loss_tok"][t])
        s["entropy_sum"] += float(out["entropy"][t])
        s["kl_sum"] += float(out["kl"][t]) if "kl" in out else 0.0
        s["obj_sum"] += float(out["obj"][t]) if "obj" in out else 0.0
        s["n_valid"] += 1
        s["n_clipped"] += 1 if out["clipped"][t] else 0
        s["n_nonfinite"] += 1 if out["nonfinite"][t] else 0
    s["n_valid_rows"] = 1 if s["n_valid"] > 0 else 0
    return s


def row_stats(out, row_off):
    """Per-row sums of loss, entropy, KL and objective and counts, tokens of row r being
    ``row_off[r]:row_off[r+1]``; ``n_valid_rows`` is 1 for a row holding a
    valid token.

    [P1] "Metric roll-up: token-weighted, not averaged": losses roll up as
    sums weighted by their token counts, counts sum.  [P4] "What it costs":
    the row-count metric counts rows, so under compaction it can exceed the
    rollouts; reading: a row counts when it holds a valid token, so pads
    (no valid tokens, [P2] "DP batch balance and padding") never count.
    """
    return [_stats_over(out, range(row_off[r], row_off[r + 1])) for r in range(len(row_off) - 1)]


def chunk_stats(out, row_off):
    """Chunk totals, summed over the rows in row order: loss_sum,
    entropy_sum, kl_sum, obj_sum (the chunk's share of the aggregated
    objective), n_valid (the chunk's divisor), n_clipped, n_nonfinite,
    n_valid_rows.  The reported chunk loss is loss_sum / max(n_valid, 1).

    [P1] "The hard part: deferred normalization" (the objective reports the
    divisor it used) and "Metric roll-up".
    """
    tot = {k: 0.0 if k.endswith("_sum") else 0 for k in STAT_KEYS}
    for r in row_stats(out, row_off):
        for k in tot:
            tot[k] += r[k]
    return tot
