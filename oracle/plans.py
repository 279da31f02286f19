"""Batch plans: fixed mini/micro index plans, token-budget dynamic packing and
context-compaction group padding.  TEST INFRASTRUCTURE ONLY (see package
docstring).  Pure Python integers; no floating point anywhere.
"""


class PlanError(ValueError):
    """A rejected plan.  ``kind`` names the failure:

    * ``EINVAL``      malformed arguments (non-positive sizes, batch not a
                      multiple of the group size, a rollout with no rows, ...)
    * ``EDIVISIBLE``  a level does not divide the one above it
    * ``ETOOLONG``    a row holds more tokens than the micro-batch budget
    * ``ECOUNT``      a step does not hold exactly the configured rollouts
    """

    def __init__(self, kind, msg):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind


def plan_fixed(batch, group_size, mini, micro):
    """Fixed mini/micro plan.

    [P1] "The config surface": ``batch`` is a positive multiple of
    ``group_size``; ``mini`` = 0 means the whole batch, ``micro`` = 0 means one
    chunk per mini-batch; the loop counts are derived as batch/mini and
    mini/micro, and each level must divide the one above exactly.
    [P1] "A worked example": 32/16/8 gives 2 x 2; 0/0 gives 1 x 1.
    [P3] section 1 and 2: the same divisibility is demanded of mini- and
    micro-batches.

    Returns ``(n_mini, n_micro, mini_rows, micro_rows)``.
    """
    if batch <= 0 or group_size <= 0:
        raise PlanError("EINVAL", "batch and group_size must be positive")
    if batch % group_size != 0:
        raise PlanError("EINVAL", "batch must be a multiple of group_size")
    if mini < 0 or micro < 0:
        raise PlanError("EINVAL", "mini and micro must be >= 0 (0 = unset)")
    mini_rows = batch if mini == 0 else mini
    micro_rows = mini_rows if micro == 0 else micro
    if batch % mini_rows != 0:
        raise PlanError("EDIVISIBLE", "mini-batch does not divide the batch")
    if mini_rows % micro_rows != 0:
        raise PlanError("EDIVISIBLE", "micro-batch does not divide the mini-batch")
    return batch // mini_rows, mini_rows // micro_rows, mini_rows, micro_rows


def chunk_rows(plan, i_mini, j_micro):
    """Row range ``[begin, end)`` of chunk (i, j) in collected-batch order.

    [P1] "The core idea": the driver passes indices only and the chunk is the
    j-th micro slice of the i-th mini slice of the collected batch.  Reading:
    slices are contiguous and unshuffled.
    """
    n_mini, n_micro, mini_rows, micro_rows = plan
    if not (0 <= i_mini < n_mini and 0 <= j_micro < n_micro):
        raise PlanError("EINVAL", "chunk index out of range")
    begin = i_mini * mini_rows + j_micro * micro_rows
    return begin, begin + micro_rows


def train_calls(plan):
    """Driver loop order: for mini in range(n_mini): for micro in range(n_micro).

    [P1] "A worked example" and "The loop at a glance".
    """
    n_mini, n_micro = plan[0], plan[1]
    calls = []
    for i in range(n_mini):
        for j in range(n_micro):
            calls.append((i, j))
    return calls


def _ceil_div(a, b):
    return -(-a // b)


def plan_dynamic(lengths, token_budget, proxy_div=4096):
    """Token-budget dynamic micro-batch packing.

    [P3] section 3: micro-batches are re-boxed so each holds at most the token
    cap, the cap must cover the longest sample, the micro-batch count starts
    from the total token count, a workload estimate per sample balances the
    boxes, and an index map restores the original order afterwards.

    The pages name no partition algorithm.  Reading taken here (a
    capacity-constrained greedy "longest processing time first"):

    1. any row longer than the budget -> ETOOLONG;
    2. k = max(1, ceil(sum(L) / budget)) boxes;
    3. workload w = proxy_div*L + L*L (proxy_div times the proxy L + L^2/proxy_div,
       kept integral);
    4. rows are visited by decreasing w, ties by increasing row index; each goes
       to the box with the smallest (workload so far, box index) among the
       boxes it still fits in;
    5. if a row fits in no box, k grows by one and packing starts over;
    6. inside a box rows keep their original order; boxes keep their index.

    Returns a dict with ``n_bins``, ``bin_off`` (n_bins+1 offsets into
    ``order``), ``order`` (packed position -> original row) and ``restore``
    (original row -> packed position).
    """
    lengths = [int(x) for x in lengths]
    if token_budget <= 0 or proxy_div <= 0:
        raise PlanError("EINVAL", "token_budget and proxy_div must be positive")
    for L in lengths:
        if L < 0:
            raise PlanError("EINVAL", "negative row length")
        if L > token_budget:
            raise PlanError("ETOOLONG", "a row exceeds the token budget")
    n = len(lengths)
    if n == 0:
        return {"n_bins": 0, "bin_off": [0], "order": [], "restore": []}
    work = [proxy_div * L + L * L for L in lengths]
    visit = sorted(range(n), key=lambda i: (-work[i], i))
    k = max(1, _ceil_div(sum(lengths), token_budget))
    while True:
        tokens = [0] * k
        wsum = [0] * k
        members = [[] for _ in range(k)]
        ok = True
        for i in visit:
            best = None
            for b in range(k):
                if tokens[b] + lengths[i] <= token_budget:
                    if best is None or (wsum[b], b) < (wsum[best], best):
                        best = b
            if best is None:
                ok = False
                break
            tokens[best] += lengths[i]
            wsum[best] += work[i]
            members[best].append(i)
        if ok:
            break
        k += 1
    order = []
    bin_off = [0]
    for b in range(k):
        order.extend(sorted(members[b]))
        bin_off.append(len(order))
    restore = [0] * n
    for p, i in enumerate(order):
        restore[i] = p
    return {"n_bins": k, "bin_off": bin_off, "order": order, "restore": restore}


def plan_compaction(rows_per_rollout, n_groups, group_size, Q, expected_rollouts,
                    dynamic=False):
    """Context-compaction rows with per-group padding to a multiple of Q.

    [P4] opening paragraphs: prompts x generations must equal the configured
    batch size, counted in rollouts; a step that does not hold exactly that many
    rollouts raises (-> ECOUNT).
    [P4] figure: each rollout contributes one row per segment; each group's rows
    are padded up to a multiple of Q; a pad row copies a real row's input, has
    reward 0 and is masked.  Worked example: segments (1,3),(2,5),(1,1), G=2,
    Q=4 -> 4+0, 7+1, 2+2 = 13 real + 3 pad = 16 rows.
    [P4] "What it costs": compaction runs with fixed batching only; dynamic
    batching is rejected (-> EINVAL when ``dynamic``).

    Readings: real rows are listed rollout-major in segment order; the pads of
    a group follow its real rows; a pad copies the group's first real row.
    ``row_src`` numbers real rows in input order (all segments of rollout 0,
    then rollout 1, ...); pads carry rollout -1 and segment -1.
    """
    if dynamic:
        raise PlanError("EINVAL", "context compaction runs with fixed batching only")
    if n_groups <= 0 or group_size <= 0 or Q <= 0:
        raise PlanError("EINVAL", "n_groups, group_size and Q must be positive")
    rows_per_rollout = [int(x) for x in rows_per_rollout]
    if n_groups * group_size != expected_rollouts:
        raise PlanError("ECOUNT", "prompts x generations != configured rollouts")
    if len(rows_per_rollout) != expected_rollouts:
        raise PlanError("ECOUNT", "the step does not hold the configured rollouts")
    for c in rows_per_rollout:
        if c < 1:
            raise PlanError("EINVAL", "a rollout without rows")
    first_src = []
    s = 0
    for c in rows_per_rollout:
        first_src.append(s)
        s += c
    row_rollout, row_seg, row_src, is_pad, group_pad = [], [], [], [], []
    for g in range(n_groups):
        real = 0
        group_first = first_src[g * group_size]
        for r in range(g * group_size, (g + 1) * group_size):
            for k in range(rows_per_rollout[r]):
                row_rollout.append(r)
                row_seg.append(k)
                row_src.append(first_src[r] + k)
                is_pad.append(0)
                real += 1
        pad = (-real) % Q
        group_pad.append(pad)
        for _ in range(pad):
            row_rollout.append(-1)
            row_seg.append(-1)
            row_src.append(group_first)
            is_pad.append(1)
    return {"n_rows": len(row_rollout), "row_rollout": row_rollout,
            "row_seg": row_seg, "row_src": row_src, "is_pad": is_pad,
            "group_pad": group_pad}


def compaction_micro_chunks(n_rows, micro_rows):
    """Micro-batches over the padded compaction rows; one optimizer step.

    [P4] "Why the row count does not change the math", item 3: more rows mean
    more micro-batches, never more optimizer steps (so n_mini = 1).
    Exact divisibility as in [P1] "The config surface".
    """
    if micro_rows <= 0:
        raise PlanError("EINVAL", "micro_rows must be positive")
    if n_rows % micro_rows != 0:
        raise PlanError("EDIVISIBLE", "micro-batch does not divide the padded rows")
    return [(c * micro_rows, (c + 1) * micro_rows) for c in range(n_rows // micro_rows)]


# --------------------------------------------------------------------------
# inner epochs and the seeded mini-batch shuffle
# --------------------------------------------------------------------------

_M64 = (1 << 64) - 1


def splitmix64_stream(seed):
    """The splitmix64 generator (Steele, Lea and Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014; Vigna's public-domain
    reference): the state advances by 0x9E3779B97F4A7C15 and each output is
    the state put through two xor-shift-multiply rounds and a final
    xor-shift.  Yields 64-bit integers."""
    state = seed & _M64
    while True:
        state = (state + 0x9E3779B97F4A7C15) & _M64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
        yield z ^ (z >> 31)


def fisher_yates(n, draws):
    """The Fisher-Yates shuffle of 0..n-1 (Knuth, TAOCP vol. 2, Algorithm P):
    for i = n-1 down to 1, swap item i with item j = draw mod (i + 1), one
    64-bit draw per i.  (The modulo's bias is below 2^-40 for n < 2^24.)"""
    a = list(range(n))
    for i in range(n - 1, 0, -1):
        j = next(draws) % (i + 1)
        a[i], a[j] = a[j], a[i]
    return a


def plan_epochs(batch, group_size, mini, micro, mu, shuffle, seed):
    """Inner epochs over one collected batch, optionally reshuffled.

    [P3] section 1: the controller hands each update its mini-batch size,
    the number of epochs and whether to shuffle with a data-loader seed; the
    iterator yields the mini-batches of the (shuffled) batch again each epoch,
    and the batch must divide into mini-batches.  [P1] "What's not done",
    item 2: inner epochs (mu > 1) reuse the frozen pi_old of the ahead pass
    unchanged.

    Reading: ``plan_fixed`` sizes the levels; epoch e visits the rows in the
    order perm[e] -- the identity without ``shuffle``, else the Fisher-Yates
    permutation driven by one splitmix64 stream seeded with ``seed`` and
    consumed epoch after epoch (n - 1 draws each) -- and mini-batch i /
    micro-batch j of epoch e are the contiguous slices of that order.  mu >= 1.

    Returns ``plan_fixed``'s tuple plus ``mu`` and ``perm`` (mu lists).
    """
    if mu < 1:
        raise PlanError("EINVAL", "mu (epochs) must be >= 1")
    n_mini, n_micro, mini_rows, micro_rows = plan_fixed(batch, group_size, mini, micro)
    draws = splitmix64_stream(seed)
    perm = [fisher_yates(batch, draws) if shuffle else list(range(batch)) for _ in range(mu)]
    return {"n_mini": n_mini, "n_micro": n_micro, "mini_rows": mini_rows, "micro_rows": micro_rows,
            "mu": mu, "perm": perm}


def epoch_chunk_rows(ep, e, i_mini, j_micro):
    """The rows (in order) of chunk (e, i, j) of an epoch plan."""
    if not (0 <= e < ep["mu"] and 0 <= i_mini < ep["n_mini"] and 0 <= j_micro < ep["n_micro"]):
        raise PlanError("EINVAL", "chunk index out of range")
    a = i_mini * ep["mini_rows"] + j_micro * ep["micro_rows"]
    return ep["perm"][e][a:a + ep["micro_rows"]]


def epoch_train_calls(ep):
    """The (e, i, j) train calls of an epoch plan, in driver order: epochs
    outermost, then mini-batches, then micro-batches."""
    return [(e, i, j) for e in range(ep["mu"]) for i in range(ep["n_mini"]) for j in range(ep["n_micro"])]
