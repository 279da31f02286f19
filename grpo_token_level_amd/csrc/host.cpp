// Host half of libgrpo: batch plans (fixed, epochs, dynamic packing,
// compaction), group advantages, the step accumulator, the frozen pi_old
// cache bookkeeping and the probe verdict.  Pure functions of their arguments
// (no allocation beyond small temporaries of the dynamic packer); the only
// device work is the forward pass a cache record enqueues through
// grpo_logprob_fwd.
//
// Sources: [P1] "Sizing mini-batches and micro-batches"; [P2] "03 Data
// Protocol and Batch Lifecycle"; [P3] "22 - mini-batch, micro-batch and
// dynamic batch size"; [P4] "How a context-compaction step fits a variable
// number of rows into one batch".

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <vector>

#include "common.h"

namespace grpo {

namespace {
thread_local char g_err[512] = "";
}

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return GRPO_OK;
}

}  // namespace grpo

using grpo::fail;
using grpo::ok;

extern "C" const char* grpo_last_error(void) { return grpo::g_err; }

extern "C" const char* grpo_version(void) { return "grpo-mi355x 0.1 (gfx950)"; }

// ---------------------------------------------------------------- plans

// [P1] "The config surface": three replica-level knobs, 0 = unset for mini and
// micro, derived loop counts, exact divisibility at every level.
extern "C" int grpo_plan_fixed(int64_t batch, int64_t group_size, int64_t mini, int64_t micro,
                               int64_t* n_mini, int64_t* n_micro, int64_t* mini_rows,
                               int64_t* micro_rows) {
    if (!n_mini || !n_micro || !mini_rows || !micro_rows)
        return fail(GRPO_EINVAL, "grpo_plan_fixed: NULL output");
    if (batch <= 0 || group_size <= 0)
        return fail(GRPO_EINVAL, "grpo_plan_fixed: batch (%lld) and group_size (%lld) must be positive",
                    (long long)batch, (long long)group_size);
    if (batch % group_size != 0)
        return fail(GRPO_EINVAL, "grpo_plan_fixed: batch %lld is not a multiple of group_size %lld",
                    (long long)batch, (long long)group_size);
    if (mini < 0 || micro < 0)
        return fail(GRPO_EINVAL, "grpo_plan_fixed: mini and micro must be >= 0 (0 = unset)");
    const int64_t mr = mini == 0 ? batch : mini;
    const int64_t ur = micro == 0 ? mr : micro;
    if (batch % mr != 0)
        return fail(GRPO_EDIVISIBLE, "grpo_plan_fixed: mini-batch %lld does not divide batch %lld",
                    (long long)mr, (long long)batch);
    if (mr % ur != 0)
        return fail(GRPO_EDIVISIBLE, "grpo_plan_fixed: micro-batch %lld does not divide mini-batch %lld",
                    (long long)ur, (long long)mr);
    *n_mini = batch / mr;
    *n_micro = mr / ur;
    *mini_rows = mr;
    *micro_rows = ur;
    return ok();
}

namespace {
// splitmix64 (Steele, Lea and Flood, OOPSLA 2014): the state advances by the
// golden-ratio increment; each output is the state through two
// xor-shift-multiply rounds and a final xor-shift.
struct SplitMix64 {
    uint64_t state;
    uint64_t next() {
        state += 0x9E3779B97F4A7C15ull;
        uint64_t z = state;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
};
}  // namespace

// [P3] section 1: epochs of the mini-batch iterator, reshuffled with a seed.
// One generator stream, consumed epoch after epoch; the Fisher-Yates shuffle
// (Knuth, Algorithm P) swaps item i with item (draw mod (i + 1)) for i from
// the last down to 1.
extern "C" int grpo_plan_epochs(int64_t batch, int64_t group_size, int64_t mini, int64_t micro, int64_t mu,
                                int32_t shuffle, uint64_t seed, int64_t* n_mini, int64_t* n_micro,
                                int64_t* mini_rows, int64_t* micro_rows, int64_t* perm) {
    if (mu < 1) return fail(GRPO_EINVAL, "grpo_plan_epochs: mu (epochs) must be >= 1");
    if (!perm) return fail(GRPO_EINVAL, "grpo_plan_epochs: NULL perm");
    int64_t a, b, c, d;
    const int rc = grpo_plan_fixed(batch, group_size, mini, micro, &a, &b, &c, &d);
    if (rc != GRPO_OK) return rc;
    SplitMix64 g{seed};
    for (int64_t e = 0; e < mu; ++e) {
        int64_t* p = perm + e * batch;
        for (int64_t i = 0; i < batch; ++i) p[i] = i;
        if (!shuffle) continue;
        for (int64_t i = batch - 1; i >= 1; --i) {
            const int64_t j = (int64_t)(g.next() % (uint64_t)(i + 1));
            std::swap(p[i], p[j]);
        }
    }
    *n_mini = a;
    *n_micro = b;
    *mini_rows = c;
    *micro_rows = d;
    return ok();
}

// [P1] "The core idea": chunk (i, j) is the j-th micro slice of the i-th mini
// slice; the driver only ever names the indices.
extern "C" int grpo_plan_chunk(int64_t batch, int64_t mini_rows, int64_t micro_rows, int64_t i_mini,
                               int64_t j_micro, int64_t* row_begin, int64_t* row_end) {
    if (!row_begin || !row_end) return fail(GRPO_EINVAL, "grpo_plan_chunk: NULL output");
    if (batch <= 0 || mini_rows <= 0 || micro_rows <= 0 || batch % mini_rows || mini_rows % micro_rows)
        return fail(GRPO_EINVAL, "grpo_plan_chunk: not a valid fixed plan");
    if (i_mini < 0 || i_mini >= batch / mini_rows || j_micro < 0 || j_micro >= mini_rows / micro_rows)
        return fail(GRPO_EINVAL, "grpo_plan_chunk: chunk (%lld, %lld) out of range", (long long)i_mini,
                    (long long)j_micro);
    *row_begin = i_mini * mini_rows + j_micro * micro_rows;
    *row_end = *row_begin + micro_rows;
    return ok();
}

// [P3] section 3: token cap per micro-batch, cap >= longest row, box count
// from the total, workload-balanced assignment, restore index.  The packer is
// a capacity-constrained greedy (heaviest workload first into the lightest box
// that fits).  Box loads live in a small array scanned linearly: the box count
// is ceil(total / budget), tens at most for the budgets in use.
extern "C" int grpo_plan_dynamic(const int64_t* len, int64_t n_rows, int64_t token_budget,
                                 int64_t proxy_div, int64_t cap_bins, int64_t* n_bins,
                                 int64_t* bin_off, int64_t* order, int64_t* restore) {
    if (!n_bins || n_rows < 0 || (n_rows > 0 && (!len || !order || !restore)) || !bin_off)
        return fail(GRPO_EINVAL, "grpo_plan_dynamic: NULL pointer or negative n_rows");
    if (token_budget <= 0 || proxy_div <= 0)
        return fail(GRPO_EINVAL, "grpo_plan_dynamic: token_budget and proxy_div must be positive");
    if (cap_bins < 0) return fail(GRPO_EINVAL, "grpo_plan_dynamic: negative cap_bins");
    int64_t total = 0;
    for (int64_t i = 0; i < n_rows; ++i) {
        if (len[i] < 0) return fail(GRPO_EINVAL, "grpo_plan_dynamic: negative length at row %lld", (long long)i);
        if (len[i] > token_budget)
            return fail(GRPO_ETOOLONG, "grpo_plan_dynamic: row %lld has %lld tokens > budget %lld",
                        (long long)i, (long long)len[i], (long long)token_budget);
        total += len[i];
    }
    if (n_rows == 0) {
        *n_bins = 0;
        bin_off[0] = 0;
        return ok();
    }
    std::vector<int64_t> work(n_rows);
    for (int64_t i = 0; i < n_rows; ++i) work[i] = proxy_div * len[i] + len[i] * len[i];
    std::vector<int64_t> visit(n_rows);
    std::iota(visit.begin(), visit.end(), int64_t{0});
    std::sort(visit.begin(), visit.end(), [&](int64_t a, int64_t b) {
        return work[a] != work[b] ? work[a] > work[b] : a < b;
    });
    int64_t k = std::max<int64_t>(1, (total + token_budget - 1) / token_budget);
    std::vector<int64_t> tok, wsum, box(n_rows);
    for (;;) {
        tok.assign(k, 0);
        wsum.assign(k, 0);
        bool fits = true;
        for (int64_t i : visit) {
            int64_t best = -1;
            for (int64_t b = 0; b < k; ++b) {
                if (tok[b] + len[i] > token_budget) continue;
                if (best < 0 || wsum[b] < wsum[best]) best = b;   // ties keep the lower box
            }
            if (best < 0) {
                fits = false;
                break;
            }
            tok[best] += len[i];
            wsum[best] += work[i];
            box[i] = best;
        }
        if (fits) break;
        ++k;
    }
    if (k > cap_bins) {
        *n_bins = k;
        return fail(GRPO_ECAPACITY, "grpo_plan_dynamic: %lld boxes needed, capacity %lld", (long long)k,
                    (long long)cap_bins);
    }
    // Counting sort by box keeps the original row order inside each box.
    std::vector<int64_t> count(k + 1, 0);
    for (int64_t i = 0; i < n_rows; ++i) ++count[box[i] + 1];
    for (int64_t b = 0; b < k; ++b) count[b + 1] += count[b];
    for (int64_t b = 0; b <= k; ++b) bin_off[b] = count[b];
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t p = count[box[i]]++;
        order[p] = i;
        restore[i] = p;
    }
    *n_bins = k;
    return ok();
}

// [P4] figure: one row per segment; each group padded to a multiple of Q with
// pad rows that copy a real row, carry reward 0 and are masked; the step holds
// exactly the configured rollouts or raises.
extern "C" int grpo_plan_compaction(const int32_t* rows_per_rollout, int64_t n_rollouts, int64_t n_groups,
                                    int64_t group_size, int64_t Q, int64_t expected_rollouts,
                                    int32_t dynamic, int64_t cap_rows, int64_t* n_rows,
                                    int32_t* row_rollout, int32_t* row_seg, int32_t* row_src,
                                    uint8_t* row_is_pad, int32_t* group_pad) {
    if (!n_rows || (n_rollouts > 0 && !rows_per_rollout))
        return fail(GRPO_EINVAL, "grpo_plan_compaction: NULL pointer");
    if (dynamic) return fail(GRPO_EINVAL, "grpo_plan_compaction: compaction runs with fixed batching only");
    if (n_groups <= 0 || group_size <= 0 || Q <= 0)
        return fail(GRPO_EINVAL, "grpo_plan_compaction: n_groups, group_size and Q must be positive");
    if (n_groups * group_size != expected_rollouts)
        return fail(GRPO_ECOUNT, "grpo_plan_compaction: %lld groups x %lld != %lld configured rollouts",
                    (long long)n_groups, (long long)group_size, (long long)expected_rollouts);
    if (n_rollouts != expected_rollouts)
        return fail(GRPO_ECOUNT, "grpo_plan_compaction: the step holds %lld rollouts, %lld configured",
                    (long long)n_rollouts, (long long)expected_rollouts);
    for (int64_t r = 0; r < n_rollouts; ++r) {
        if (rows_per_rollout[r] < 1)
            return fail(GRPO_EINVAL, "grpo_plan_compaction: rollout %lld has no rows", (long long)r);
    }
    int64_t need = 0;
    for (int64_t g = 0; g < n_groups; ++g) {
        int64_t real = 0;
        for (int64_t r = g * group_size; r < (g + 1) * group_size; ++r) real += rows_per_rollout[r];
        need += real + ((Q - real % Q) % Q);
    }
    if (need > cap_rows) {
        *n_rows = need;
        return fail(GRPO_ECAPACITY, "grpo_plan_compaction: %lld rows needed, capacity %lld", (long long)need,
                    (long long)cap_rows);
    }
    if (!row_rollout || !row_seg || !row_src || !row_is_pad || !group_pad)
        return fail(GRPO_EINVAL, "grpo_plan_compaction: NULL output");
    int64_t out = 0, src = 0;
    for (int64_t g = 0; g < n_groups; ++g) {
        const int64_t first = src;
        int64_t real = 0;
        for (int64_t r = g * group_size; r < (g + 1) * group_size; ++r) {
            for (int32_t k = 0; k < rows_per_rollout[r]; ++k) {
                row_rollout[out] = (int32_t)r;
                row_seg[out] = k;
                row_src[out] = (int32_t)(src++);
                row_is_pad[out] = 0;
                ++out;
                ++real;
            }
        }
        const int64_t pad = (Q - real % Q) % Q;
        group_pad[g] = (int32_t)pad;
        for (int64_t k = 0; k < pad; ++k) {
            row_rollout[out] = -1;
            row_seg[out] = -1;
            row_src[out] = (int32_t)first;
            row_is_pad[out] = 1;
            ++out;
        }
    }
    *n_rows = out;
    return ok();
}

extern "C" int grpo_row_offsets(const int64_t* len, const int64_t* order, int64_t n_rows, int64_t* row_off) {
    if (n_rows < 0 || !row_off || (n_rows > 0 && !len)) return fail(GRPO_EINVAL, "grpo_row_offsets: bad arguments");
    row_off[0] = 0;
    for (int64_t k = 0; k < n_rows; ++k) {
        int64_t r = k;
        if (order) {
            r = order[k];
            if (r < 0 || r >= n_rows) return fail(GRPO_EINVAL, "grpo_row_offsets: order[%lld] out of range", (long long)k);
        }
        if (len[r] < 0) return fail(GRPO_EINVAL, "grpo_row_offsets: negative length");
        row_off[k + 1] = row_off[k] + len[r];
    }
    return ok();
}

// ---------------------------------------------------------------- advantage

// [P2] "Field Lineage": advantages come from trajectory rewards once per
// update; [P4] item 2: one value per rollout.  Formula not on the pages:
// (r - mean) / (unbiased std + eps), or r - mean, or 0 for groups of one.
extern "C" int grpo_group_advantage(const float* reward, int64_t n_rollouts, int64_t group_size, float eps,
                                    int32_t norm_by_std, float* adv_rollout) {
    if (n_rollouts < 0 || group_size <= 0 || (n_rollouts > 0 && (!reward || !adv_rollout)))
        return fail(GRPO_EINVAL, "grpo_group_advantage: bad arguments");
    if (n_rollouts % group_size != 0)
        return fail(GRPO_EINVAL, "grpo_group_advantage: %lld rollouts is not a whole number of groups of %lld",
                    (long long)n_rollouts, (long long)group_size);
    const int64_t G = group_size;
    for (int64_t g = 0; g < n_rollouts / G; ++g) {
        const float* r = reward + g * G;
        float* a = adv_rollout + g * G;
        if (G == 1) {
            a[0] = 0.0f;
            continue;
        }
        double sum = 0.0;
        for (int64_t k = 0; k < G; ++k) sum += (double)r[k];
        const double mean = sum / (double)G;
        double sq = 0.0;
        for (int64_t k = 0; k < G; ++k) sq += ((double)r[k] - mean) * ((double)r[k] - mean);
        const double sd = std::sqrt(sq / (double)(G - 1));
        for (int64_t k = 0; k < G; ++k) {
            const double d = (double)r[k] - mean;
            a[k] = (float)(norm_by_std ? d / (sd + (double)eps) : d);
        }
    }
    return ok();
}

extern "C" int grpo_rows_advantage(const float* adv_rollout, int64_t n_rollouts, const int32_t* row_rollout,
                                   int64_t n_rows, float* adv_row) {
    if (n_rows < 0 || n_rollouts < 0 || (n_rows > 0 && (!row_rollout || !adv_row)))
        return fail(GRPO_EINVAL, "grpo_rows_advantage: bad arguments");
    for (int64_t i = 0; i < n_rows; ++i) {
        if (row_rollout[i] >= n_rollouts)
            return fail(GRPO_EINVAL, "grpo_rows_advantage: row %lld names rollout %d of %lld", (long long)i,
                        row_rollout[i], (long long)n_rollouts);
    }
    for (int64_t i = 0; i < n_rows; ++i) adv_row[i] = row_rollout[i] < 0 ? 0.0f : adv_rollout[row_rollout[i]];
    return ok();
}

// ---------------------------------------------------------------- accumulator

// The window state behind the opaque grpo_accum handle.
struct grpo_accum {
    uint64_t magic;     // kAccumMagic once grpo_accum_init has run
    int64_t n_micro;
    int64_t pos;        // chunks accumulated in the open window
    int64_t skip;       // calls still to swallow
    int32_t done;       // a completed window waits for grpo_accum_finalize
    int32_t reserved;
    grpo_stats open;    // sums of the open window
    grpo_stats closed;  // sums of the completed window
};

namespace {
constexpr uint64_t kAccumMagic = 0x6772706f61636331ull;
bool accum_ready(const grpo_accum* a) { return a && a->magic == kAccumMagic && a->n_micro >= 1; }

void stats_zero(grpo_stats* s) { std::memset(s, 0, sizeof(*s)); }
void stats_add(grpo_stats* a, const grpo_stats* b) {
    a->loss_sum += b->loss_sum;
    a->entropy_sum += b->entropy_sum;
    a->kl_sum += b->kl_sum;
    a->obj_sum += b->obj_sum;
    a->n_valid += b->n_valid;
    a->n_clipped += b->n_clipped;
    a->n_nonfinite += b->n_nonfinite;
    a->n_valid_rows += b->n_valid_rows;
}
}  // namespace

extern "C" int grpo_stats_sum(const grpo_stats* rows, int64_t n, grpo_stats* out) {
    if (n < 0 || !out || (n > 0 && !rows)) return fail(GRPO_EINVAL, "grpo_stats_sum: bad arguments");
    grpo_stats s;
    stats_zero(&s);
    for (int64_t r = 0; r < n; ++r) stats_add(&s, rows + r);
    *out = s;
    return ok();
}

extern "C" size_t grpo_accum_size(void) { return sizeof(grpo_accum); }

extern "C" int grpo_accum_init(grpo_accum* acc, int64_t n_micro) {
    if (!acc || n_micro < 1) return fail(GRPO_EINVAL, "grpo_accum_init: n_micro must be >= 1");
    std::memset(acc, 0, sizeof(*acc));
    acc->magic = kAccumMagic;
    acc->n_micro = n_micro;
    return ok();
}

// [P1] "The poisoned-window countdown": on a non-finite chunk the window is
// discarded and exactly the remaining chunks of that window are swallowed.
extern "C" int grpo_accum_add(grpo_accum* acc, const grpo_stats* c) {
    if (!accum_ready(acc) || !c) return fail(GRPO_EINVAL, "grpo_accum_add: NULL or unprepared argument");
    if (acc->done) return fail(GRPO_ESTATE, "grpo_accum_add: finalize the completed window first");
    if (acc->skip > 0) {
        --acc->skip;
        return fail(GRPO_ESKIPPED, "grpo_accum_add: call swallowed, %lld more to skip", (long long)acc->skip);
    }
    if (c->n_nonfinite > 0 || !std::isfinite(c->loss_sum) || !std::isfinite(c->entropy_sum) ||
        !std::isfinite(c->kl_sum) || !std::isfinite(c->obj_sum)) {
        acc->skip = acc->n_micro - 1 - acc->pos;
        acc->pos = 0;
        stats_zero(&acc->open);
        return fail(GRPO_ENONFINITE, "grpo_accum_add: non-finite chunk; window discarded, %lld calls to skip",
                    (long long)acc->skip);
    }
    stats_add(&acc->open, c);
    if (++acc->pos == acc->n_micro) {
        acc->closed = acc->open;
        acc->done = 1;
        acc->pos = 0;
        stats_zero(&acc->open);
    }
    return ok();
}

// [P1] "Metric roll-up": token-weighted loss, summed counts; "The hard part":
// one gradient scale 1/max(sum of divisors, 1).
extern "C" int grpo_accum_finalize(grpo_accum* acc, grpo_step_result* out, int32_t* stepped) {
    if (!accum_ready(acc) || !out || !stepped)
        return fail(GRPO_EINVAL, "grpo_accum_finalize: NULL or unprepared argument");
    if (!acc->done) {
        *stepped = 0;
        return ok();
    }
    const grpo_stats& s = acc->closed;
    const double denom = (double)std::max<int64_t>(s.n_valid, 1);
    out->loss = s.loss_sum / denom;
    out->entropy = s.entropy_sum / denom;
    out->kl = s.kl_sum / denom;
    out->obj_sum = s.obj_sum;
    out->grad_scale = 1.0 / denom;
    out->n_valid = s.n_valid;
    out->n_valid_rows = s.n_valid_rows;
    out->n_clipped = s.n_clipped;
    acc->done = 0;
    stats_zero(&acc->closed);
    *stepped = 1;
    return ok();
}

// ---------------------------------------------------------------- frozen pi_old

// [P1] "pi_old must be frozen across the window -- the ahead pass": the gate.
extern "C" int32_t grpo_needs_ahead_pass(int64_t n_mini, int32_t use_rollout_logprobs,
                                         int32_t consumes_old_logprobs) {
    return (n_mini > 1 && !use_rollout_logprobs && consumes_old_logprobs) ? 1 : 0;
}

extern "C" int grpo_old_cache_init(grpo_old_cache* c, float* buf, int64_t capacity, int64_t* off, int64_t n_calls) {
    if (!c || !off || n_calls < 1 || capacity < 0 || (capacity > 0 && !buf))
        return fail(GRPO_EINVAL, "grpo_old_cache_init: need n_calls >= 1, capacity >= 0, buf and off");
    c->buf = buf;
    c->capacity = capacity;
    c->off = off;
    c->n_calls = n_calls;
    return grpo_old_cache_reset(c);
}

extern "C" int grpo_old_cache_reset(grpo_old_cache* c) {
    if (!c || !c->off || c->n_calls < 1) return fail(GRPO_EINVAL, "grpo_old_cache_reset: uninitialised cache");
    c->recorded = 0;
    c->replayed = 0;
    c->off[0] = 0;
    return ok();
}

// Record k is the chunk's forward-only log-probs, appended after record k-1.
namespace {

int old_cache_record(bool paired, void* stream, grpo_old_cache* c, int32_t dtype, const void* logits, int64_t ld,
                     int64_t n_tok, int64_t V, const int32_t* target, const uint8_t* mask, float** slot) {
    if (!c || !c->off || c->n_calls < 1 || n_tok < 0) return fail(GRPO_EINVAL, "grpo_old_cache_record: bad arguments");
    if (c->replayed > 0) return fail(GRPO_ESTATE, "grpo_old_cache_record: replay has begun; reset for the next batch");
    if (c->recorded >= c->n_calls)
        return fail(GRPO_ESTATE, "grpo_old_cache_record: all %lld calls of the walk are recorded",
                    (long long)c->n_calls);
    const int64_t k = c->recorded, at = c->off[k];
    if (at + n_tok > c->capacity)
        return fail(GRPO_ECAPACITY, "grpo_old_cache_record: %lld floats needed, %lld available",
                    (long long)(at + n_tok), (long long)c->capacity);
    float* dst = c->buf ? c->buf + at : nullptr;
    if (n_tok > 0) {
        const int rc = paired ? grpo_logprob_fwd_paired(stream, dtype, logits, ld, n_tok, V, target, mask, dst,
                                                        nullptr, nullptr)
                              : grpo_logprob_fwd(stream, dtype, logits, ld, n_tok, V, target, mask, dst, nullptr,
                                                 nullptr);
        if (rc != GRPO_OK) return rc;
    }
    c->off[k + 1] = at + n_tok;
    c->recorded = k + 1;
    if (slot) *slot = dst;
    return ok();
}

}  // namespace

extern "C" int grpo_old_cache_record(void* stream, grpo_old_cache* c, int32_t dtype, const void* logits, int64_t ld,
                                     int64_t n_tok, int64_t V, const int32_t* target, const uint8_t* mask,
                                     float** slot) {
    return old_cache_record(false, stream, c, dtype, logits, ld, n_tok, V, target, mask, slot);
}

extern "C" int grpo_old_cache_record_paired(void* stream, grpo_old_cache* c, int32_t dtype, const void* logits,
                                            int64_t ld, int64_t n_tok, int64_t V, const int32_t* target,
                                            const uint8_t* mask, float** slot) {
    return old_cache_record(true, stream, c, dtype, logits, ld, n_tok, V, target, mask, slot);
}

// Inner epochs without a shuffle visit the chunks in the same order again:
// the records are replayed from call 0.
extern "C" int grpo_old_cache_rewind(grpo_old_cache* c) {
    if (!c || !c->off || c->n_calls < 1) return fail(GRPO_EINVAL, "grpo_old_cache_rewind: uninitialised cache");
    if (c->recorded != c->n_calls || c->replayed != c->n_calls)
        return fail(GRPO_ESTATE, "grpo_old_cache_rewind: needs a complete recorded and replayed walk");
    c->replayed = 0;
    return ok();
}

extern "C" int grpo_old_cache_replay(grpo_old_cache* c, int64_t n_tok, const float** old_logp) {
    if (!c || !c->off || !old_logp) return fail(GRPO_EINVAL, "grpo_old_cache_replay: bad arguments");
    const int64_t k = c->replayed;
    if (k >= c->recorded)
        return fail(GRPO_ESTATE, "grpo_old_cache_replay: call %lld was not recorded", (long long)k);
    const int64_t have = c->off[k + 1] - c->off[k];
    if (have != n_tok)
        return fail(GRPO_EINVAL, "grpo_old_cache_replay: call %lld has %lld tokens, record has %lld (walks diverged)",
                    (long long)k, (long long)n_tok, (long long)have);
    *old_logp = c->buf ? c->buf + c->off[k] : nullptr;
    c->replayed = k + 1;
    return ok();
}

extern "C" int grpo_probe_init(grpo_probe* p, double bound, double max_fraction) {
    if (!p || !(bound >= 0.0) || !(max_fraction >= 0.0 && max_fraction <= 1.0))
        return fail(GRPO_EINVAL, "grpo_probe_init: need bound >= 0 and 0 <= max_fraction <= 1");
    p->bound = bound;
    p->max_fraction = max_fraction;
    p->done = 0;
    p->passed = 0;
    return ok();
}

extern "C" int grpo_probe_finish(grpo_probe* p, const grpo_probe_stats* s, int32_t* passed) {
    if (!p || !s || !passed) return fail(GRPO_EINVAL, "grpo_probe_finish: NULL argument");
    if (p->done) return fail(GRPO_ESTATE, "grpo_probe_finish: the probe runs once per run");
    p->done = 1;
    p->passed = (double)s->n_moved <= p->max_fraction * (double)s->n_valid ? 1 : 0;
    *passed = p->passed;
    return ok();
}
