/*
 * grpo.h -- C ABI of libgrpo: the token-level GRPO policy-loss hot path on
 * AMD MI355X (gfx950).
 *
 * Sources (cited by title and section):
 *   [P1] "Sizing mini-batches and micro-batches" (cosmos-framework post-training
 *        how-to on batching)
 *   [P2] "03 Data Protocol and Batch Lifecycle" (verl source reading)
 *   [P3] "22 - mini-batch, micro-batch and dynamic batch size" (verl article)
 *   [P4] "How a context-compaction step fits a variable number of rows into
 *        one batch" (NeMo-RL explainer)
 *
 * Conventions
 *   - Every call returns a status: GRPO_OK (0) or a negative GRPO_E* code.  A
 *     readable message for the last failure on the calling thread is in
 *     grpo_last_error() (static storage, valid until the thread's next call).
 *   - Host functions ("host") are pure and re-entrant, read and write host
 *     memory only, never allocate, and write their outputs only on GRPO_OK
 *     (GRPO_ECAPACITY writes back the capacity that is needed).
 *   - Device functions ("device") take a hipStream_t as void*, enqueue kernels
 *     on it and return without synchronising.  All their pointers are device
 *     pointers owned by the caller; the library allocates no memory.  Arguments
 *     are checked on the host before any launch; a launch failure returns
 *     GRPO_EDEVICE.  Device-side data errors (a target outside [0, V), a token
 *     whose row index is outside [0, n_rows)) never read out of bounds: the
 *     token is reported non-finite instead.
 *   - No C++ exception crosses this boundary.
 */
#ifndef GRPO_H
#define GRPO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */
#define GRPO_OK          0
#define GRPO_EINVAL     (-1)  /* malformed arguments */
#define GRPO_EDIVISIBLE (-2)  /* a batch level does not divide the one above ([P1] "The config surface") */
#define GRPO_ETOOLONG   (-3)  /* a row exceeds the micro-batch token budget ([P3] section 3) */
#define GRPO_ECOUNT     (-4)  /* a step does not hold the configured rollouts ([P4] opening paragraphs) */
#define GRPO_ENONFINITE (-5)  /* a chunk's loss is not finite: window discarded ([P1] "The poisoned-window countdown") */
#define GRPO_ESKIPPED   (-6)  /* the call was swallowed by the countdown */
#define GRPO_ECAPACITY  (-7)  /* an output buffer is too small; the needed size was written back */
#define GRPO_EDEVICE    (-8)  /* a HIP launch or runtime call failed */
#define GRPO_ESTATE     (-9)  /* accumulator misuse: a completed window was not finalized */

typedef enum grpo_dtype { GRPO_F32 = 0, GRPO_BF16 = 1 } grpo_dtype;

/* Per-token KL estimators against a reference policy, d = ref_logp - logp
 * (the pages name a KL loss but no estimator): k1 = -d, k2 = d^2/2,
 * k3 = e^d - d - 1 (non-negative); no clamp. */
#define GRPO_KL_K1 1
#define GRPO_KL_K2 2
#define GRPO_KL_K3 3

/* Loss-aggregation modes ([P3] section 5: token-mean over the global valid
 * token count N, sequence-level modes over the global batch size B):
 *   token-mean           L = sum_t l_t / N
 *   seq-mean-token-sum   L = sum_r sum_{t in r} l_t / B
 *   seq-mean-token-mean  L = sum_r (sum_{t in r} l_t / L_r) / B
 * with L_r the valid tokens of row r and B the rows holding a valid token. */
#define GRPO_AGG_TOKEN_MEAN 0
#define GRPO_AGG_SEQ_MEAN_TOKEN_SUM 1
#define GRPO_AGG_SEQ_MEAN_TOKEN_MEAN 2

/* Sums over a row or a chunk.  [P1] "Metric roll-up: token-weighted, not
 * averaged": losses are carried as sums with their token counts so that the
 * step loss is sum(loss_sum) / sum(n_valid); counts sum.  n_valid is the
 * chunk's divisor ([P1] "The hard part: deferred normalization").
 * n_valid_rows counts rows holding at least one valid token ([P4] "What it
 * costs": row counts can exceed rollouts under compaction; pads never count). */
typedef struct grpo_stats {
    double  loss_sum;      /* sum over valid tokens of the per-token loss */
    double  entropy_sum;   /* sum over valid tokens of the entropy (nats) */
    double  kl_sum;        /* sum over valid tokens of the KL estimate (0 without a reference) */
    double  obj_sum;       /* sum over valid tokens of s_t (l_t - ent_coef H_t + kl_coef KL_t): the
                              objective whose gradient the chunk wrote (s_t = the token's factor) */
    int64_t n_valid;       /* valid (mask = 1) tokens */
    int64_t n_clipped;     /* valid tokens whose gradient the clip removed */
    int64_t n_nonfinite;   /* valid tokens with a non-finite log-prob, loss or entropy */
    int64_t n_valid_rows;  /* rows with n_valid > 0 */
} grpo_stats;

const char* grpo_last_error(void);
const char* grpo_version(void);

/* ================================================================== plans */

/* host.  Fixed mini/micro plan.  [P1] "The config surface" and "A worked
 * example": batch is a positive multiple of group_size (else EINVAL);
 * mini = 0 means the whole batch and micro = 0 one chunk per mini-batch;
 * n_mini = batch / mini_rows and n_micro = mini_rows / micro_rows, each
 * division exact (else EDIVISIBLE).  32/16/8 -> 2 x 2; 0/0 -> 1 x 1.
 * Outputs are single int64 values. */
int grpo_plan_fixed(int64_t batch, int64_t group_size, int64_t mini, int64_t micro,
                    int64_t* n_mini, int64_t* n_micro, int64_t* mini_rows, int64_t* micro_rows);

/* host.  Rows [row_begin, row_end) of chunk (i_mini, j_micro) of a fixed plan:
 * contiguous, unshuffled slices in collected-batch order ([P1] "The core
 * idea": the driver passes indices only).  EINVAL for an index out of range. */
int grpo_plan_chunk(int64_t batch, int64_t mini_rows, int64_t micro_rows,
                    int64_t i_mini, int64_t j_micro, int64_t* row_begin, int64_t* row_end);

/* host.  Inner epochs over one collected batch with an optional seeded
 * shuffle ([P3] section 1: each update gets the mini-batch size, the number
 * of epochs and a shuffle flag with a data-loader seed, and the iterator
 * yields the mini-batches again each epoch; [P1] "What's not done", item 2:
 * inner epochs reuse the frozen pi_old of the ahead pass unchanged).  The
 * levels are sized as grpo_plan_fixed (same errors); mu >= 1 (EINVAL).
 * perm[mu * batch]: epoch e visits rows perm[e*batch .. e*batch + batch) in
 * order -- the identity without shuffle, else the Fisher-Yates permutation
 * (for i = batch-1 down to 1 swap items i and draw mod (i+1)) driven by one
 * splitmix64 stream seeded with `seed` (Steele, Lea and Flood 2014) consumed
 * epoch after epoch.  Chunk (e, i, j) is rows
 * perm[e*batch + i*mini_rows + j*micro_rows ..  + micro_rows). */
int grpo_plan_epochs(int64_t batch, int64_t group_size, int64_t mini, int64_t micro, int64_t mu, int32_t shuffle,
                     uint64_t seed, int64_t* n_mini, int64_t* n_micro, int64_t* mini_rows, int64_t* micro_rows,
                     int64_t* perm);

/* host.  Token-budget dynamic packing ([P3] section 3).  len[n_rows] are row
 * token counts (>= 0).  A row longer than token_budget -> ETOOLONG.  Boxes
 * start at max(1, ceil(sum(len) / budget)); workload w = proxy_div*L + L*L;
 * rows are placed by decreasing w (ties: lower index first) into the box with
 * the least workload so far (ties: lower box) among those that still fit; if
 * a row fits nowhere, one more box is added and packing restarts.  Rows keep
 * their original order inside a box.
 * Outputs: *n_bins; bin_off[n_bins + 1] offsets into order; order[n_rows]
 * (packed position -> original row); restore[n_rows] (original row -> packed
 * position).  bin_off must hold cap_bins + 1 entries: if the packing needs
 * more boxes, ECAPACITY is returned with *n_bins set to the number needed.
 * n_rows = 0 gives n_bins = 0. */
int grpo_plan_dynamic(const int64_t* len, int64_t n_rows, int64_t token_budget, int64_t proxy_div,
                      int64_t cap_bins, int64_t* n_bins, int64_t* bin_off,
                      int64_t* order, int64_t* restore);

/* host.  Context-compaction rows ([P4] figure and opening paragraphs).
 * rows_per_rollout[n_rollouts] (each >= 1, else EINVAL): segment rows per
 * rollout, rollouts grouped G at a time.  n_groups * group_size must equal
 * expected_rollouts and so must n_rollouts (else ECOUNT: the step raises
 * unless it holds exactly the configured rollouts).  dynamic != 0 -> EINVAL
 * (compaction runs with fixed batching only, [P4] "What it costs").
 * Per group: its real rows rollout-major in segment order, then
 * (-real) mod Q pad rows, each copying the group's first real row.
 * Outputs per padded row (capacity cap_rows, else ECAPACITY with *n_rows set):
 * row_rollout (-1 for a pad), row_seg (segment index, -1 for a pad), row_src
 * (input row, numbering all segment rows rollout-major), row_is_pad; and
 * group_pad[n_groups]. */
int grpo_plan_compaction(const int32_t* rows_per_rollout, int64_t n_rollouts, int64_t n_groups,
                         int64_t group_size, int64_t Q, int64_t expected_rollouts, int32_t dynamic,
                         int64_t cap_rows, int64_t* n_rows, int32_t* row_rollout, int32_t* row_seg,
                         int32_t* row_src, uint8_t* row_is_pad, int32_t* group_pad);

/* host.  Prefix offsets of rows laid end to end: row_off[0] = 0,
 * row_off[k+1] = row_off[k] + len[order ? order[k] : k].  Used for the packed
 * (variable-length) layout, [P3] section 3. */
int grpo_row_offsets(const int64_t* len, const int64_t* order, int64_t n_rows, int64_t* row_off);

/* ================================================================== plan trace */

/* One plan, as the chunks a training walk visits, for the trace dump.
 * [P2] "Trace Entry" lists what a minimal trace records per row of a group:
 * stage, field, producer and consumer, shape or nested length, dtype and
 * device, valid length, response_mask.sum(), uid and trajectory key, the
 * global step, and is_padding.  All pointers are host pointers. */
typedef struct grpo_trace_plan {
    int32_t struct_size;        /* = sizeof(grpo_trace_plan) */
    int32_t dtype;              /* grpo_dtype of the logits the chunks read */
    const char* stage;          /* label of the plan ([A-Za-z0-9_.-], 1..63 characters) */
    int64_t n_rows;             /* rows of the collected batch (after compaction: segment and pad rows) */
    int64_t T;                  /* padded positions per row, or 0 for a packed (nested) layout */
    int64_t V;                  /* vocabulary: a row's logits are [len x V] */
    const int64_t* row_len;     /* [n_rows] positions of the row (its nested length; <= T when padded) */
    const int64_t* row_valid;   /* [n_rows] response_mask.sum() of the row (<= row_len) */
    const int32_t* row_uid;     /* [n_rows] group (prompt uid) of the row, >= 0 */
    const int32_t* row_traj;    /* [n_rows] rollout (trajectory key) of the row; >= 0, or -1 on a pad row */
    const int32_t* row_seg;     /* NULL or [n_rows] segment index within the rollout (compaction); -1 on a pad */
    const uint8_t* row_is_pad;  /* NULL (no pads) or [n_rows] 1 = padding row */
    int64_t n_calls;            /* training calls (chunks) in visiting order */
    const int64_t* call_off;    /* [n_calls + 1] offsets into call_rows, non-decreasing from 0 */
    const int64_t* call_rows;   /* rows of each call, in the order the chunk lays them out */
    const int64_t* call_step;   /* [n_calls] optimizer step (global mini-batch index) of each call */
} grpo_trace_plan;

/* host.  Writes the trace of a plan as JSON lines into buf: for every call k,
 * one object per row it holds,
 *   {"stage", "call", "step", "pos", "row", "uid", "traj", "seg", "field",
 *    "producer", "consumer", "shape", "dtype", "device", "len", "valid",
 *    "is_padding"}
 * ("pos" = the row's place in the chunk, "shape" = [len, V] nested or [T, V]
 * padded, "field" = "logits", producer "policy forward", consumer
 * "grpo_loss_fwd_bwd"; "traj" and "seg" are null on a pad row that names no
 * rollout), then one summary object per call
 *   {"stage", "call", "step", "summary": true, "rows", "pads", "positions",
 *    "valid"}.
 * Each line ends with '\n' and the text with a terminating NUL.  Checks: rows
 * in range, lengths and counts consistent (valid <= len, len <= T when
 * padded), EINVAL otherwise.  *need receives the bytes the text takes
 * (NUL included); if cap < *need the result is ECAPACITY and buf is untouched. */
int grpo_plan_trace(const grpo_trace_plan* plan, char* buf, size_t cap, size_t* need);


/* ============================================================== advantage */

/* host.  One advantage per rollout, relative to its group of group_size
 * consecutive rollouts ([P2] "Field Lineage", reward/log-prob/advantage;
 * [P4] "Why the row count does not change the math", item 2).  The pages
 * give no formula; this is A = (r - mean) / (std + eps) with the unbiased
 * (G - 1) standard deviation, or A = r - mean when norm_by_std = 0; a group
 * of one rollout has A = 0.  Accumulates in double.  n_rollouts must be a
 * multiple of group_size (EINVAL). */
int grpo_group_advantage(const float* reward, int64_t n_rollouts, int64_t group_size,
                         float eps, int32_t norm_by_std, float* adv_rollout);

/* host.  adv_row[r] = adv_rollout[row_rollout[r]], or 0 for a pad
 * (row_rollout < 0) ([P4] item 2: copied to all rows of the rollout, pads 0).
 * A row_rollout >= n_rollouts is EINVAL. */
int grpo_rows_advantage(const float* adv_rollout, int64_t n_rollouts,
                        const int32_t* row_rollout, int64_t n_rows, float* adv_row);

/* ============================================================ device path */

/* device.  *n_valid (device int64) = number of non-zero bytes of
 * mask[n_tok]: N, the valid tokens of a step ([P1] "The hard part: deferred
 * normalization"; [P3] section 5: the token mean divides by the summed loss
 * mask; [P4] item 1: padding counts 0).  Overwrites *n_valid. */
int grpo_count_valid(void* stream, const uint8_t* mask, int64_t n_tok, int64_t* n_valid);

/* device.  *n_seq (device int64) = number of rows r holding at least one
 * mask-1 token in [row_off[r], row_off[r+1]): B, the sequence count of the
 * seq-level aggregation modes ([P3] section 5: they divide by the global
 * batch size; masked padding rows, [P4] "Why the row count does not change
 * the math", do not count).  row_off: device int64 [n_rows + 1],
 * non-decreasing, within [0, n_tok].  Overwrites *n_seq. */
int grpo_count_rows(void* stream, const uint8_t* mask, const int64_t* row_off, int64_t n_rows, int64_t n_tok,
                    int64_t* n_seq);

/* device.  Per-row gradient factors of an aggregation mode (GRPO_AGG_*),
 * for grpo_loss_args.row_weight: token-mean 1 (the 1/N goes in scale or
 * denom); seq-mean-token-sum 1/max(B, 1); seq-mean-token-mean
 * 1/(max(B, 1) * L_r), 0 for a row without valid tokens.  B = *n_seq (device
 * int64, grpo_count_rows over the whole mini-batch); L_r counted from mask
 * over [row_off[r], row_off[r+1]).  w_row: device float [n_rows]. */
int grpo_row_weights(void* stream, const uint8_t* mask, const int64_t* row_off, int64_t n_rows, int64_t n_tok,
                     int32_t mode, const int64_t* n_seq, float* w_row);

/* device.  Chunk resolution from indices ([P1] "The core idea": the driver
 * passes indices only): tok_src[t] = src_row_off[rows[r]] + (t - dst_row_off[r])
 * for dst_row_off[r] <= t < dst_row_off[r+1], i.e. the batch token index of
 * every token of a chunk made of batch rows `rows` laid end to end.
 * src_row_off: device int64 [n_src_rows + 1] (batch layout); rows: device
 * int64 [n_rows] in [0, n_src_rows); dst_row_off: device int64 [n_rows + 1],
 * dst_row_off[r+1] - dst_row_off[r] = that row's length.  A row index out of
 * range gives -1 for its tokens. */
int grpo_chunk_tok_src(void* stream, const int64_t* src_row_off, int64_t n_src_rows, const int64_t* rows,
                       int64_t n_rows, const int64_t* dst_row_off, int64_t n_tok, int64_t* tok_src);

/* device.  dst[k] = src[idx[k]] for k < n, elements of elem_bytes (1, 2, 4
 * or 8) bytes: per-row or per-token values of a chunk whose rows sit anywhere
 * in the batch (advantages, aggregation weights, cached pi_old).  idx[k]
 * outside [0, n_src) writes zero bytes. */
int grpo_gather(void* stream, const void* src, int64_t n_src, const int64_t* idx, int64_t n, int64_t elem_bytes,
                void* dst);

/* device.  tok_row[t] = the row r with row_off[r] <= t < row_off[r+1]
 * (row_off: device int64 [n_rows + 1], non-decreasing), or -1 if none. */
int grpo_tok_row(void* stream, const int64_t* row_off, int64_t n_rows, int64_t n_tok, int32_t* tok_row);

/* device.  Ahead pass: per-token log-prob, logsumexp and entropy, forward
 * only ([P1] "pi_old must be frozen across the window -- the ahead pass";
 * [P2] "Field Lineage": the normal-mode recompute yields old log-probs and
 * entropy).  logits: dtype, token t's row at logits + t*ld (ld >= V elements),
 * [n_tok x V].  target int32 [n_tok]; mask uint8 [n_tok].  Outputs float
 * [n_tok]: logp = z_y - lse, lse = log sum exp z, entropy = -sum p log p; 0 at
 * mask-0 tokens.  lse and entropy may be NULL.  Reads V elements per valid
 * token once and writes nothing V-sized. */
int grpo_logprob_fwd(void* stream, int32_t dtype, const void* logits, int64_t ld, int64_t n_tok,
                     int64_t V, const int32_t* target, const uint8_t* mask,
                     float* logp, float* lse, float* entropy);

/* device.  grpo_logprob_fwd whose sums run in the lane partition and order of
 * grpo_loss_fwd_bwd, so that logp, lse and entropy equal the fused loss's bit
 * for bit on the same logits: a pi_old recorded by this pass at unchanged
 * weights gives the ratio exactly 1 in the first training call ([P1] "pi_old
 * must be frozen across the window": the ratio of the current policy to its
 * detached copy).  It takes the fused loss's kernel shapes: the row held on
 * chip (registers, then LDS, then for bf16 a part re-read) up to 262 144 bf16
 * or 114 688 fp32 logits, and rows off 16-byte alignment on chip as the fused
 * loss does when its dlogits rows share their phase (in place).  Where the
 * fused loss streams (longer rows, or rows whose dlogits rows are off 16-byte
 * alignment in another phase or dtype, such as fp32 logits into bf16 dlogits
 * with V not a multiple of 8) the two agree to float32 summation order only.  Slower than
 * grpo_logprob_fwd for rows past 1024 vectors (the row on chip instead of
 * streamed: 5.7 against 6.6 TB/s at V = 151 936 bf16).  Arguments, outputs and
 * errors as grpo_logprob_fwd. */
int grpo_logprob_fwd_paired(void* stream, int32_t dtype, const void* logits, int64_t ld, int64_t n_tok,
                            int64_t V, const int32_t* target, const uint8_t* mask, float* logp, float* lse,
                            float* entropy);

/* grpo_loss_args.flags: leave the row and chunk reductions to a later
 * grpo_loss_stats call (row_off, row_stats and chunk_stats are then not read
 * and may be NULL), so that one reduction can serve several chunks. */
#define GRPO_LOSS_DEFER_STATS 1

/* Arguments of grpo_loss_fwd_bwd (all pointers are device pointers). */
typedef struct grpo_loss_args {
    int32_t struct_size;        /* = sizeof(grpo_loss_args) */
    int32_t in_dtype;           /* grpo_dtype of logits */
    int32_t out_dtype;          /* grpo_dtype of dlogits */
    int32_t reserved0;          /* 0 */
    const void* logits;         /* token t's V logits at logits + t*ld */
    int64_t ld;                 /* row stride in elements, >= V */
    int64_t n_tok;              /* token rows in this chunk (>= 0) */
    int64_t V;                  /* vocabulary (>= 1) */
    const int32_t* target;      /* [n_tok] next-token ids */
    const uint8_t* mask;        /* [n_tok] 1 = policy token ([P2] response mask) */
    const float* old_logp;      /* [n_tok] pi_old log-probs (ignored where mask = 0) */
    const int32_t* tok_row;     /* [n_tok] row of each token within the chunk */
    const float* adv_row;       /* [n_rows] advantage per row (0 for pads) */
    const int64_t* row_off;     /* [n_rows + 1] token offsets of the rows (row stats) */
    int64_t n_rows;             /* rows in this chunk (>= 1 when n_tok > 0) */
    float eps_low, eps_high;    /* clip band [1 - eps_low, 1 + eps_high] */
    float scale;                /* gradient factor: 1/max(N,1) for a known step N, 1 to defer */
    int32_t flags;              /* 0, or GRPO_LOSS_DEFER_STATS */
    const int64_t* denom;       /* NULL, or device int64: coef is further divided by max(*denom, 1) */
    void* dlogits;              /* out_dtype, token t at dlogits + t*ld_out; may equal logits
                                   when the dtypes and strides match; NULL = no gradient */
    int64_t ld_out;             /* row stride of dlogits in elements, >= V */
    float* logp;                /* [n_tok] required */
    float* lse;                 /* [n_tok] or NULL */
    float* entropy;             /* [n_tok] required */
    float* loss_tok;            /* [n_tok] required: per-token surrogate loss l_t */
    uint8_t* tok_flags;         /* [n_tok] required: bit0 valid, bit1 clipped, bit2 non-finite */
    grpo_stats* row_stats;      /* [n_rows] required */
    grpo_stats* chunk_stats;    /* [1] required: rows summed in row order */
    /* Extra terms ([P3] section 5: the policy, entropy and KL losses share one aggregation). */
    const float* row_weight;    /* NULL (all 1) or [n_rows]: per-row factor of the token's gradient */
    const float* ref_logp;      /* NULL or [n_tok]: reference-policy log-probs (KL term) */
    float* kl_tok;              /* [n_tok], required when ref_logp is set: per-token KL estimate */
    float ent_coef;             /* entropy bonus: the token's objective gains -ent_coef * H */
    float kl_coef;              /* KL weight: the token's objective gains +kl_coef * KL (needs ref_logp) */
    int32_t kl_type;            /* GRPO_KL_K1 / K2 / K3 (read when ref_logp is set) */
    int32_t reserved2;          /* 0 */
    /* Chunks of batch rows in any order (shuffled epochs) without copies. */
    const int64_t* tok_src;     /* NULL, or [n_tok] (grpo_chunk_tok_src): token t's logits, dlogits, target,
                                   mask, old_logp and ref_logp are those of batch token tok_src[t]; the
                                   per-token outputs, tok_row, adv_row, row_weight, row_off and the stats stay
                                   chunk-local.  Entries must be distinct when dlogits is written. */
    int64_t n_src;              /* batch token rows behind logits / dlogits / the per-token inputs when
                                   tok_src is set (a tok_src[t] outside [0, n_src) makes token t non-finite,
                                   with no V-sized access) */
} grpo_loss_args;

/* device.  Fused forward and backward of the token-level GRPO loss over one
 * micro-batch chunk.  Per valid token (mask = 1), reading the token's logits
 * once:
 *   lse = log sum_v exp z_v, logp = z_y - lse, H = -sum_v p_v log p_v,
 *   rho = exp(logp - old_logp), A = adv_row[tok_row[t]],
 *   l = -min(rho*A, clip(rho, 1-eps_low, 1+eps_high)*A),
 *   g = 0 if (A > 0 and rho > 1+eps_high) or (A < 0 and rho < 1-eps_low) else 1,
 *   s = scale (/ max(*denom, 1) when denom is set) (* row_weight[row] when set),
 *   KL, dKL/dlogp from ref_logp (GRPO_KL_*; 0 without ref_logp),
 *   coef = s * (A * rho * g - kl_coef * dKL/dlogp),
 *   dlogits_v = coef * (p_v - [v == y]) + ent_coef * s * p_v * (z_v - lse + H),
 * the gradient of the token's objective s * (l - ent_coef * H + kl_coef * KL)
 * (with ent_coef = kl_coef = 0 and no row weights: coef * (p_v - [v == y])).
 * Mask-0 tokens: outputs 0 and a zero dlogits row.
 * [P1] "The hard part: deferred normalization" (token mean over N; chunk
 * gradients add up to the step gradient, so scale = 1/N on every chunk makes
 * the chunked gradient equal the un-chunked one token for token);
 * [P1] "pi_old must be frozen" (ratio and epsilon clip);
 * [P2] "Field Lineage" (response mask, advantage broadcast over the row);
 * [P4] "Why the row count does not change the math" items 1-2 (pads: no
 * valid tokens, advantage 0).
 * Then row_stats[r] sums tokens row_off[r] .. row_off[r+1]-1 and
 * chunk_stats sums the rows in row order; the reductions have a fixed order,
 * so results are bit-for-bit reproducible and a row's stats do not depend on
 * where the row sits in the chunk. */
int grpo_loss_fwd_bwd(void* stream, const grpo_loss_args* args);

/* device.  The row and chunk reductions of grpo_loss_fwd_bwd on their own,
 * over the per-token outputs (loss_tok, entropy, kl_tok when ref_logp is set,
 * tok_flags) of args->n_tok tokens in args->n_rows rows (row_off), with the
 * gradient factor fields (scale, denom, row_weight, ent_coef, kl_coef) that
 * the tokens were computed with: row_stats[r] and chunk_stats exactly as
 * grpo_loss_fwd_bwd would write them for a chunk of those rows.  Use after
 * calls made with GRPO_LOSS_DEFER_STATS: the rows of several chunks of one
 * optimizer step can be reduced by one call ([P1] "Metric roll-up": rows
 * carry sums and counts, so a chunk's stats are the sum of its rows',
 * grpo_stats_sum).  The other fields of args are not read. */
int grpo_loss_stats(void* stream, const grpo_loss_args* args);

/* host.  out = the sum of rows[0 .. n) added in index order (float64 sums,
 * integer counts): a chunk's stats from its rows' (n >= 0; n = 0 gives
 * zeros). */
int grpo_stats_sum(const grpo_stats* rows, int64_t n, grpo_stats* out);

/* ========================================================= LM-head variant */

/* device.  dst[c * ld_dst + r] = src[r * ld_src + c] for a bf16 matrix of
 * rows x cols (the transpose).  Used once per step to give the LM-head path W^T. */
int grpo_transpose_bf16(void* stream, const void* src, int64_t rows, int64_t cols, int64_t ld_src,
                        void* dst, int64_t ld_dst);

/* The weight-gradient window: dW of several chunks as one GEMM.  [P1] "The
 * hard part: deferred normalization": the step's gradient is the sum of its
 * chunks' gradients, and dW = sum over the step's valid tokens of
 * dz_t^T h_t needs nothing else of a chunk.  A chunk called with a window
 * (GRPO_LMHEAD_DEFER_DW) appends h^T and dz^T of its valid tokens to it
 * instead of multiplying them out; grpo_lmhead_dw_flush then adds the whole
 * window's dz^T h to dW in one GEMM, whose K (the window's tokens) is long
 * enough to amortise each tile's start and end, and dW is read and written
 * once instead of once per chunk.  Plain data, caller-allocated; buf is
 * device memory, the rest host fields.  Not thread-safe: one stream of calls
 * per window. */
typedef struct grpo_lmhead_dw_window {
    void* buf;          /* device, >= grpo_lmhead_dw_window_size(cap_tok, H, V) bytes, 256-byte aligned:
                         * a fill counter, then h^T [H x cap] and dz^T [V x cap] (bf16, cap = cap_tok
                         * rounded up to 64) */
    size_t bytes;
    int64_t cap_tok;    /* tokens the window holds */
    int64_t H, V;
    int64_t reserved;   /* host: columns reserved by the calls since the last flush (each call
                         * reserves n_tok rounded up to 64; its valid tokens fill the front of that) */
} grpo_lmhead_dw_window;

/* host.  Bytes of a window of cap_tok tokens (0 for bad sizes):
 * 256 + 2 * cap * (H + V) rounded up to 256-byte parts, cap = cap_tok rounded
 * up to 64.  At V = 151 936, H = 2048: ~0.31 MB per token. */
size_t grpo_lmhead_dw_window_size(int64_t cap_tok, int64_t H, int64_t V);

/* device.  Sets up w over buf and empties it (a kernel on `stream` clears the
 * fill counter; nothing else needs to start at zero).  EINVAL for NULL or
 * misaligned buf, bad sizes or cap_tok above 2^30; ECAPACITY if bytes is
 * below grpo_lmhead_dw_window_size. */
int grpo_lmhead_dw_window_init(void* stream, grpo_lmhead_dw_window* w, void* buf, size_t bytes, int64_t cap_tok,
                               int64_t H, int64_t V);

/* device.  dW (fp32 [V x H], 16-byte aligned) += the sum over the window's
 * tokens of dz_t^T h_t (one bf16 MFMA GEMM, fp32 accumulation), then empties
 * the window.  An empty window leaves dW as it is.  Calls on the stream
 * before it must be the ones that filled the window.  EINVAL for a NULL or
 * uninitialised window or dW. */
int grpo_lmhead_dw_flush(void* stream, grpo_lmhead_dw_window* w, float* dW);

/* Arguments of grpo_lmhead_fwd_bwd (all pointers are device pointers). */
typedef struct grpo_lmhead_args {
    int32_t struct_size;        /* = sizeof(grpo_lmhead_args) */
    int32_t reserved0;          /* 0 */
    const void* h;              /* bf16 [n_tok x H] hidden states, row stride ldh (16-byte aligned) */
    int64_t ldh;                /* >= H, multiple of 8 */
    const void* W;              /* bf16 [V x H] LM-head weight, rows contiguous (16-byte aligned) */
    const void* Wt;             /* bf16 [H x V]: W transposed (grpo_transpose_bf16), 16-byte aligned */
    int64_t n_tok, H, V;        /* n_tok <= 4194240 (65535 x 64); H and V multiples of 8 */
    const int32_t* target;      /* [n_tok] */
    const uint8_t* mask;        /* [n_tok] 1 = policy token; pads and observations 0 */
    const float* old_logp;      /* [n_tok] */
    const int32_t* tok_row;     /* [n_tok] row of each token within the chunk */
    const float* adv_row;       /* [n_rows] advantage per row (0 for pads) */
    const int64_t* row_off;     /* [n_rows + 1] token offsets of the rows */
    int64_t n_rows;
    float eps_low, eps_high;    /* clip band */
    float scale;                /* gradient factor (see grpo_loss_args) */
    int32_t flags;              /* 0, or GRPO_LMHEAD_KEEP_Z and / or GRPO_LMHEAD_DEFER_DW */
    const int64_t* denom;       /* NULL or device int64 N: factor further divided by max(N, 1) */
    float* dh;                  /* fp32 [n_tok x H]: dL/dh, overwritten */
    float* dW;                  /* fp32 [V x H], 16-byte aligned: dL/dW of this chunk is ADDED (accumulate);
                                 * unused (may be NULL) with GRPO_LMHEAD_DEFER_DW */
    float* logp;                /* [n_tok] required */
    float* lse;                 /* [n_tok] or NULL */
    float* entropy;             /* [n_tok] required */
    float* loss_tok;            /* [n_tok] required */
    uint8_t* tok_flags;         /* [n_tok] required: bit0 valid, bit1 clipped, bit2 non-finite */
    grpo_stats* row_stats;      /* [n_rows] required */
    grpo_stats* chunk_stats;    /* [1] required */
    void* workspace;            /* >= grpo_lmhead_workspace_size_flags(n_tok, H, V, flags) bytes, 16-byte aligned */
    size_t workspace_bytes;
    const float* row_weight;    /* extra terms exactly as in grpo_loss_args */
    const float* ref_logp;
    float* kl_tok;
    float ent_coef;
    float kl_coef;
    int32_t kl_type;
    int32_t reserved2;
    grpo_lmhead_dw_window* dw_window;   /* host pointer, with GRPO_LMHEAD_DEFER_DW (else NULL) */
} grpo_lmhead_args;

/* grpo_lmhead_args.flags: keep the chunk's logits.  Pass 1 stores z (fp32,
 * [valid tokens x V]) in the workspace and pass 2 forms dz from it with an
 * elementwise kernel instead of a second GEMM over h W^T (same dz bits, about
 * 13 % less time at the compaction workload's sizes), at the price of holding
 * 4 * n_tok * V bytes more: the chunk's [tokens x V] logits, which the default
 * path never holds.  Not available with grpo_lmhead_fwd_bwd_noalloc. */
#define GRPO_LMHEAD_KEEP_Z 1

/* grpo_lmhead_args.flags: defer dW.  The chunk's h^T and dz^T (its valid
 * tokens, in order) go to args->dw_window instead of a dW GEMM; dW is not
 * touched until grpo_lmhead_dw_flush.  The workspace then holds neither.
 * ECAPACITY, before any launch, if the window's reserved columns plus n_tok
 * rounded up to 64 exceed its cap_tok rounded up to 64 (flush first);
 * EINVAL if the window is missing or its H, V differ from the call's, or
 * with grpo_lmhead_fwd_bwd_noalloc. */
#define GRPO_LMHEAD_DEFER_DW 2

/* host.  Workspace bytes grpo_lmhead_fwd_bwd needs for a chunk of n_tok tokens
 * without flags: per-token slice partials of the log-softmax (16 B per token
 * per 64 vocabulary columns), h^T, one vocabulary chunk (at most 65536
 * columns) of dz in two layouts (bf16), up to 16 fp32 split partials of dh and
 * the chunk's valid-token index maps.  It grows with n_tok * V / 4,
 * n_tok * 262144 and n_tok * H * 64, never with n_tok * V * 2. */
size_t grpo_lmhead_workspace_size(int64_t n_tok, int64_t H, int64_t V);

/* host.  The same for the given flags.  With GRPO_LMHEAD_KEEP_Z: plus the
 * fp32 logits (4 * n_tok * V), and dz in two layouts for up to the whole
 * vocabulary (4 * n_tok * V) in place of one 65536-column chunk.  With
 * GRPO_LMHEAD_DEFER_DW: without h^T and dz^T (they go to the window), and dz
 * (bf16) for up to the whole vocabulary (2 * n_tok * V).  0 for unknown flags
 * or bad sizes. */
size_t grpo_lmhead_workspace_size_flags(int64_t n_tok, int64_t H, int64_t V, int32_t flags);

/* device.  The fused loss of grpo_loss_fwd_bwd with the logits produced by the
 * LM head, z = h W^T, and the gradient pushed through it:
 *   per valid token the same logp / entropy / surrogate / coef as
 *   grpo_loss_fwd_bwd, dz = coef * (softmax(z) - onehot(y)),
 *   dh = dz W (overwritten), dW += dz^T h (accumulated across chunks: [P1] "The
 *   hard part: deferred normalization" -- chunk gradients add up to the step's).
 * z and dz are formed tile by tile in registers by bf16 MFMA GEMMs (fp32
 * accumulation) and never stored for the whole vocabulary (unless flags holds
 * GRPO_LMHEAD_KEEP_Z); dz feeds the two gradient GEMMs in bf16, one
 * vocabulary chunk at a time.  Masked tokens
 * (pads, [P4] figure; observations, [P2] "Field Lineage") get zero outputs and
 * contribute nothing; the GEMMs skip them: the chunk's valid tokens are listed
 * on the device first and only their rows are multiplied (the host never
 * waits for the count).  Row and chunk stats as in grpo_loss_fwd_bwd.
 * ECAPACITY if the workspace is too small; EINVAL for unknown flags. */
int grpo_lmhead_fwd_bwd(void* stream, const grpo_lmhead_args* args);

/* Bytes of the fixed device scratch behind grpo_lmhead_fwd_bwd_noalloc. */
#define GRPO_LMHEAD_NOALLOC_SCRATCH_BYTES (256u << 20)

/* device.  grpo_lmhead_fwd_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation, but its scratch lives in a fixed
 * 256 MiB array that the library holds on every GPU it runs on until the
 * process ends, so the call allocates nothing and args->workspace /
 * workspace_bytes are ignored.  The vocabulary chunk width and the dh split
 * count are chosen to fit that scratch (narrower than the workspace path may
 * use when the chunk is large, so dh and dW can differ from
 * grpo_lmhead_fwd_bwd in summation order, not in what they compute).  A chunk
 * whose narrowest plan still needs more than
 * GRPO_LMHEAD_NOALLOC_SCRATCH_BYTES (grpo_lmhead_workspace_size's per-token
 * parts grow with n_tok * V / 4 and n_tok * H) returns GRPO_ECAPACITY with
 * the size it needs.  Nothing in the scratch has to start at zero.  All calls
 * on one GPU share that GPU's scratch: calls that overlap on one GPU (two
 * streams, or two threads) race and must be serialised by the caller.
 * flags must be 0 (EINVAL for GRPO_LMHEAD_KEEP_Z: the logits do not fit the
 * scratch; EINVAL for GRPO_LMHEAD_DEFER_DW: the window is a caller buffer of
 * the workspace path). */
int grpo_lmhead_fwd_bwd_noalloc(void* stream, const grpo_lmhead_args* args);

/* ===================================================== frozen pi_old (ahead pass) */

/* host.  [P1] "pi_old must be frozen across the window -- the ahead pass":
 * with n_mini > 1 optimizer steps per collected batch, pi_old recomputed from
 * the current policy makes every ratio 1 and the clip never binds, so the
 * whole (mini, micro) product is walked once before training and pi_old is
 * recorded per chunk.  Returns 1 when that pass is needed: n_mini > 1, the
 * loss does not use the rollout's own log-probs, and the objective consumes
 * old log-probs; else 0 (n_mini = 1 always skips it). */
int32_t grpo_needs_ahead_pass(int64_t n_mini, int32_t use_rollout_logprobs, int32_t consumes_old_logprobs);

/* The pi_old records of one collected batch, keyed by call order ([P1]: both
 * walks visit the chunks in the same order, so training call k pairs with
 * ahead call k).  Plain data, caller-allocated; buf (device) and off (host)
 * are caller-owned.  Not thread-safe: one walk per cache. */
typedef struct grpo_old_cache {
    float* buf;         /* device float [capacity]: the records end to end */
    int64_t capacity;   /* floats in buf */
    int64_t* off;       /* host int64 [n_calls + 1]: record k is buf[off[k] .. off[k+1]) */
    int64_t n_calls;    /* calls in one walk */
    int64_t recorded;   /* records made */
    int64_t replayed;   /* training calls served */
} grpo_old_cache;

/* host.  n_calls >= 1, capacity >= 0, buf and off non-NULL (EINVAL). */
int grpo_old_cache_init(grpo_old_cache* c, float* buf, int64_t capacity, int64_t* off, int64_t n_calls);
/* host.  Empties the cache for the next collected batch. */
int grpo_old_cache_reset(grpo_old_cache* c);
/* device.  Records the next call: the forward-only log-prob pass
 * (grpo_logprob_fwd, same arguments) of the chunk into buf + off[k], k =
 * c->recorded; *slot (if slot is non-NULL) receives that device address.
 * ESTATE when all n_calls are recorded or a replay has begun (reset first);
 * ECAPACITY when the record does not fit in buf. */
int grpo_old_cache_record(void* stream, grpo_old_cache* c, int32_t dtype, const void* logits, int64_t ld,
                          int64_t n_tok, int64_t V, const int32_t* target, const uint8_t* mask, float** slot);
/* device.  grpo_old_cache_record with the record made by
 * grpo_logprob_fwd_paired: replayed into grpo_loss_fwd_bwd on logits that
 * have not changed since, the ratio is exactly 1 (on the rows
 * grpo_logprob_fwd_paired covers). */
int grpo_old_cache_record_paired(void* stream, grpo_old_cache* c, int32_t dtype, const void* logits, int64_t ld,
                                 int64_t n_tok, int64_t V, const int32_t* target, const uint8_t* mask,
                                 float** slot);
/* host.  After a complete walk was recorded and replayed, starts the next
 * inner epoch's replay from call 0 (same order: unshuffled epochs reuse the
 * records by call order).  ESTATE otherwise.  A shuffled epoch reads pi_old
 * per token instead: with the ahead walk in batch order, buf holds the whole
 * batch's pi_old in batch token order, and grpo_loss_args.tok_src selects it. */
int grpo_old_cache_rewind(grpo_old_cache* c);
/* host.  pi_old of the next training call: *old_logp = buf + off[k], k =
 * c->replayed (device float [n_tok], as grpo_loss_args.old_logp).  ESTATE if
 * call k was not recorded; EINVAL if n_tok differs from record k's token
 * count (the training walk diverged from the ahead walk). */
int grpo_old_cache_replay(grpo_old_cache* c, int64_t n_tok, const float** old_logp);

/* The determinism probe ([P1], same section): on the first ahead chunk of a
 * run, the chunk re-scored in training mode is compared with its record at
 * unchanged weights; the gate is on the fraction of tokens whose log-prob
 * moved past a per-token bound, under the tolerance the model declares
 * (bound, largest moved fraction); the strict default is 0.05 nats on any
 * token.  It runs once per run. */
#define GRPO_PROBE_STRICT_BOUND 0.05
#define GRPO_PROBE_STRICT_FRACTION 0.0

typedef struct grpo_probe_stats {
    int64_t n_valid;    /* mask-1 tokens compared */
    int64_t n_moved;    /* of those, |recorded - rescored| > bound (float32) or not finite */
    double max_abs;     /* largest |recorded - rescored| (infinity if one is not finite) */
} grpo_probe_stats;

/* device.  Compares two per-token log-prob arrays (device float [n_tok])
 * over mask-1 tokens into *out (device grpo_probe_stats); fixed-order
 * reduction.  Overwrites *out. */
int grpo_probe_compare(void* stream, const float* recorded, const float* rescored, const uint8_t* mask,
                       int64_t n_tok, float bound, grpo_probe_stats* out);

typedef struct grpo_probe {
    double bound;        /* per-token bound (nats) */
    double max_fraction; /* largest allowed moved fraction */
    int32_t done;        /* the probe has run */
    int32_t passed;      /* its verdict */
} grpo_probe;

/* host.  bound >= 0, 0 <= max_fraction <= 1 (EINVAL). */
int grpo_probe_init(grpo_probe* p, double bound, double max_fraction);
/* host.  Takes the verdict from a host copy of the compare's stats:
 * *passed = (n_moved <= max_fraction * n_valid).  ESTATE on a second call
 * (the probe is one-shot). */
int grpo_probe_finish(grpo_probe* p, const grpo_probe_stats* stats, int32_t* passed);

/* ============================================================ accumulator */

/* One optimizer-step window of n_micro chunks, caller-allocated, plain data.
 * [P1] "The hard part: deferred normalization": divisors add up and the
 * gradient is scaled once by 1/max(sum, 1); [P1] "Metric roll-up": the step
 * loss is sum(loss_sum)/max(sum(n_valid), 1) and counts sum; [P1] "The
 * poisoned-window countdown": a non-finite chunk at position j discards the
 * window and the next n_micro - 1 - j calls are swallowed. */
typedef struct grpo_accum grpo_accum;   /* opaque: the caller provides grpo_accum_size() bytes,
                                           aligned to 8, and grpo_accum_init prepares them */

/* host.  Bytes of one accumulator (a small constant; no pointers inside, so a
 * copy of the bytes is a copy of the state). */
size_t grpo_accum_size(void);

typedef struct grpo_step_result {
    double  loss;          /* sum(loss_sum) / max(N, 1) */
    double  entropy;       /* sum(entropy_sum) / max(N, 1) */
    double  kl;            /* sum(kl_sum) / max(N, 1) */
    double  obj_sum;       /* sum(obj_sum): the step objective when the chunks carried the
                              normalisation (global N or row weights); times grad_scale in
                              the deferred token-mean mode (scale = 1) */
    double  grad_scale;    /* 1 / max(N, 1): apply to gradients accumulated with scale = 1 */
    int64_t n_valid;       /* N */
    int64_t n_valid_rows;
    int64_t n_clipped;
} grpo_step_result;

/* host.  Prepares acc (grpo_accum_size() bytes) for windows of n_micro >= 1
 * chunks.  Every other accum call refuses (EINVAL) a buffer that was not
 * prepared. */
int grpo_accum_init(grpo_accum* acc, int64_t n_micro);
/* host.  Adds one chunk's stats (host copy).  Returns GRPO_OK, GRPO_ENONFINITE
 * (window discarded; zero your accumulated gradients), GRPO_ESKIPPED (call
 * swallowed by the countdown) or GRPO_ESTATE (finalize the completed window
 * first).  A chunk is non-finite when n_nonfinite > 0 or a sum is not finite. */
int grpo_accum_add(grpo_accum* acc, const grpo_stats* chunk);
/* host.  *stepped = 1 and *out filled when a window is complete (the window is
 * then closed); *stepped = 0 otherwise. */
int grpo_accum_finalize(grpo_accum* acc, grpo_step_result* out, int32_t* stepped);

#ifdef __cplusplus
}
#endif

#endif /* GRPO_H */
