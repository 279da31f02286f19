// Per-token clipped-surrogate arithmetic shared by the fused loss kernel and
// the LM-head kernels (device code).
//
// [P1] "pi_old must be frozen across the window": ratio = exp(logp - old) and
// an epsilon clip; the loss is l = -min(rho*A, clip(rho, 1-eps_low, 1+eps_high)*A)
// and its gradient with respect to logp is -A*rho where the unclipped branch is
// the smaller one (both edges inclusive), 0 where the clip binds.
// [P1] "The hard part: deferred normalization": the gradient carries the
// per-token factor s = scale (/ max(N, 1) when N is given on the device).
// [P3] section 5: the entropy and KL losses are aggregated like the policy
// loss, so they carry the same factor s (times the row's aggregation weight).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "grpo.h"

namespace grpo_dev {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

struct Surrogate {
    float loss;     // l_t
    float kl;       // KL estimate (0 without a reference)
    float coef;     // dlogits_v = coef * (p_v - [v == y]) + entropy part
    bool clipped;   // policy-gradient part removed by the clip
    bool bad;       // non-finite log-prob, loss, entropy or KL
};

// Extra objective terms of a call (0 / NULL when unused).
struct Terms {
    const float* row_weight;   // per-row aggregation factor, NULL = 1
    const float* ref_logp;     // reference log-probs, NULL = no KL
    float ent_coef;
    float kl_coef;
    int kl_type;
};

// The per-token gradient factor: scale, divided by max(*denom, 1) when set.
__device__ __forceinline__ float step_scale(float scale, const int64_t* denom) {
    if (!denom) return scale;
    const int64_t n = *denom;
    return (float)((double)scale / (double)(n > 1 ? n : 1));
}

// s of a token of row `row` (a row outside [0, n_rows) gives NaN).
__device__ __forceinline__ float token_factor(float s0, const float* row_weight, int32_t row, int64_t n_rows) {
    if (!row_weight) return s0;
    return (uint32_t)row < (uint64_t)n_rows ? s0 * row_weight[row] : __builtin_nanf("");
}

// KL estimate against the reference and its derivative in logp, d = ref - logp:
// k1 = -d; k2 = d^2/2; k3 = e^d - d - 1 (as expm1(d) - d, no cancellation of
// the leading 1).
__device__ __forceinline__ void kl_term(float logp, float ref, int type, float& kl, float& dkl) {
    const float d = ref - logp;
    if (type == GRPO_KL_K1) {
        kl = -d;
        dkl = 1.0f;
    } else if (type == GRPO_KL_K2) {
        kl = 0.5f * d * d;
        dkl = -d;
    } else {
        const float em = expm1f(d);
        kl = em - d;
        dkl = -em;
    }
}

__device__ __forceinline__ Surrogate surrogate(float logp, float H, float old_logp, float A, float eps_low,
                                               float eps_high, float s, const Terms& x, int64_t t) {
    const float rho = expf(logp - old_logp);
    const float lo = 1.0f - eps_low, hi = 1.0f + eps_high;
    const float s1 = rho * A;
    const float s2 = fminf(fmaxf(rho, lo), hi) * A;
    Surrogate r;
    r.loss = -fminf(s1, s2);
    r.clipped = (A > 0.0f && rho > hi) || (A < 0.0f && rho < lo);
    r.coef = r.clipped ? 0.0f : s * A * rho;
    r.kl = 0.0f;
    if (x.ref_logp) {
        float dkl;
        kl_term(logp, x.ref_logp[t], x.kl_type, r.kl, dkl);
        if (x.kl_coef != 0.0f) r.coef -= s * x.kl_coef * dkl;
    }
    r.bad = !(isfinite(logp) && isfinite(r.loss) && isfinite(H) && isfinite(r.kl));
    return r;
}

}  // namespace grpo_dev
