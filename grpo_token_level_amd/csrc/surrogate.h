// Per-token clipped-surrogate arithmetic shared by the fused loss kernel and
// the LM-head kernels (device code).
//
// [P1] "pi_old must be frozen across the window": ratio = exp(logp - old) and
// an epsilon clip; the loss is l = -min(rho*A, clip(rho, 1-eps_low, 1+eps_high)*A)
// and its gradient with respect to logp is -A*rho where the unclipped branch is
// the smaller one (both edges inclusive), 0 where the clip binds.
// [P1] "The hard part: deferred normalization": the gradient carries the
// per-token factor s = scale (/ max(N, 1) when N is given on the device).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace grpo_dev {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

struct Surrogate {
    float loss;     // l_t
    float coef;     // d(s * l_t)/d logp_t negated: dlogits_v = coef * (p_v - [v == y])
    bool clipped;   // gradient removed by the clip
    bool bad;       // non-finite log-prob, loss or entropy
};

// The per-token gradient factor: scale, divided by max(*denom, 1) when set.
__device__ __forceinline__ float step_scale(float scale, const int64_t* denom) {
    if (!denom) return scale;
    const int64_t n = *denom;
    return (float)((double)scale / (double)(n > 1 ? n : 1));
}

__device__ __forceinline__ Surrogate surrogate(float logp, float H, float old_logp, float A, float eps_low,
                                               float eps_high, float s) {
    const float rho = expf(logp - old_logp);
    const float lo = 1.0f - eps_low, hi = 1.0f + eps_high;
    const float s1 = rho * A;
    const float s2 = fminf(fmaxf(rho, lo), hi) * A;
    Surrogate r;
    r.loss = -fminf(s1, s2);
    r.clipped = (A > 0.0f && rho > hi) || (A < 0.0f && rho < lo);
    r.coef = r.clipped ? 0.0f : s * A * rho;
    r.bad = !(isfinite(logp) && isfinite(r.loss) && isfinite(H));
    return r;
}

}  // namespace grpo_dev
