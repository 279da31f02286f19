// Internal helpers shared by the host and device translation units of libgrpo.
#pragma once

#include <cstdarg>
#include <cstdint>

#include "grpo.h"

namespace grpo {

// Records a printf-style message for grpo_last_error() and returns `code`.
int fail(int code, const char* fmt, ...);
// Clears the thread's last error and returns GRPO_OK.
int ok();

// The pieces of a token's objective factor and extra terms that the row
// statistics need: s_r = scale (/ max(*denom, 1)) (* row_weight[r]); a row's
// objective share is s_r * (sum l - ent_coef * sum H + kl_coef * sum KL).
struct ObjTerms {
    float scale;
    const int64_t* denom;
    const float* row_weight;
    float ent_coef;
    float kl_coef;
};

// Enqueues the row-stats and chunk-stats reductions of one chunk on `stream`
// (a hipStream_t): per-token loss / entropy / KL (NULL = 0) / flags ->
// row_stats[n_rows] and chunk_stats[1], fixed reduction order.
int launch_stats(void* stream, const float* loss_tok, const float* entropy, const float* kl_tok,
                 const uint8_t* flags, const int64_t* row_off, int64_t n_rows, int64_t n_tok, const ObjTerms& obj,
                 grpo_stats* row_stats, grpo_stats* chunk_stats);

// Host checks of the extra-term arguments shared by the two loss entry points.
int check_terms(const char* who, int64_t n_tok, const float* ref_logp, const float* kl_tok, float ent_coef,
                float kl_coef, int32_t kl_type);

}  // namespace grpo
