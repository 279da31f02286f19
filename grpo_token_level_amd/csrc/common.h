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

// Enqueues the row-stats and chunk-stats reductions of one chunk on `stream`
// (a hipStream_t): per-token loss / entropy / flags -> row_stats[n_rows] and
// chunk_stats[1], fixed reduction order.
int launch_stats(void* stream, const float* loss_tok, const float* entropy, const uint8_t* flags,
                 const int64_t* row_off, int64_t n_rows, int64_t n_tok, grpo_stats* row_stats,
                 grpo_stats* chunk_stats);

}  // namespace grpo
