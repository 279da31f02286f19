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

}  // namespace grpo
