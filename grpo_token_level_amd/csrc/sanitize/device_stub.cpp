// Stand-ins for the device entry points that the host half calls, for the
// host-only build under AddressSanitizer and UndefinedBehaviorSanitizer.
// That build has no GPU code: a call that would enqueue device work fails
// with GRPO_EDEVICE and a message instead.

#include "common.h"

extern "C" int grpo_logprob_fwd(void*, int32_t, const void*, int64_t, int64_t, int64_t, const int32_t*,
                                const uint8_t*, float*, float*, float*) {
    return grpo::fail(GRPO_EDEVICE, "grpo_logprob_fwd: the host-only sanitizer build has no device code");
}

extern "C" int grpo_logprob_fwd_paired(void*, int32_t, const void*, int64_t, int64_t, int64_t, const int32_t*,
                                       const uint8_t*, float*, float*, float*) {
    return grpo::fail(GRPO_EDEVICE, "grpo_logprob_fwd_paired: the host-only sanitizer build has no device code");
}
