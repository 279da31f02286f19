// Plan trace dump of libgrpo: the rows each training call of a plan holds,
// written as JSON lines with the fields a minimal batch trace records.
//
// Source: [P2] "03 Data Protocol and Batch Lifecycle", "Trace Entry" (stage,
// field, producer / consumer, shape or nested length, dtype / device, valid
// length, response_mask.sum(), uid / trajectory key, global step,
// is_padding) and "Batch Shape Transitions" (the nested length of a row and
// the positions that carry a policy gradient are different numbers).

#include <cstdio>
#include <cstring>

#include "common.h"

using grpo::fail;
using grpo::ok;

namespace {

bool label_ok(const char* s) {
    if (!s) return false;
    size_t n = 0;
    for (; s[n]; ++n) {
        const char c = s[n];
        const bool good = (c >= 'a' && c <= 'z') || (c >= 'A' && c <= 'Z') || (c >= '0' && c <= '9') || c == '_' ||
                          c == '.' || c == '-';
        if (!good || n >= 63) return false;
    }
    return n > 0;
}

const char* dtype_name(int32_t d) { return d == GRPO_BF16 ? "bf16" : "f32"; }

// Appends one formatted line: counts its bytes into *used and, when `out` is
// set, copies it there.  Lines are short (well under the stack buffer).
class Sink {
  public:
    explicit Sink(char* out) : out_(out) {}
    size_t used() const { return used_; }
    void line(const char* fmt, ...) {
        char tmp[768];
        va_list ap;
        va_start(ap, fmt);
        const int n = std::vsnprintf(tmp, sizeof(tmp), fmt, ap);
        va_end(ap);
        const size_t k = n < 0 ? 0 : ((size_t)n < sizeof(tmp) ? (size_t)n : sizeof(tmp) - 1);
        if (out_) std::memcpy(out_ + used_, tmp, k);
        used_ += k;
    }

  private:
    char* out_;
    size_t used_ = 0;
};

int check(const grpo_trace_plan* p) {
    if (!p || p->struct_size != (int32_t)sizeof(grpo_trace_plan))
        return fail(GRPO_EINVAL, "grpo_plan_trace: NULL plan or struct_size mismatch");
    if (!label_ok(p->stage)) return fail(GRPO_EINVAL, "grpo_plan_trace: stage must be 1..63 of [A-Za-z0-9_.-]");
    if (p->dtype != GRPO_F32 && p->dtype != GRPO_BF16) return fail(GRPO_EINVAL, "grpo_plan_trace: unknown dtype");
    if (p->n_rows < 0 || p->n_calls < 0 || p->T < 0 || p->V < 1)
        return fail(GRPO_EINVAL, "grpo_plan_trace: negative size or V < 1");
    if (p->n_rows > 0 && (!p->row_len || !p->row_valid || !p->row_uid || !p->row_traj))
        return fail(GRPO_EINVAL, "grpo_plan_trace: NULL row array");
    if (!p->call_off || (p->n_calls > 0 && !p->call_step)) return fail(GRPO_EINVAL, "grpo_plan_trace: NULL call array");
    for (int64_t r = 0; r < p->n_rows; ++r) {
        if (p->row_len[r] < 0 || p->row_valid[r] < 0 || p->row_valid[r] > p->row_len[r] ||
            (p->T > 0 && p->row_len[r] > p->T))
            return fail(GRPO_EINVAL, "grpo_plan_trace: row %lld has length %lld and %lld valid positions (T %lld)",
                        (long long)r, (long long)p->row_len[r], (long long)p->row_valid[r], (long long)p->T);
        const bool pad = p->row_is_pad && p->row_is_pad[r];
        if (p->row_uid[r] < 0 || (!pad && (p->row_traj[r] < 0 || (p->row_seg && p->row_seg[r] < 0))))
            return fail(GRPO_EINVAL, "grpo_plan_trace: row %lld has a negative uid, rollout or segment", (long long)r);
    }
    if (p->call_off[0] != 0) return fail(GRPO_EINVAL, "grpo_plan_trace: call_off[0] must be 0");
    for (int64_t k = 0; k < p->n_calls; ++k) {
        if (p->call_off[k + 1] < p->call_off[k]) return fail(GRPO_EINVAL, "grpo_plan_trace: call_off decreases");
        if (p->call_step[k] < 0) return fail(GRPO_EINVAL, "grpo_plan_trace: negative step");
    }
    if (p->call_off[p->n_calls] > 0 && !p->call_rows) return fail(GRPO_EINVAL, "grpo_plan_trace: NULL call_rows");
    for (int64_t i = 0; i < p->call_off[p->n_calls]; ++i)
        if (p->call_rows[i] < 0 || p->call_rows[i] >= p->n_rows)
            return fail(GRPO_EINVAL, "grpo_plan_trace: call_rows[%lld] = %lld is not a row", (long long)i,
                        (long long)p->call_rows[i]);
    return GRPO_OK;
}

void emit(const grpo_trace_plan* p, Sink& s) {
    const char* dt = dtype_name(p->dtype);
    for (int64_t k = 0; k < p->n_calls; ++k) {
        int64_t pads = 0, positions = 0, valid = 0;
        const int64_t a = p->call_off[k], b = p->call_off[k + 1];
        for (int64_t i = a; i < b; ++i) {
            const int64_t r = p->call_rows[i];
            const int pad = p->row_is_pad ? (p->row_is_pad[r] != 0) : 0;
            const int64_t len = p->row_len[r];
            const int64_t shape0 = p->T > 0 ? p->T : len;
            char traj[16] = "null", seg[16] = "null";
            if (p->row_traj[r] >= 0) std::snprintf(traj, sizeof(traj), "%d", p->row_traj[r]);
            if (!p->row_seg) std::snprintf(seg, sizeof(seg), "0");
            else if (p->row_seg[r] >= 0) std::snprintf(seg, sizeof(seg), "%d", p->row_seg[r]);
            s.line("{\"stage\": \"%s\", \"call\": %lld, \"step\": %lld, \"pos\": %lld, \"row\": %lld, \"uid\": %d, "
                   "\"traj\": %s, \"seg\": %s, \"field\": \"logits\", \"producer\": \"policy forward\", "
                   "\"consumer\": \"grpo_loss_fwd_bwd\", \"shape\": [%lld, %lld], \"dtype\": \"%s\", "
                   "\"device\": \"gpu\", \"len\": %lld, \"valid\": %lld, \"is_padding\": %s}\n",
                   p->stage, (long long)k, (long long)p->call_step[k], (long long)(i - a), (long long)r,
                   p->row_uid[r], traj, seg, (long long)shape0,
                   (long long)p->V, dt, (long long)len, (long long)p->row_valid[r], pad ? "true" : "false");
            pads += pad;
            positions += shape0;
            valid += p->row_valid[r];
        }
        s.line("{\"stage\": \"%s\", \"call\": %lld, \"step\": %lld, \"summary\": true, \"rows\": %lld, "
               "\"pads\": %lld, \"positions\": %lld, \"valid\": %lld}\n",
               p->stage, (long long)k, (long long)p->call_step[k], (long long)(b - a), (long long)pads,
               (long long)positions, (long long)valid);
    }
}

}  // namespace

extern "C" int grpo_plan_trace(const grpo_trace_plan* plan, char* buf, size_t cap, size_t* need) {
    if (!need) return fail(GRPO_EINVAL, "grpo_plan_trace: NULL need");
    const int rc = check(plan);
    if (rc != GRPO_OK) return rc;
    Sink count(nullptr);
    emit(plan, count);
    *need = count.used() + 1;
    if (!buf || cap < *need)
        return fail(GRPO_ECAPACITY, "grpo_plan_trace: the trace takes %zu bytes, the buffer holds %zu", *need, cap);
    Sink write(buf);
    emit(plan, write);
    buf[write.used()] = '\0';
    return ok();
}
