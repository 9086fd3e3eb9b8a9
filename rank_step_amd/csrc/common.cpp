// Error reporting and small host utilities of librank_step.so.
#include <algorithm>
#include <cstdarg>
#include <cstdio>

#include "internal.h"

namespace fsdp {

namespace {
// A fixed buffer, so that recording an error never allocates (and so never
// throws, even when host memory has run out).
thread_local char g_last_error[512];
}

int32_t fail(int32_t code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

int32_t ok() { return FSDP_OK; }

bool mul_i64(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }
bool add_i64(int64_t a, int64_t b, int64_t* out) { return !__builtin_add_overflow(a, b, out); }

int32_t check_aliases(std::vector<Range>& ranges) {
    ranges.erase(std::remove_if(ranges.begin(), ranges.end(),
                                [](const Range& r) { return r.hi <= r.lo; }),
                 ranges.end());
    std::sort(ranges.begin(), ranges.end(),
              [](const Range& a, const Range& b) { return a.lo < b.lo; });
    // Sweep in start order, remembering the furthest-reaching written range and
    // the furthest-reaching range of any kind seen so far.
    const Range* far_any = nullptr;
    const Range* far_written = nullptr;
    for (const Range& r : ranges) {
        if (far_written && r.lo < far_written->hi)
            return fail(FSDP_E_ALIAS, "%s of shard %d overlaps written %s of shard %d", r.what,
                        r.owner, far_written->what, far_written->owner);
        if (r.written && far_any && r.lo < far_any->hi)
            return fail(FSDP_E_ALIAS, "written %s of shard %d overlaps %s of shard %d", r.what,
                        r.owner, far_any->what, far_any->owner);
        if (!far_any || r.hi > far_any->hi) far_any = &r;
        if (r.written && (!far_written || r.hi > far_written->hi)) far_written = &r;
    }
    return FSDP_OK;
}

}  // namespace fsdp

extern "C" const char* fsdp_last_error(void) { return fsdp::g_last_error; }
