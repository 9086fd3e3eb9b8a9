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

void Footprint::merge(std::vector<Span>& spans) {
    std::sort(spans.begin(), spans.end());
    size_t n = 0;
    for (const Span& s : spans) {
        if (n > 0 && s.first <= spans[n - 1].second)
            spans[n - 1].second = std::max(spans[n - 1].second, s.second);
        else
            spans[n++] = s;
    }
    spans.resize(n);
    spans.shrink_to_fit();
}

void Footprint::build(const std::vector<Range>& ranges) {
    written_.clear();
    read_.clear();
    for (const Range& r : ranges) {
        if (r.hi <= r.lo) continue;
        (r.written ? written_ : read_).emplace_back(r.lo, r.hi);
    }
    merge(written_);
    merge(read_);
}

bool Footprint::hits(const std::vector<Span>& spans, uintptr_t lo, uintptr_t hi) {
    if (hi <= lo) return false;
    // the first span that ends after lo; the spans are disjoint and sorted, so
    // their ends are sorted too
    const auto it = std::upper_bound(spans.begin(), spans.end(), lo,
                                     [](uintptr_t x, const Span& s) { return x < s.second; });
    return it != spans.end() && it->first < hi;
}

bool Footprint::hits_written(uintptr_t lo, uintptr_t hi) const { return hits(written_, lo, hi); }

bool Footprint::hits_any(uintptr_t lo, uintptr_t hi) const {
    return hits(written_, lo, hi) || hits(read_, lo, hi);
}

}  // namespace fsdp

extern "C" const char* fsdp_last_error(void) { return fsdp::g_last_error; }
