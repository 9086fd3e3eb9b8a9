// Internal helpers shared by the host sources of librank_step.so.
#pragma once

#include <cstdint>
#include <new>
#include <utility>
#include <vector>

#include "fsdp_step.h"

namespace fsdp {

// Records `code` with a printf-style message as this thread's last error and
// returns `code`.
int32_t fail(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int32_t ok();

// Overflow-checked int64 arithmetic; return false on overflow.
bool mul_i64(int64_t a, int64_t b, int64_t* out);
bool add_i64(int64_t a, int64_t b, int64_t* out);

// A byte range [lo, hi) of one buffer named `what`, written or read-only.
struct Range {
    uintptr_t lo, hi;
    bool written;
    int32_t owner;  // tensor index inside a plan, or 0
    const char* what;
};

// FSDP_E_ALIAS if a written range overlaps any other range (read-only ranges
// may overlap each other); empty ranges never overlap.
int32_t check_aliases(std::vector<Range>& ranges);

// The byte ranges of every buffer a plan's shards name, kept so that the
// further device buffers a plan call takes (a scale, an amax array, a sum)
// can be checked against them in O(log n).  `written` holds the buffers some
// plan call writes, `read` the read-only ones (the gradient slices); each is
// kept as a sorted union of disjoint intervals.
class Footprint {
public:
    void build(const std::vector<Range>& ranges);
    // Whether [lo, hi) overlaps a written buffer of the plan.
    bool hits_written(uintptr_t lo, uintptr_t hi) const;
    // Whether [lo, hi) overlaps any buffer of the plan.
    bool hits_any(uintptr_t lo, uintptr_t hi) const;

private:
    using Span = std::pair<uintptr_t, uintptr_t>;
    static void merge(std::vector<Span>& spans);
    static bool hits(const std::vector<Span>& spans, uintptr_t lo, uintptr_t hi);
    std::vector<Span> written_, read_;
};

// Runs an entry point's body and turns a C++ exception into an error code, so
// that nothing throws across the C ABI.  The only one the bodies can raise is
// std::bad_alloc, from host-side tables and lists when host memory runs out.
template <typename F>
int32_t guarded(const char* who, F&& body) noexcept {
    try {
        return body();
    } catch (const std::bad_alloc&) {
        return fail(FSDP_E_CAPACITY, "%s: out of host memory", who);
    } catch (...) {
        return fail(FSDP_E_ARG, "%s: unexpected host-side error", who);
    }
}

}  // namespace fsdp
