// Host logic of librank_step.so under AddressSanitizer and UBSan (CPU only).
//
// Built with g++ from the library's own host sources (layout.cpp, common.cpp)
// and run by tests/test_host_sanitized.py.  Two modes:
//
//   layout < cases   one case per input line:
//                      mode N rank has_master n  numel dim0 dtype  ...
//                    prints per case: rc, then (rc == 0) the 7 fields of each
//                    view and the 9 fields of the summary, space-separated.
//   alias SEED K     K random sets of byte ranges checked by check_aliases and
//                    by a pairwise brute force; prints "cases mismatches".
//   footprint SEED K K random sets of byte ranges indexed by Footprint, each
//                    queried with random intervals against a brute force;
//                    prints "cases queries mismatches".
//
// Any out-of-bounds access, signed overflow or other undefined behaviour
// aborts the run (it is compiled with -fno-sanitize-recover=all).
#include <cinttypes>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "internal.h"

namespace {

int run_layout() {
    std::string line;
    while (std::getline(std::cin, line)) {
        if (line.empty()) continue;
        std::istringstream in(line);
        int32_t mode, N, rank, has_master, n;
        in >> mode >> N >> rank >> has_master >> n;
        std::vector<fsdp_tensor_shape> shapes(static_cast<size_t>(n > 0 ? n : 0));
        for (auto& s : shapes) {
            long long numel, dim0;
            int dt;
            in >> numel >> dim0 >> dt;
            s.numel = numel;
            s.dim0 = dim0;
            s.dtype = dt;
            s.reserved = 0;
        }
        // exact-size output array: an overrun is an ASan error
        std::vector<fsdp_shard_view> views(shapes.size());
        fsdp_layout_summary summ;
        const int32_t rc = fsdp_shard_layout(mode, N, rank, shapes.empty() ? nullptr : shapes.data(),
                                             n, has_master, views.empty() ? nullptr : views.data(),
                                             &summ);
        std::printf("%d", rc);
        if (rc == FSDP_OK) {
            for (const auto& v : views)
                std::printf(" %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64
                            " %" PRId64,
                            v.shard_numel, v.valid, v.global_offset, v.view_offset, v.view_numel,
                            v.tensor_offset, v.owner);
            std::printf(" %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64 " %" PRId64
                        " %" PRId64 " %" PRId64 " %" PRId64,
                        summ.logical_numel, summ.physical_numel, summ.shard_numel, summ.pad_numel,
                        summ.bytes_param, summ.bytes_grad, summ.bytes_optim, summ.bytes_master,
                        summ.bytes_grad_unsharded);
        } else if (std::strlen(fsdp_last_error()) == 0) {
            std::printf(" nomessage");
        }
        std::printf("\n");
    }
    return 0;
}

// splitmix64: a small, well-known counter-based generator
uint64_t mix(uint64_t& s) {
    uint64_t z = (s += 0x9e3779b97f4a7c15ULL);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

int run_alias(uint64_t seed, int cases) {
    uint64_t s = seed;
    int mismatches = 0;
    for (int c = 0; c < cases; ++c) {
        const int n = static_cast<int>(mix(s) % 12);
        const uint64_t span = 16 + mix(s) % 512;   // small address space: overlaps are common
        std::vector<fsdp::Range> rs;
        for (int i = 0; i < n; ++i) {
            const uintptr_t lo = 4096 + mix(s) % span;
            const uintptr_t len = (mix(s) % 4 == 0) ? 0 : mix(s) % 64;
            rs.push_back(fsdp::Range{lo, lo + len, mix(s) % 2 == 0, i, "r"});
        }
        bool expect_alias = false;
        for (int i = 0; i < n; ++i)
            for (int j = i + 1; j < n; ++j) {
                const auto& a = rs[i];
                const auto& b = rs[j];
                if (a.hi <= a.lo || b.hi <= b.lo) continue;
                if ((a.written || b.written) && a.lo < b.hi && b.lo < a.hi) expect_alias = true;
            }
        std::vector<fsdp::Range> copy = rs;
        const int32_t rc = fsdp::check_aliases(copy);
        if ((rc == FSDP_E_ALIAS) != expect_alias || (rc != FSDP_OK && rc != FSDP_E_ALIAS))
            ++mismatches;
    }
    std::printf("%d %d\n", cases, mismatches);
    return 0;
}

int run_footprint(uint64_t seed, int cases) {
    uint64_t s = seed;
    long queries = 0, mismatches = 0;
    for (int c = 0; c < cases; ++c) {
        const int n = static_cast<int>(mix(s) % 16);
        const uint64_t span = 16 + mix(s) % 512;
        std::vector<fsdp::Range> rs;
        for (int i = 0; i < n; ++i) {
            const uintptr_t lo = 4096 + mix(s) % span;
            const uintptr_t len = (mix(s) % 5 == 0) ? 0 : mix(s) % 64;
            rs.push_back(fsdp::Range{lo, lo + len, mix(s) % 2 == 0, i, "r"});
        }
        fsdp::Footprint fp;
        fp.build(rs);
        for (int k = 0; k < 32; ++k) {
            const uintptr_t lo = 4000 + mix(s) % (span + 200);
            const uintptr_t len = (mix(s) % 6 == 0) ? 0 : 1 + mix(s) % 48;
            const uintptr_t hi = lo + len;
            bool want_w = false, want_any = false;
            for (const auto& r : rs) {
                const bool meet = r.lo < r.hi && lo < hi && r.lo < hi && lo < r.hi;
                want_any = want_any || meet;
                want_w = want_w || (meet && r.written);
            }
            ++queries;
            if (fp.hits_written(lo, hi) != want_w || fp.hits_any(lo, hi) != want_any) ++mismatches;
        }
    }
    std::printf("%d %ld %ld\n", cases, queries, mismatches);
    return 0;
}

}  // namespace

int main(int argc, char** argv) {
    if (argc >= 2 && std::strcmp(argv[1], "layout") == 0) return run_layout();
    if (argc >= 4 && std::strcmp(argv[1], "alias") == 0)
        return run_alias(std::strtoull(argv[2], nullptr, 10), std::atoi(argv[3]));
    if (argc >= 4 && std::strcmp(argv[1], "footprint") == 0)
        return run_footprint(std::strtoull(argv[2], nullptr, 10), std::atoi(argv[3]));
    std::fprintf(stderr, "usage: %s layout < cases | alias SEED K | footprint SEED K\n", argv[0]);
    return 2;
}
