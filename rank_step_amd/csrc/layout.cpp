// fsdp_shard_layout: the integer shard arithmetic of one rank (host only).
//
// FLAT mode follows the FlatParameter of the FSDP chapter (yangyitao.com,
// ch. 18), §18.12: the unit's parameters are flattened and concatenated in
// registration order into one vector that is sharded once, and they must
// share a dtype.  The tail padding to N * ceil(P / N) and the possibly empty
// per-rank views of the original parameters are from the ZeRO state sharding
// post (blog.cptz.space), section "FlatParameter 与 Padding".
//
// OWNER mode is ZeRO-1's owner assignment (ZeroRedundancyOptimizer) from the
// ZeRO state sharding post, sections "ZeRO-1：Optimizer State Sharding" and
// "Optimizer Step 的所有权": whole parameters go to owner ranks, balanced by
// bytes rather than by parameter count.
//
// SHARD0 mode follows FSDP2's per-parameter Shard(0) (MindSpeed-LLM FSDP2 doc,
// section "DTensor"; torchtitan FSDP2 article, §2.3): each parameter is split
// along dim 0 on its own.  When N does not divide dim 0 every rank still gets
// ceil(dim0 / N) rows and the rows past the end are padding.

#include <algorithm>
#include <cstdint>
#include <functional>
#include <queue>
#include <utility>
#include <vector>

#include "internal.h"

namespace {

using fsdp::fail;

int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0); }
int64_t clamp(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }
int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

int64_t dtype_size(int32_t dt) { return dt == FSDP_DT_F32 ? 4 : 2; }

int32_t shard_layout(int32_t mode, int32_t world_size, int32_t rank,
                     const fsdp_tensor_shape* tensors, int32_t n_tensors, int32_t has_master,
                     fsdp_shard_view* views_out, fsdp_layout_summary* summary_out) {
    if (mode != FSDP_LAYOUT_FLAT && mode != FSDP_LAYOUT_SHARD0 && mode != FSDP_LAYOUT_OWNER)
        return fail(FSDP_E_ARG, "fsdp_shard_layout: unknown mode %d", mode);
    if (world_size < 1) return fail(FSDP_E_ARG, "fsdp_shard_layout: world_size %d < 1", world_size);
    if (rank < 0 || rank >= world_size)
        return fail(FSDP_E_ARG, "fsdp_shard_layout: rank %d outside [0, %d)", rank, world_size);
    if (n_tensors < 0) return fail(FSDP_E_ARG, "fsdp_shard_layout: n_tensors %d < 0", n_tensors);
    if (n_tensors > 0 && (tensors == nullptr || views_out == nullptr))
        return fail(FSDP_E_ARG, "fsdp_shard_layout: null tensors or views_out");

    // Validate every shape before writing anything.
    int64_t logical = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        const fsdp_tensor_shape& t = tensors[i];
        if (t.reserved != 0) return fail(FSDP_E_ARG, "tensor %d: reserved field must be 0", i);
        if (t.dtype != FSDP_DT_F32 && t.dtype != FSDP_DT_BF16)
            return fail(FSDP_E_DTYPE, "tensor %d: unknown dtype %d", i, t.dtype);
        if (t.numel < 0 || t.dim0 < 0)
            return fail(FSDP_E_ARG, "tensor %d: negative numel or dim0", i);
        if (t.numel > 0 && (t.dim0 < 1 || t.numel % t.dim0 != 0))
            return fail(FSDP_E_ARG, "tensor %d: numel %lld is not a multiple of dim0 %lld", i,
                        (long long)t.numel, (long long)t.dim0);
        if (mode == FSDP_LAYOUT_FLAT && t.dtype != tensors[0].dtype)
            return fail(FSDP_E_DTYPE, "FLAT unit mixes dtypes (tensor %d vs tensor 0)", i);
        if (!fsdp::add_i64(logical, t.numel, &logical))
            return fail(FSDP_E_ARG, "total element count overflows int64");
    }

    const int64_t N = world_size;
    const int64_t r = rank;
    std::vector<fsdp_shard_view> views(static_cast<size_t>(n_tensors));
    fsdp_layout_summary s{};
    s.logical_numel = logical;

    if (mode == FSDP_LAYOUT_FLAT) {
        const int64_t S = ceil_div(logical, N);
        int64_t phys;
        if (!fsdp::mul_i64(S, N, &phys)) return fail(FSDP_E_ARG, "padded size overflows int64");
        const int64_t shard_lo = r * S;
        const int64_t valid = clamp(logical - shard_lo, 0, S);
        int64_t off = 0;
        for (int32_t i = 0; i < n_tensors; ++i) {
            const int64_t n = tensors[i].numel;
            const int64_t lo = max64(off, shard_lo);
            const int64_t hi = min64(off + n, shard_lo + S);
            fsdp_shard_view& v = views[i];
            v.shard_numel = S;
            v.valid = valid;
            v.global_offset = off;
            if (hi > lo) {
                v.view_offset = lo - shard_lo;
                v.view_numel = hi - lo;
                v.tensor_offset = lo - off;
            } else {
                v.view_offset = min64(lo - shard_lo, S);
                v.view_numel = 0;
                v.tensor_offset = min64(lo - off, n);
            }
            v.owner = -1;
            off += n;
        }
        const int64_t esize = n_tensors > 0 ? dtype_size(tensors[0].dtype) : 4;
        s.physical_numel = phys;
        s.shard_numel = S;
        s.pad_numel = S - valid;
        if (!fsdp::mul_i64(S, esize, &s.bytes_param))
            return fail(FSDP_E_ARG, "byte counts overflow int64");
    } else if (mode == FSDP_LAYOUT_SHARD0) {
        int64_t off = 0, packed = 0, phys = 0, bytes_param = 0, pad = 0;
        for (int32_t i = 0; i < n_tensors; ++i) {
            const fsdp_tensor_shape& t = tensors[i];
            int64_t sn = 0, valid = 0, toff = 0;
            if (t.numel > 0) {
                const int64_t row = t.numel / t.dim0;
                const int64_t c = ceil_div(t.dim0, N);
                const int64_t rows = clamp(t.dim0 - r * c, 0, c);
                if (!fsdp::mul_i64(c, row, &sn)) return fail(FSDP_E_ARG, "shard size overflows");
                valid = rows * row;
                toff = min64(r * c, t.dim0) * row;
            }
            fsdp_shard_view& v = views[i];
            v.shard_numel = sn;
            v.valid = valid;
            v.global_offset = off;
            v.view_offset = packed;
            v.view_numel = valid;
            v.tensor_offset = toff;
            v.owner = -1;
            int64_t sn_all, b;
            if (!fsdp::mul_i64(sn, N, &sn_all) || !fsdp::add_i64(phys, sn_all, &phys) ||
                !fsdp::add_i64(packed, sn, &packed) ||
                !fsdp::mul_i64(sn, dtype_size(t.dtype), &b) ||
                !fsdp::add_i64(bytes_param, b, &bytes_param))
                return fail(FSDP_E_ARG, "layout sizes overflow int64");
            off += t.numel;
            pad += sn - valid;
        }
        s.physical_numel = phys;
        s.shard_numel = packed;
        s.pad_numel = pad;
        s.bytes_param = bytes_param;
    } else {
        // OWNER: largest parameters first, each to the least-loaded rank
        // (ties: the lower rank).  Only the first min(N, n_tensors) ranks can
        // ever be chosen: until every one of them holds bytes, one of them
        // still has load 0, the least possible, and it has the lowest index
        // among the ranks at 0.  So a heap of (load, rank) over those ranks
        // gives the same choices as a scan over all N, in memory independent
        // of N.
        std::vector<int64_t> bytes(static_cast<size_t>(n_tensors));
        std::vector<int32_t> order(static_cast<size_t>(n_tensors));
        int64_t all_bytes = 0;
        for (int32_t i = 0; i < n_tensors; ++i) {
            order[i] = i;
            if (!fsdp::mul_i64(tensors[i].numel, dtype_size(tensors[i].dtype), &bytes[i]) ||
                !fsdp::add_i64(all_bytes, bytes[i], &all_bytes))
                return fail(FSDP_E_ARG, "layout sizes overflow int64");
        }
        std::stable_sort(order.begin(), order.end(),
                         [&](int32_t a, int32_t b) { return bytes[a] > bytes[b]; });
        using Load = std::pair<int64_t, int64_t>;  // (bytes held, rank)
        std::priority_queue<Load, std::vector<Load>, std::greater<Load>> least;
        for (int64_t q = 0; q < std::min<int64_t>(N, n_tensors); ++q) least.push({0, q});
        std::vector<int64_t> owner(static_cast<size_t>(n_tensors), 0);
        for (int32_t i : order) {
            const Load top = least.top();
            least.pop();
            owner[i] = top.second;
            least.push({top.first + bytes[i], top.second});
        }
        int64_t off = 0, packed = 0;
        for (int32_t i = 0; i < n_tensors; ++i) {
            const int64_t n = tensors[i].numel;
            fsdp_shard_view& v = views[i];
            const bool mine = owner[i] == r;
            v.shard_numel = mine ? n : 0;
            v.valid = mine ? n : 0;
            v.global_offset = off;
            v.view_offset = packed;
            v.view_numel = mine ? n : 0;
            v.tensor_offset = 0;
            v.owner = owner[i];
            if (mine) packed += n;
            off += n;
        }
        s.physical_numel = logical;
        s.shard_numel = packed;
        s.pad_numel = 0;
        s.bytes_param = all_bytes;
    }
    if (!fsdp::mul_i64(s.shard_numel, 8, &s.bytes_optim))
        return fail(FSDP_E_ARG, "byte counts overflow int64");
    s.bytes_grad = s.shard_numel * 4;
    s.bytes_master = has_master ? s.shard_numel * 4 : 0;
    // no_sync accumulation holds the whole gradient: the padded flat vector
    // (FLAT) or every full parameter (SHARD0), in fp32
    const int64_t unsharded = mode == FSDP_LAYOUT_FLAT ? s.physical_numel : s.logical_numel;
    // ZeRO-1 keeps the whole (all-reduced) gradient on every rank
    if (mode == FSDP_LAYOUT_OWNER && !fsdp::mul_i64(logical, 4, &s.bytes_grad))
        return fail(FSDP_E_ARG, "byte counts overflow int64");
    if (!fsdp::mul_i64(unsharded, 4, &s.bytes_grad_unsharded))
        return fail(FSDP_E_ARG, "byte counts overflow int64");
    for (int32_t i = 0; i < n_tensors; ++i) views_out[i] = views[i];
    if (summary_out) *summary_out = s;
    return FSDP_OK;
}

}  // namespace

extern "C" int32_t fsdp_shard_layout(int32_t mode, int32_t world_size, int32_t rank,
                                     const fsdp_tensor_shape* tensors, int32_t n_tensors,
                                     int32_t has_master, fsdp_shard_view* views_out,
                                     fsdp_layout_summary* summary_out) {
    return fsdp::guarded("fsdp_shard_layout", [&] {
        return shard_layout(mode, world_size, rank, tensors, n_tensors, has_master, views_out,
                            summary_out);
    });
}

namespace {

constexpr int64_t kRegionAlign = int64_t(2) << 20;  // every region's start
constexpr int64_t kRowLine = 64;                    // slice rows start on these element multiples
constexpr int64_t kRowPad = 256;                    // elements between one row's shard and the next row

int32_t rank_buffer_layout(int64_t S, int32_t n_slices, int32_t slice_dtype, int32_t bf16_slots,
                           int32_t grad_out, int32_t fp8_out, fsdp_rank_buffers* out) {
    const char* who = "fsdp_rank_buffer_layout";
    if (!out) return fail(FSDP_E_ARG, "%s: null out", who);
    if (S < 0) return fail(FSDP_E_ARG, "%s: shard_numel %lld < 0", who, static_cast<long long>(S));
    if (slice_dtype != FSDP_DT_F32 && slice_dtype != FSDP_DT_BF16)
        return fail(FSDP_E_DTYPE, "%s: unknown slice dtype %d", who, slice_dtype);
    if (n_slices < 1 || n_slices > 1024)
        return fail(FSDP_E_ARG, "%s: n_slices %d outside [1, 1024]", who, n_slices);
    if (bf16_slots < 0) return fail(FSDP_E_ARG, "%s: bf16_slots %d < 0", who, bf16_slots);
    if ((grad_out != 0 && grad_out != 1) || (fp8_out != 0 && fp8_out != 1))
        return fail(FSDP_E_ARG, "%s: grad_out and fp8_out must be 0 or 1", who);
    const int64_t es = slice_dtype == FSDP_DT_F32 ? 4 : 2;
    fsdp_rank_buffers r{};
    r.region_align = kRegionAlign;
    int64_t stride = S;
    if (n_slices > 1) {
        int64_t up;
        if (!fsdp::add_i64(S, kRowLine - 1, &up) || !fsdp::add_i64(up / kRowLine * kRowLine, kRowPad, &stride))
            return fail(FSDP_E_ARG, "%s: sizes overflow int64", who);
    }
    r.slice_stride = stride;
    // each present region: start at the next boundary, then advance by its bytes
    int64_t end = 0;
    bool ok = true;
    auto place = [&](int64_t elems, int64_t esize, bool present) -> int64_t {
        if (!present || !ok) return -1;
        int64_t start, bytes;
        if (!fsdp::add_i64(end, kRegionAlign - 1, &start) || !fsdp::mul_i64(elems, esize, &bytes)) {
            ok = false;
            return -1;
        }
        start = start / kRegionAlign * kRegionAlign;
        if (!fsdp::add_i64(start, bytes, &end)) ok = false;
        return start;
    };
    int64_t slice_elems = 0, bf16_elems = 0;
    if (!fsdp::mul_i64(stride, n_slices, &slice_elems) || !fsdp::mul_i64(S, bf16_slots, &bf16_elems))
        return fail(FSDP_E_ARG, "%s: sizes overflow int64", who);
    r.param_offset = place(S, 4, true);
    r.exp_avg_offset = place(S, 4, true);
    r.exp_avg_sq_offset = place(S, 4, true);
    r.slices_offset = place(slice_elems, es, true);
    r.bf16_offset = place(bf16_elems, 2, bf16_slots > 0);
    r.grad_out_offset = place(S, 4, grad_out != 0);
    r.fp8_offset = place(S, 1, fp8_out != 0);
    if (!ok) return fail(FSDP_E_ARG, "%s: sizes overflow int64", who);
    r.total_bytes = end;
    *out = r;
    return FSDP_OK;
}

}  // namespace

extern "C" int32_t fsdp_rank_buffer_layout(int64_t shard_numel, int32_t n_slices, int32_t slice_dtype,
                                           int32_t bf16_slots, int32_t grad_out, int32_t fp8_out,
                                           fsdp_rank_buffers* out) {
    return fsdp::guarded("fsdp_rank_buffer_layout", [&] {
        return rank_buffer_layout(shard_numel, n_slices, slice_dtype, bf16_slots, grad_out, fp8_out, out);
    });
}
