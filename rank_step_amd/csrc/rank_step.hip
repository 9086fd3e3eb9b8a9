// HIP kernels and device entry points of librank_step.so (gfx950 / MI355X).
//
// One FSDP FULL_SHARD rank's step after the backward reduce-scatter and before
// the next forward all-gather: the fp32 mean of the N gradient slices of the
// rank's shard, decoupled-weight-decay AdamW on that shard only, and the bf16
// cast of the updated shard into the all-gather input slot.  The arithmetic
// and its sources are stated at each device function below and in the header.
//
// The path is bound by HBM bandwidth (about half a flop per byte), so there is
// no matrix-core work: every kernel is a streaming pass.  A workgroup is one
// wave64 and covers one 256-element tile: each lane moves 4 consecutive
// elements per access (one 16-byte load per fp32 array, one 8-byte load per
// bf16 slice), and every load of the tile is issued before its first use.
// Gradient slices, the low-precision copies and the state loads are touched
// once and use non-temporal accesses.  Every streaming pass writes its
// stores through to memory (plain or non-temporal write-through, by its mix
// of bytes), so that a launch does not end with dirty lines in L2 for its
// release to write back.  The vector path needs a shard's fp32 buffers
// 16-byte aligned; its slices and copies may start at any element (shifted
// loads, stores in narrower pieces), and a plan splits a shard whose fp32
// buffers all start off a boundary into a short head and an aligned rest.
// What is left (shards whose fp32 buffers disagree, partial groups, the
// padding) goes element by element with the same arithmetic
// (bit-identical results).
//
// Residency is capped on purpose: each streaming launch reserves enough LDS
// (which the kernels do not otherwise use) that only a few workgroups share a
// compute unit.  On MI355X the HBM stacks deliver markedly more bandwidth to
// this mix of reads and in-place writes when each CU keeps tens of kilobytes
// of loads in flight rather than the few hundred that full occupancy issues.
//
// The multi-tensor launch reads a host-built chunk-descriptor table: entry
// b/8 names a shard and a 2048-element range of it, and workgroup b takes the
// (b%8)-th tile of that range, reading the entry and the shard's descriptor
// with scalar loads.
//
// Floating point: fp32, FMA only where written (built with -ffp-contract=off),
// IEEE-correct division and square root, denormals kept.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <type_traits>
#include <vector>

#include "internal.h"

using fsdp::fail;

namespace {

// Build-time tunables.  The defaults are the fastest measured on MI355X;
// other values exist for measurement.
// Non-temporal hints: 1 = nt on the access class, 0 = ordinary access.
#ifndef RS_NT_SLICES
#define RS_NT_SLICES 1
#endif
#ifndef RS_NT_OUT
#define RS_NT_OUT 1
#endif
// State loads (master, moments, a no_sync accumulator): non-temporal since
// the stores write through, with which the 7B shard's step runs 1.6 % faster
// (5.28 against 5.37 ms), the 70B shard's 1.0 %, the small workloads 1.5-2.7 %.
#ifndef RS_NT_STATE_LD
#define RS_NT_STATE_LD 1
#endif
// The synchronised accumulation's load of the running sum it adds to: an
// ordinary load (2.94 ms per micro-batch on the 7B shard, 3.01 non-temporal).
#ifndef RS_NT_ACC_LD
#define RS_NT_ACC_LD 0
#endif
#ifndef RS_NT_STATE_ST
#define RS_NT_STATE_ST 0
#endif
// Cache policy of the fused step's state stores: -1 chooses per plan from
// its mix of reads and writes (see store_policy), 0/1/2 force plain stores,
// write-through or non-temporal write-through.
#ifndef RS_ST_POLICY
#define RS_ST_POLICY -1
#endif
// The same for the stores of the other streaming passes (the clipped update,
// the fp8 steps and code pass, the reduce/accumulate pass, the no_sync
// accumulation): -1 chooses per launch from the pass's own mix of reads and
// writes, by the fused step's rule; 0/1/2 force one policy.
#ifndef RS_ST_POLICY_PASSES
#define RS_ST_POLICY_PASSES -1
#endif
// Bytes of HBM traffic (loads and stores) one CU should keep in flight: each
// launch caps its resident workgroups at this divided by what one workgroup
// moves, through its LDS reservation.
#ifndef RS_INFLIGHT_KB
#define RS_INFLIGHT_KB 100
#endif
// The fused steps that also reduce |p'| and write fp8 codes keep each wave
// longer for the same bytes, so they need more resident waves: their budget.
#ifndef RS_INFLIGHT_KB_FP8
#define RS_INFLIGHT_KB_FP8 105
#endif
// The fused step's budgets under its write-through store policies (see
// StorePolicy): write-through keeps the general budget; non-temporal
// write-through, whose writes are close to half the traffic, needs fewer
// resident waves (the 70B shard: 10.09 against 10.27 ms at 100 KB).
#ifndef RS_INFLIGHT_KB_WT
#define RS_INFLIGHT_KB_WT RS_INFLIGHT_KB
#endif
#ifndef RS_INFLIGHT_KB_NTWT
#define RS_INFLIGHT_KB_NTWT 80
#endif
// The synchronised accumulation pass (reduce, then add into the stored
// gradient) ran 7 % slower at 16 resident workgroups per CU than at 15, which
// the general budget would give it: its budget.
#ifndef RS_INFLIGHT_KB_ACC
#define RS_INFLIGHT_KB_ACC 90
#endif
// 256-element tiles per workgroup of the fp8 code pass (1, 2, 4 or 8): it
// moves 5 bytes per element, so its lanes take several groups each.  It reads
// four bytes for every one it writes and runs uncapped: the residency cap
// helps the passes that write back what they read, not this one.
#ifndef RS_CAST_TILES
#define RS_CAST_TILES 4
#endif
// 1: the copy passes (fp8 codes, bf16 cast) read the updated parameter with
// non-temporal loads: it is read once there, and the code pass ran 4 % faster.
#ifndef RS_NT_CAST_LD
#define RS_NT_CAST_LD 1
#endif
// 1: fp8 codes from the hardware's packed fp32 -> OCP E4M3 conversion;
// 0: from the integer rounding e4m3_rne.
#ifndef RS_FP8_HW
#define RS_FP8_HW 1
#endif
// Slice counts other than 1, 2, 4 and 8 are read in batches of this many
// bytes per lane (4 bf16 or 2 fp32 slices): a batch's loads are issued
// together, before its first add, and a launch sizes its residency from one
// batch.  Slice by slice, N = 16 bf16 slices ran at 2.5 TB/s; in these
// batches, at 6.1-6.4.
#ifndef RS_RT_BATCH_BYTES
#define RS_RT_BATCH_BYTES 32
#endif
// 1: a plan whose shards lie back to back in every buffer, and start on a
// chunk-entry boundary of the whole but for a negligible share of its
// elements, runs its fused step as one range described by the kernel's
// arguments: the same tiles on the same XCDs as through the chunk table,
// without the two dependent table loads before a workgroup's first access;
// 0: every plan goes through its chunk table.
#ifndef RS_RUN_STEP
#define RS_RUN_STEP 1
#endif
// Budget of that one-range step under write-through stores, for the slice
// counts compiled in: its waves stream from their first instructions, so
// fewer resident waves keep the bytes in flight (one Llama-7B block at N = 8:
// 162.5-163.0 us at 75 KB, 165.0 at 100; the 128 MiB flat unit: 55.2 against
// 55.7).  Batched slice counts keep the general budget: at 75 KB, N = 5, 16
// and 32 bf16 slices lost 12-14 % (5.45, 5.66, 5.31 against 6.23, 6.29,
// 6.06 TB/s).
#ifndef RS_INFLIGHT_KB_RUN
#define RS_INFLIGHT_KB_RUN 75
#endif
// A launch whose share of that budget would allow this many resident
// workgroups per CU or more is left uncapped (light kernels want every wave).
#ifndef RS_OCC_UNCAPPED
#define RS_OCC_UNCAPPED 32
#endif

constexpr int kBlock = 64;              // threads per workgroup: one wave64
constexpr int kGroup = 4;               // elements per lane access
constexpr int kTile = kBlock * kGroup;  // elements per workgroup
constexpr int kTilesPerChunk = 8;
constexpr int64_t kChunk = int64_t(kTilesPerChunk) * kTile;  // elements per chunk entry
constexpr int kMaxSlices = 1024;
constexpr int kMaxDevices = 64;         // devices whose per-device library state is tracked
constexpr int kLdsPerCu = 160 * 1024;   // gfx950

// Dynamic LDS that leaves room for `occ` workgroups per CU but not occ + 1.
constexpr size_t lds_for(int occ) {
    return occ <= 0 ? 0 : static_cast<size_t>(2 * kLdsPerCu / (2 * occ + 1)) & ~size_t(255);
}
constexpr bool lds_admits(int occ) {
    return occ <= 0 || (lds_for(occ) <= 64 * 1024 && lds_for(occ) * occ <= kLdsPerCu &&
                        lds_for(occ) * (occ + 1) > kLdsPerCu);
}
constexpr int kMinOcc = 4, kMaxOcc = 16;   // residency range a cap may set
constexpr bool all_admitted(int occ) {
    return occ > kMaxOcc || (lds_admits(occ) && all_admitted(occ + 1));
}
static_assert(all_admitted(kMinOcc),
              "every capped residency fits one workgroup's LDS limit and admits exactly its count");

// The LDS reservation of a streaming launch whose lanes each move
// `bytes_per_elem` bytes for each of their kGroup elements, for an in-flight
// budget of `budget_kb` per CU.
constexpr size_t lds_reserve(int64_t bytes_per_elem, int64_t budget_kb = RS_INFLIGHT_KB) {
    const int64_t per_wg = bytes_per_elem * kTile;
    const int64_t occ = per_wg > 0 ? budget_kb * 1024 / per_wg : RS_OCC_UNCAPPED;
    if (occ >= RS_OCC_UNCAPPED) return 0;
    return lds_for(static_cast<int>(std::min<int64_t>(std::max<int64_t>(occ, kMinOcc), kMaxOcc)));
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One shard as the kernels see it.
struct TensorDesc {
    float* param;
    float* m;
    float* v;
    const void* slices;
    uint16_t* out_bf16;  // null: no cast
    float* grad_out;     // null: reduced gradient not stored
    uint8_t* out_fp8;    // null: no fp8 copy
    const void* const* slice_ptrs;  // null: slice q at slices + q*slice_stride;
                                    // else slice q at slice_ptrs[q] (device table)
    int64_t slice_stride;
    int64_t shard_numel;
    int64_t valid;
    int64_t vec_ok;      // the buffers the vector path needs aligned are aligned
    int64_t index;       // position of the shard in the plan's input list
    int64_t gen;         // kGenStore | kGenLoad: a low-precision copy / a slice is not
                         // vector-aligned (then the any-alignment forms run)
};

constexpr int64_t kGenStore = 1, kGenLoad = 2;

// One entry of the chunk-descriptor table: elements [begin, begin+count) of a shard.
struct ChunkDesc {
    int64_t begin;
    int32_t tensor;
    int32_t count;
};
static_assert(sizeof(ChunkDesc) == 16, "chunk entries are 16 bytes");

// fp32 scalars of one step, derived on the host in double.
struct StepConsts {
    float decay;         // 1 - lr*wd
    float beta1, omb1;   // beta1, 1 - beta1
    float beta2, omb2;   // beta2, 1 - beta2
    float step_size;     // lr / (1 - beta1^t)
    float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
    float eps;
    float inv_n;         // 1/N, used when N is a power of two (then x*(1/N) == x/N exactly)
    float n_f;           // N as fp32, the divisor otherwise
    int32_t n;           // N
    int32_t n_pow2;
};

// beta^t by binary exponentiation: the same IEEE double products on the host
// and on the device, so that both derive bit-identical scalars from t.
__host__ __device__ inline double pow_steps(double b, int64_t t) {
    double r = 1.0, x = b;
    for (; t > 0; t >>= 1) {
        if (t & 1) r = r * x;
        x = x * x;
    }
    return r;
}

// The scalars that depend on the step count t or on the learning rate:
// 1 - lr*wd, lr / (1 - beta1^t) and 1 / sqrt(1 - beta2^t), in double
// (correctly rounded division and square root on the host and on the device
// alike), each rounded once to fp32.
__host__ __device__ inline void count_scalars(StepConsts& c, double lr, double wd, double beta1,
                                              double beta2, int64_t t) {
    c.decay = static_cast<float>(1.0 - lr * wd);
    const double bc1 = 1.0 - pow_steps(beta1, t);
    const double bc2 = 1.0 - pow_steps(beta2, t);
    c.step_size = static_cast<float>(lr / bc1);
    c.inv_sqrt_bc2 = static_cast<float>(1.0 / sqrt(bc2));
}

// ---------------------------------------------------------------- device math

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest with ties to even; the carry out of the low
// half rounds up, overflow reaches the infinity pattern; NaN becomes the quiet
// NaN 0x7fc0 with the input's sign.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t qnan = ((u >> 16) & 0x8000u) | 0x7fc0u;
    return (u & 0x7fffffffu) > 0x7f800000u ? qnan : rounded;
}

// fp32 -> OCP FP8 E4M3 ("e4m3fn": bias 7, 3 fraction bits, largest finite
// 448, no infinities), round to nearest with ties to even.  The input is
// already within [-448, 448] or NaN.  Normal results: round the fp32
// fraction to 3 bits (the carry may raise the exponent) and rebias the
// exponent from 127 to 7.  Below 2^-6 the grid is 2^-9: scale by 2^9 (exact)
// and round to an integer.  NaN becomes S.1111.111.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t ua = u & 0x7fffffffu;
    const float a = __uint_as_float(ua);
    const uint32_t sub = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
    const uint32_t r = ua + 0x7ffffu + ((ua >> 20) & 1u);
    const uint32_t nrm = (r >> 20) - (120u << 3);
    const uint32_t code = ua > 0x7f800000u ? 0x7fu : (a < 0.015625f ? sub : nrm);
    return sign | code;
}

// The value an fp8 code encodes: the product with the tensor's scale in fp32,
// clamped to +-448 (NaN kept).
__device__ __forceinline__ float fp8_scaled(float p, float scale) {
    const float y = p * scale;
    return y > 448.0f ? 448.0f : (y < -448.0f ? -448.0f : y);
}

// The fp8 code of one updated value, rounded once.  gfx950's packed
// conversion rounds fp32 to OCP E4M3 to nearest even; on the clamped range
// it gives the same codes as e4m3_rne (checked over every fp32 pattern), in
// one instruction per pair instead of about fifteen per value.
__device__ __forceinline__ uint32_t fp8_code(float p, float scale) {
    if constexpr (RS_FP8_HW)
        return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(fp8_scaled(p, scale), 0.0f, 0, false)) & 0xffu;
    else
        return e4m3_rne(fp8_scaled(p, scale));
}

// Codes of four values, element j in byte j.
__device__ __forceinline__ uint32_t pack_fp8(const f32x4& p, float scale) {
    if constexpr (RS_FP8_HW) {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_scaled(p[0], scale), fp8_scaled(p[1], scale), 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_scaled(p[2], scale), fp8_scaled(p[3], scale), w, true);
        return static_cast<uint32_t>(w);
    } else {
        return fp8_code(p[0], scale) | (fp8_code(p[1], scale) << 8) | (fp8_code(p[2], scale) << 16) |
               (fp8_code(p[3], scale) << 24);
    }
}

// Mean of the slices: the fp32 sum in slice order, then one division by N.
__device__ __forceinline__ float finish_mean(float s, const StepConsts& c) {
    if (c.n == 1) return s;
    return c.n_pow2 ? s * c.inv_n : s / c.n_f;
}

// Decoupled-weight-decay AdamW on one element, as torch.optim.AdamW does it:
// decay the old parameter by (1 - lr*wd), update both moments, bias-correct
// them, and step by lr * mhat / (sqrt(vhat) + eps).
__device__ __forceinline__ void adamw(float& p, float& m, float& v, float g, const StepConsts& c) {
    const float p1 = p * c.decay;
    const float mn = __builtin_fmaf(c.beta1, m, c.omb1 * g);
    const float gg = g * g;
    const float vn = __builtin_fmaf(c.beta2, v, c.omb2 * gg);
    const float den = __builtin_fmaf(sqrtf(vn), c.inv_sqrt_bc2, c.eps);
    const float pn = __builtin_fmaf(-c.step_size, mn / den, p1);
    p = pn;
    m = mn;
    v = vn;
}

// Every buffer is device global memory: address it as such so the compiler
// emits global (not flat) loads and stores.
template <typename T>
using global_ptr = __attribute__((address_space(1))) T*;

template <typename T>
__device__ __forceinline__ T ld(const T* p) { return *(const global_ptr<T>)p; }
template <typename T>
__device__ __forceinline__ void st(T* p, T x) { *(global_ptr<T>)p = x; }

// Streaming accesses; NT selects the non-temporal form.
template <bool NT, typename T>
__device__ __forceinline__ T ld_s(const T* p) {
    if constexpr (NT) return __builtin_nontemporal_load((const global_ptr<T>)p);
    else return ld(p);
}
template <bool NT, typename T>
__device__ __forceinline__ void st_s(T* p, T x) {
    if constexpr (NT) __builtin_nontemporal_store(x, (global_ptr<T>)p);
    else st(p, x);
}
template <typename T> __device__ __forceinline__ T ld_slice(const T* p) { return ld_s<RS_NT_SLICES>(p); }
template <typename T> __device__ __forceinline__ T ld_state(const T* p) { return ld_s<RS_NT_STATE_LD>(p); }
template <typename T> __device__ __forceinline__ void st_state(T* p, T x) { st_s<RS_NT_STATE_ST>(p, x); }
template <typename T> __device__ __forceinline__ void st_out(T* p, T x) { st_s<RS_NT_OUT>(p, x); }

// How the fused step stores the updated state (the values are the same
// whichever is used).  Plain: ordinary stores, which L2 holds as dirty lines
// until it evicts them or the launch ends.  Write-through (sc1, system
// coherence scope): the lines go on to memory as they are written, so the
// launch does not end with L2 full of dirty state to write back; the fused
// step over a 25 M-param block runs 2.5 % faster and the 7B shard about 2 %.
// Non-temporal write-through (nt and sc1): the same, streamed; the better of
// the two where writes are close to half the traffic (the 70B shard's
// 14 of 30 bytes per param).  Under either, the bf16 copy is written through
// and streamed as well (another 1 % on the 25 M-param block and the 70B
// shard).
enum StorePolicy : int { kStPlain = 0, kStWriteThrough = 1, kStNtWriteThrough = 2 };

// A wave-uniform copy of a pointer that every active lane holds alike.
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
    const uintptr_t u = reinterpret_cast<uintptr_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
    return reinterpret_cast<P*>((static_cast<uintptr_t>(hi) << 32) | lo);
}

// This lane's group of 4 fp32 state values at `lane_ptr`, which is the
// group's base plus 4 * threadIdx.x elements, stored under policy POL: a raw
// buffer store from the group's uniform base (the cache-policy bits are an
// immediate of the buffer store: sc1 = 16, nt = 2), or an ordinary store.
template <int POL>
__device__ __forceinline__ void st_state_pol(float* lane_ptr, const f32x4& x) {
    if constexpr (POL == kStPlain) {
        st_state(reinterpret_cast<f32x4*>(lane_ptr), x);
    } else {
        constexpr int kAux = POL == kStWriteThrough ? 16 : 16 | 2;
        float* base = uniform_ptr(lane_ptr - threadIdx.x * kGroup);
        // raw buffer: no format conversion, unbounded within 2 GiB of the base
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r,
                                               static_cast<int>(threadIdx.x) * 16, 0, kAux);
    }
}

// This lane's 4 bf16 of the all-gather copy at `lane_ptr` (the group's base
// plus 4 * threadIdx.x elements, 8-byte aligned), written through to memory
// and streamed (nt and sc1): under a write-through state policy the copy
// leaves no dirty lines either.
__device__ __forceinline__ void st_bf16_wt(uint16_t* lane_ptr, const u32x2& x) {
    uint16_t* base = uniform_ptr(lane_ptr - threadIdx.x * kGroup);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b64(x, r, static_cast<int>(threadIdx.x) * 8, 0, 16 | 2);
}

// This lane's 4 fp8 codes at `lane_ptr` (the group's base plus 4 *
// threadIdx.x bytes, 4-byte aligned), written through and streamed.
__device__ __forceinline__ void st_fp8_wt(uint8_t* lane_ptr, uint32_t x) {
    uint8_t* base = uniform_ptr(lane_ptr - threadIdx.x * kGroup);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b32(x, r, static_cast<int>(threadIdx.x) * 4, 0, 16 | 2);
}

// Sums and maxima over the wave in a fixed order (xor-shuffle steps); every
// lane ends with the result.
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x = std::max(x, static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), off)));
    return x;
}

// ---------------------------------------------------------------- 4-element groups

// One group of a slice: 4 bf16 in 8 bytes or 4 fp32 in 16 bytes.
template <bool BF16> struct SliceVecT { using type = u32x4; };
template <> struct SliceVecT<true> { using type = u32x2; };
template <bool BF16> using SliceVec = typename SliceVecT<BF16>::type;

template <bool BF16>
__device__ __forceinline__ SliceVec<BF16> load_group(const void* base, int64_t i) {
    using V = SliceVec<BF16>;
    if constexpr (BF16) return ld_slice(reinterpret_cast<const V*>(static_cast<const uint16_t*>(base) + i));
    else return ld_slice(reinterpret_cast<const V*>(static_cast<const float*>(base) + i));
}

// The group starting `sh` bytes into A (0 <= sh < sizeof A, a multiple of
// the element size), given A and the vector B that follows it; A itself
// when sh is 0.
template <bool BF16>
__device__ __forceinline__ SliceVec<BF16> join_shifted(const SliceVec<BF16>& A, const SliceVec<BF16>& B,
                                                       uint32_t sh) {
    if constexpr (BF16) {
        // sh = 0, 2, 4 or 6: dword offset w, byte offset b within it
        const bool w = sh >= 4;
        const uint32_t b = sh & 3u;
        const uint32_t x0 = w ? A[1] : A[0];
        const uint32_t x1 = w ? B[0] : A[1];
        const uint32_t x2 = w ? B[1] : B[0];
        return u32x2{__builtin_amdgcn_alignbyte(x1, x0, b), __builtin_amdgcn_alignbyte(x2, x1, b)};
    } else {
        // sh = 0, 4, 8 or 12: whole dwords
        const bool d0 = sh == 0, d1 = sh == 4, d2 = sh == 8;
        return u32x4{d0 ? A[0] : (d1 ? A[1] : (d2 ? A[2] : A[3])),
                     d0 ? A[1] : (d1 ? A[2] : (d2 ? A[3] : B[0])),
                     d0 ? A[2] : (d1 ? A[3] : (d2 ? B[0] : B[1])),
                     d0 ? A[3] : (d1 ? B[0] : (d2 ? B[1] : B[2]))};
    }
}

// The parts of a group load at any element alignment.  `lo` is the aligned
// vector at or before the group (the group itself when aligned), `hi` the
// address of the next vector when the group spans two (else lo again, so
// that no load leaves the group's vectors), and `sh` the group's offset in
// bytes past `lo`.
struct AnyGroup {
    uintptr_t lo, hi;
    uint32_t sh;
};

template <bool BF16>
__device__ __forceinline__ AnyGroup any_group(const void* base, int64_t i) {
    constexpr uintptr_t W = sizeof(SliceVec<BF16>);
    const uint32_t sh = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(base) & (W - 1));
    const uintptr_t lo = reinterpret_cast<uintptr_t>(base) + static_cast<uintptr_t>(i) * (W / kGroup) - sh;
    return AnyGroup{lo, sh ? lo + W : lo, sh};
}

// Groups at element e of the slices j < min(K, n), each slice at any element
// alignment (base(j) gives slice j's start), into w[].  Every lane loads the
// two aligned vectors that hold its group (the group's own vector twice
// when it is aligned), all loads before the first join: no test on a
// slice's alignment sits between them.  Each vector loaded holds bytes of
// the group, so none reaches past the page (or the allocation) the slice
// lies in.
template <int K, bool BF16, typename Base>
__device__ __forceinline__ void load_any(SliceVec<BF16> w[K], Base&& base, int n, int64_t e) {
    using V = SliceVec<BF16>;
    AnyGroup g[K];
    V A[K], B[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        if (j < n) {
            g[j] = any_group<BF16>(base(j), e);
            A[j] = ld_slice(reinterpret_cast<const V*>(g[j].lo));
            B[j] = ld_slice(reinterpret_cast<const V*>(g[j].hi));
        }
    }
#pragma unroll
    for (int j = 0; j < K; ++j)
        if (j < n) w[j] = join_shifted<BF16>(A[j], B[j], g[j].sh);
}

template <bool BF16>
__device__ __forceinline__ void widen(const SliceVec<BF16>& w, float x[kGroup]) {
    if constexpr (BF16) {
        x[0] = bf16_lo(w[0]);
        x[1] = bf16_hi(w[0]);
        x[2] = bf16_lo(w[1]);
        x[3] = bf16_hi(w[1]);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = __uint_as_float(w[j]);
    }
}

// Raw slice data of one group, loaded before any arithmetic.
template <int NS, bool BF16>
struct SliceRegs {
    SliceVec<BF16> w[NS > 0 ? NS : 1];
};

// Start of slice q of a shard.  TABLE: the shard has a table of slice
// pointers (N receive buffers that need not share an allocation), read
// through the constant address space, so the uniform entries arrive by
// scalar loads.  Otherwise q slice strides past the first slice.  The
// kernels choose TABLE once per tile, on the shard's uniform descriptor, so
// the stride form's code is the same as without tables.
template <typename T>
using const_ptr = const __attribute__((address_space(4))) T*;

template <bool BF16, bool TABLE>
__device__ __forceinline__ const void* slice_base(const TensorDesc& T, int q) {
    if constexpr (TABLE) {
        return *(const_ptr<const void*>)(T.slice_ptrs + q);
    } else {
        using E = typename std::conditional<BF16, uint16_t, float>::type;
        return static_cast<const E*>(T.slices) + q * T.slice_stride;
    }
}

// GEN: the slices may start at any element alignment.
template <int NS, bool BF16, bool TABLE, bool GEN = false>
__device__ __forceinline__ void load_slices(SliceRegs<NS, BF16>& r, const TensorDesc& T,
                                            int64_t e) {
    static_assert(NS > 0, "compile-time slice count");
    if constexpr (GEN) {
        load_any<NS, BF16>(r.w, [&](int q) { return slice_base<BF16, TABLE>(T, q); }, NS, e);
    } else {
#pragma unroll
        for (int q = 0; q < NS; ++q) r.w[q] = load_group<BF16>(slice_base<BF16, TABLE>(T, q), e);
    }
}

template <int NS, bool BF16>
__device__ __forceinline__ void reduce_regs(const SliceRegs<NS, BF16>& r, float g[kGroup],
                                            const StepConsts& c) {
    widen<BF16>(r.w[0], g);
#pragma unroll
    for (int q = 1; q < NS; ++q) {
        float x[kGroup];
        widen<BF16>(r.w[q], x);
#pragma unroll
        for (int j = 0; j < kGroup; ++j) g[j] = g[j] + x[j];
    }
#pragma unroll
    for (int j = 0; j < kGroup; ++j) g[j] = finish_mean(g[j], c);
}

// Slices per batch of the runtime slice-count loop.
template <bool BF16>
constexpr int rt_batch() {
    return std::max<int>(1, RS_RT_BATCH_BYTES / static_cast<int>(sizeof(SliceVec<BF16>)));
}

// Runtime slice count: the slices in batches of rt_batch().  Every load of a
// batch is issued before the batch's first add, and the adds run in slice
// order, so the sum is the one taken slice by slice.  The batch bounds are
// uniform, so the tests on them are scalar branches.
template <bool BF16, bool TABLE, bool GEN = false>
__device__ __forceinline__ void reduce_runtime(const TensorDesc& T, int64_t e, float g[kGroup],
                                               const StepConsts& c) {
    constexpr int KB = rt_batch<BF16>();
    for (int q0 = 0; q0 < c.n; q0 += KB) {
        SliceVec<BF16> w[KB];
        if constexpr (GEN) {
            load_any<KB, BF16>(w, [&](int j) { return slice_base<BF16, TABLE>(T, q0 + j); }, c.n - q0, e);
        } else {
#pragma unroll
            for (int j = 0; j < KB; ++j)
                if (q0 + j < c.n) w[j] = load_group<BF16>(slice_base<BF16, TABLE>(T, q0 + j), e);
        }
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            if (q0 + j < c.n) {
                float x[kGroup];
                widen<BF16>(w[j], x);
                if (j == 0 && q0 == 0) {
#pragma unroll
                    for (int k = 0; k < kGroup; ++k) g[k] = x[k];
                } else {
#pragma unroll
                    for (int k = 0; k < kGroup; ++k) g[k] = g[k] + x[k];
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kGroup; ++j) g[j] = finish_mean(g[j], c);
}

// The mean of the slices on the group at e, N known at compile time or not.
template <int NS, bool BF16, bool TABLE = false, bool GEN = false>
__device__ __forceinline__ void reduce_group(const TensorDesc& T, int64_t e, float g[kGroup],
                                             const StepConsts& c) {
    if constexpr (NS > 0) {
        SliceRegs<NS, BF16> sr;
        load_slices<NS, BF16, TABLE, GEN>(sr, T, e);
        reduce_regs<NS, BF16>(sr, g, c);
    } else {
        reduce_runtime<BF16, TABLE, GEN>(T, e, g, c);
    }
}

struct StateRegs {
    f32x4 p, m, v;
};

__device__ __forceinline__ void load_state(StateRegs& s, const TensorDesc& T, int64_t e) {
    s.p = ld_state(reinterpret_cast<const f32x4*>(T.param + e));
    s.m = ld_state(reinterpret_cast<const f32x4*>(T.m + e));
    s.v = ld_state(reinterpret_cast<const f32x4*>(T.v + e));
}

__device__ __forceinline__ u32x2 pack_bf16(const f32x4& p) {
    return u32x2{bf16_rne(p[0]) | (bf16_rne(p[1]) << 16), bf16_rne(p[2]) | (bf16_rne(p[3]) << 16)};
}

// The 4 bf16 of a group (w, element j in half j) at p, which lies `sh` bytes
// past an 8-byte boundary (sh uniform, from the copy's base).  Unaligned:
// 4-byte pieces where the address allows, 2-byte ones at the ends.
__device__ __forceinline__ void store_bf16_any(uint16_t* p, const u32x2& w, uint32_t sh) {
    if (sh == 0) {
        st_out(reinterpret_cast<u32x2*>(p), w);
    } else if (sh == 4) {
        st_out(reinterpret_cast<uint32_t*>(p), w[0]);
        st_out(reinterpret_cast<uint32_t*>(p + 2), w[1]);
    } else {
        st_out(p, static_cast<uint16_t>(w[0]));
        st_out(reinterpret_cast<uint32_t*>(p + 1), (w[0] >> 16) | (w[1] << 16));
        st_out(p + 3, static_cast<uint16_t>(w[1] >> 16));
    }
}

// The 4 fp8 codes of a group (byte j of w) at p, `sh` bytes past a 4-byte
// boundary (uniform).
__device__ __forceinline__ void store_fp8_any(uint8_t* p, uint32_t w, uint32_t sh) {
    if (sh == 0) {
        st_out(reinterpret_cast<uint32_t*>(p), w);
    } else if (sh == 2) {
        st_out(reinterpret_cast<uint16_t*>(p), static_cast<uint16_t>(w));
        st_out(reinterpret_cast<uint16_t*>(p + 2), static_cast<uint16_t>(w >> 16));
    } else {
        st_out(p, static_cast<uint8_t>(w));
        st_out(reinterpret_cast<uint16_t*>(p + 1), static_cast<uint16_t>(w >> 8));
        st_out(p + 3, static_cast<uint8_t>(w >> 24));
    }
}

__device__ __forceinline__ uint32_t misalign(const void* p, uintptr_t w) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p) & (w - 1));
}

// AdamW on a group and the stores of its results.  WRITE_G: also store the
// reduced gradient when the shard has a grad_shard_out.
// AMAX: also fold |p'| of the group into *amax (fp32 bit patterns of
// non-negative values order like the values; NaN patterns sort above all).
// FP8: also store the fp8 codes of p' with the given per-tensor scale.
// GEN: the low-precision copies may start at any element alignment.
template <bool WRITE_G = true, bool AMAX = false, bool FP8 = false, bool GEN = false, int POL = kStPlain>
__device__ __forceinline__ void update_store(StateRegs& s, const float g[kGroup],
                                             const TensorDesc& T, int64_t e, const StepConsts& c,
                                             uint32_t* amax = nullptr, float fp8_scale = 0.0f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float p = s.p[j], m = s.m[j], v = s.v[j];
        adamw(p, m, v, g[j], c);
        s.p[j] = p;
        s.m[j] = m;
        s.v[j] = v;
        if constexpr (AMAX) *amax = std::max(*amax, __float_as_uint(p) & 0x7fffffffu);
    }
    st_state_pol<POL>(T.param + e, s.p);
    st_state_pol<POL>(T.m + e, s.m);
    st_state_pol<POL>(T.v + e, s.v);
    if (T.out_bf16) {
        if constexpr (GEN) store_bf16_any(T.out_bf16 + e, pack_bf16(s.p), misalign(T.out_bf16, 8));
        else if constexpr (POL != kStPlain) st_bf16_wt(T.out_bf16 + e, pack_bf16(s.p));
        else st_out(reinterpret_cast<u32x2*>(T.out_bf16 + e), pack_bf16(s.p));
    }
    if constexpr (FP8) {
        if (T.out_fp8) {
            if constexpr (GEN) store_fp8_any(T.out_fp8 + e, pack_fp8(s.p, fp8_scale), misalign(T.out_fp8, 4));
            else if constexpr (POL != kStPlain) st_fp8_wt(T.out_fp8 + e, pack_fp8(s.p, fp8_scale));
            else st_out(reinterpret_cast<uint32_t*>(T.out_fp8 + e), pack_fp8(s.p, fp8_scale));
        }
    }
    if (WRITE_G && T.grad_out) {
        if constexpr (POL != kStPlain) st_state_pol<kStNtWriteThrough>(T.grad_out + e, f32x4{g[0], g[1], g[2], g[3]});
        else st_out(reinterpret_cast<f32x4*>(T.grad_out + e), f32x4{g[0], g[1], g[2], g[3]});
    }
}

// ---------------------------------------------------------------- single elements

template <bool BF16>
__device__ __forceinline__ float slice_elem(const void* slices, int64_t i) {
    if constexpr (BF16) {
        return __uint_as_float(static_cast<uint32_t>(ld(static_cast<const uint16_t*>(slices) + i)) << 16);
    } else {
        return ld(static_cast<const float*>(slices) + i);
    }
}

template <bool BF16, bool TABLE = false>
__device__ __forceinline__ float reduce_elem(const TensorDesc& T, int64_t k, const StepConsts& c) {
    float s = slice_elem<BF16>(slice_base<BF16, TABLE>(T, 0), k);
    for (int q = 1; q < c.n; ++q) s = s + slice_elem<BF16>(slice_base<BF16, TABLE>(T, q), k);
    return finish_mean(s, c);
}

// The whole fused step on element k (any alignment); +0 everywhere in the pad
// (fp8 code 0).
template <bool BF16, bool AMAX = false, bool FP8 = false, bool TABLE = false>
__device__ __forceinline__ void fused_elem(const TensorDesc& T, int64_t k, const StepConsts& c,
                                           uint32_t* amax = nullptr, float fp8_scale = 0.0f) {
    if (k < T.valid) {
        const float g = reduce_elem<BF16, TABLE>(T, k, c);
        float p = ld(T.param + k), m = ld(T.m + k), v = ld(T.v + k);
        adamw(p, m, v, g, c);
        if constexpr (AMAX) *amax = std::max(*amax, __float_as_uint(p) & 0x7fffffffu);
        st(T.param + k, p);
        st(T.m + k, m);
        st(T.v + k, v);
        if (T.out_bf16) st(T.out_bf16 + k, static_cast<uint16_t>(bf16_rne(p)));
        if (FP8 && T.out_fp8) st(T.out_fp8 + k, static_cast<uint8_t>(fp8_code(p, fp8_scale)));
        if (T.grad_out) st(T.grad_out + k, g);
    } else {
        st(T.param + k, 0.0f);
        st(T.m + k, 0.0f);
        st(T.v + k, 0.0f);
        if (T.out_bf16) st(T.out_bf16 + k, uint16_t(0));
        if (FP8 && T.out_fp8) st(T.out_fp8 + k, uint8_t(0));
        if (T.grad_out) st(T.grad_out + k, 0.0f);
    }
}

// AdamW on element k from the stored reduced gradient times `scale` (the clip
// coefficient); +0 everywhere in the pad.  The gradient buffer is not written.
__device__ __forceinline__ void scaled_elem(const TensorDesc& T, int64_t k, float scale,
                                            const StepConsts& c) {
    if (k < T.valid) {
        const float g = ld(T.grad_out + k) * scale;
        float p = ld(T.param + k), m = ld(T.m + k), v = ld(T.v + k);
        adamw(p, m, v, g, c);
        st(T.param + k, p);
        st(T.m + k, m);
        st(T.v + k, v);
        if (T.out_bf16) st(T.out_bf16 + k, static_cast<uint16_t>(bf16_rne(p)));
    } else {
        st(T.param + k, 0.0f);
        st(T.m + k, 0.0f);
        st(T.v + k, 0.0f);
        if (T.out_bf16) st(T.out_bf16 + k, uint16_t(0));
    }
}

// ---------------------------------------------------------------- ranges of a shard

// End of the vector part of [begin, end): whole groups below `valid` when the
// shard's fp32 buffers are aligned for vectors; the rest (the partial group
// at `valid`, the padding, shards whose fp32 buffers are not) goes element
// by element.
__device__ __forceinline__ int64_t vector_end(const TensorDesc& T, int64_t begin, int64_t end) {
    const int64_t vend = T.vec_ok ? std::min(end, T.valid & ~int64_t(kGroup - 1)) : begin;
    return std::max(vend, begin);
}

// The fused step on elements [begin, end) of shard T; `begin` is a multiple of
// kGroup.  AMAX and FP8 as in update_store, GEN_ST as its GEN; TABLE as in
// slice_base; GEN_LD: the slices may start at any element alignment.
template <int NS, bool BF16, bool AMAX = false, bool FP8 = false, bool TABLE = false,
          bool GEN_LD = false, bool GEN_ST = false, int POL = kStPlain>
__device__ __forceinline__ void fused_range(const TensorDesc& T, int64_t begin, int64_t end,
                                            const StepConsts& c, uint32_t* amax = nullptr,
                                            float fp8_scale = 0.0f) {
    const int64_t vend = vector_end(T, begin, end);
    for (int64_t e = begin + threadIdx.x * kGroup; e < vend; e += kTile) {
        StateRegs s;
        if constexpr (NS > 0) {
            // every load of the group before the first arithmetic
            SliceRegs<NS, BF16> sr;
            load_slices<NS, BF16, TABLE, GEN_LD>(sr, T, e);
            load_state(s, T, e);
            float g[kGroup];
            reduce_regs<NS, BF16>(sr, g, c);
            update_store<true, AMAX, FP8, GEN_ST, POL>(s, g, T, e, c, amax, fp8_scale);
        } else {
            load_state(s, T, e);
            float g[kGroup];
            reduce_runtime<BF16, TABLE, GEN_LD>(T, e, g, c);
            update_store<true, AMAX, FP8, GEN_ST, POL>(s, g, T, e, c, amax, fp8_scale);
        }
    }
    for (int64_t k = vend + threadIdx.x; k < end; k += kBlock)
        fused_elem<BF16, AMAX, FP8, TABLE>(T, k, c, amax, fp8_scale);
}

// Reduce only: grad_out = mean of the slices on [begin, end); GEN: the
// slices may start at any element alignment.
template <int NS, bool BF16, bool GEN = false, int POL = kStPlain>
__device__ __forceinline__ void reduce_range(const TensorDesc& T, int64_t begin, int64_t end,
                                             const StepConsts& c) {
    const int64_t vend = vector_end(T, begin, end);
    for (int64_t e = begin + threadIdx.x * kGroup; e < vend; e += kTile) {
        float g[kGroup];
        reduce_group<NS, BF16, false, GEN>(T, e, g, c);
        if constexpr (POL != kStPlain) st_state_pol<POL>(T.grad_out + e, f32x4{g[0], g[1], g[2], g[3]});
        else st_out(reinterpret_cast<f32x4*>(T.grad_out + e), f32x4{g[0], g[1], g[2], g[3]});
    }
    for (int64_t k = vend + threadIdx.x; k < end; k += kBlock)
        st(T.grad_out + k, k < T.valid ? reduce_elem<BF16>(T, k, c) : 0.0f);
}

// Reduce into grad_out on [begin, end): with `acc` the mean of the slices
// is added to what grad_out holds (one fp32 add, old + new: gradient
// accumulation over micro-batches), else it replaces it.  SQ: return this
// lane's sum of the squares of the stored values, in fp64 (each fp32
// square is exact in fp64).  The padding is +0 either way.
template <int NS, bool BF16, bool SQ, bool TABLE = false, bool GEN = false, int POL = kStPlain>
__device__ __forceinline__ double reduce_store_range(const TensorDesc& T, int64_t begin,
                                                     int64_t end, const StepConsts& c, bool acc) {
    double sq = 0.0;
    const int64_t vend = vector_end(T, begin, end);
    for (int64_t e = begin + threadIdx.x * kGroup; e < vend; e += kTile) {
        f32x4* go = reinterpret_cast<f32x4*>(T.grad_out + e);
        f32x4 old = {0.f, 0.f, 0.f, 0.f};
        if (acc) old = ld_s<RS_NT_ACC_LD>(go);
        float g[kGroup];
        reduce_group<NS, BF16, TABLE, GEN>(T, e, g, c);
        if (acc) {
#pragma unroll
            for (int j = 0; j < kGroup; ++j) g[j] = old[j] + g[j];
        }
        if constexpr (POL != kStPlain) st_state_pol<POL>(T.grad_out + e, f32x4{g[0], g[1], g[2], g[3]});
        else st_out(go, f32x4{g[0], g[1], g[2], g[3]});
        if constexpr (SQ) {
#pragma unroll
            for (int j = 0; j < kGroup; ++j) sq += static_cast<double>(g[j]) * static_cast<double>(g[j]);
        }
    }
    for (int64_t k = vend + threadIdx.x; k < end; k += kBlock) {
        float gk = 0.0f;
        if (k < T.valid) {
            gk = reduce_elem<BF16, TABLE>(T, k, c);
            if (acc) gk = ld(T.grad_out + k) + gk;
        }
        st(T.grad_out + k, gk);
        if constexpr (SQ) sq += static_cast<double>(gk) * static_cast<double>(gk);
    }
    return sq;
}

// In-place accumulation of one micro-batch's unsharded gradient, elements
// [begin, end): acc = acc + x (fp32 add), or acc = x exactly for the first.
// GEN: x may start at any element alignment (acc is aligned).
template <bool BF16, bool GEN = false, int POL = kStPlain>
__device__ __forceinline__ void accumulate_range(float* a, const void* x, int64_t begin,
                                                 int64_t end, bool accum, bool vec) {
    const int64_t vend = vec ? std::max(begin, end & ~int64_t(kGroup - 1)) : begin;
    for (int64_t e = begin + threadIdx.x * kGroup; e < vend; e += kTile) {
        f32x4* ap = reinterpret_cast<f32x4*>(a + e);
        SliceVec<BF16> w;
        if constexpr (GEN) load_any<1, BF16>(&w, [&](int) { return x; }, 1, e);
        else w = load_group<BF16>(x, e);
        f32x4 av = {0.f, 0.f, 0.f, 0.f};
        if (accum) av = ld_state(ap);
        float xv[kGroup];
        widen<BF16>(w, xv);
#pragma unroll
        for (int j = 0; j < kGroup; ++j) av[j] = accum ? av[j] + xv[j] : xv[j];
        if constexpr (POL != kStPlain) st_state_pol<POL>(a + e, av);
        else st_state(ap, av);
    }
    for (int64_t k = vend + threadIdx.x; k < end; k += kBlock) {
        const float xk = slice_elem<BF16>(x, k);
        st(a + k, accum ? ld(a + k) + xk : xk);
    }
}

// AdamW + cast on [begin, end) from the stored reduced gradient times `scale`.
template <bool GEN = false, int POL = kStPlain>
__device__ __forceinline__ void scaled_range(const TensorDesc& T, int64_t begin, int64_t end,
                                             float scale, const StepConsts& c) {
    const int64_t vend = vector_end(T, begin, end);
    for (int64_t e = begin + threadIdx.x * kGroup; e < vend; e += kTile) {
        const f32x4 gv = ld_slice(reinterpret_cast<const f32x4*>(T.grad_out + e));
        StateRegs s;
        load_state(s, T, e);
        float g[kGroup];
#pragma unroll
        for (int j = 0; j < kGroup; ++j) g[j] = gv[j] * scale;
        update_store<false, false, false, GEN, POL>(s, g, T, e, c);
    }
    for (int64_t k = vend + threadIdx.x; k < end; k += kBlock) scaled_elem(T, k, scale, c);
}

// fp8 copy of the updated shard on [begin, end), at most TILES tiles; codes 0
// in the pad.  Each lane loads all of its groups before converting any.
template <int TILES, bool GEN = false, int POL = kStPlain>
__device__ __forceinline__ void fp8_range(const TensorDesc& T, int64_t begin, int64_t end,
                                          float scale) {
    const int64_t vend = vector_end(T, begin, end);
    f32x4 a[TILES];
#pragma unroll
    for (int u = 0; u < TILES; ++u) {
        const int64_t e = begin + (u * kBlock + threadIdx.x) * kGroup;
        if (e < vend) a[u] = ld_s<RS_NT_CAST_LD>(reinterpret_cast<const f32x4*>(T.param + e));
    }
#pragma unroll
    for (int u = 0; u < TILES; ++u) {
        const int64_t e = begin + (u * kBlock + threadIdx.x) * kGroup;
        if (e < vend) {
            if constexpr (GEN) store_fp8_any(T.out_fp8 + e, pack_fp8(a[u], scale), misalign(T.out_fp8, 4));
            else if constexpr (POL != kStPlain) st_fp8_wt(T.out_fp8 + e, pack_fp8(a[u], scale));
            else st_out(reinterpret_cast<uint32_t*>(T.out_fp8 + e), pack_fp8(a[u], scale));
        }
    }
    for (int64_t k = vend + threadIdx.x; k < end; k += kBlock)
        st(T.out_fp8 + k, k < T.valid ? static_cast<uint8_t>(fp8_code(ld(T.param + k), scale))
                                      : uint8_t(0));
}

// Cast only: out_bf16 = RNE(param) on [begin, end); GEN: the copy may start
// at any element alignment.
template <bool GEN = false, int POL = kStPlain>
__device__ __forceinline__ void cast_range(const TensorDesc& T, int64_t begin, int64_t end) {
    const int64_t vend = vector_end(T, begin, end);
    for (int64_t e = begin + threadIdx.x * kGroup; e < vend; e += kTile) {
        const f32x4 a = ld_s<RS_NT_CAST_LD>(reinterpret_cast<const f32x4*>(T.param + e));
        if constexpr (GEN) store_bf16_any(T.out_bf16 + e, pack_bf16(a), misalign(T.out_bf16, 8));
        else if constexpr (POL != kStPlain) st_bf16_wt(T.out_bf16 + e, pack_bf16(a));
        else st_out(reinterpret_cast<u32x2*>(T.out_bf16 + e), pack_bf16(a));
    }
    for (int64_t k = vend + threadIdx.x; k < end; k += kBlock)
        st(T.out_bf16 + k, k < T.valid ? static_cast<uint16_t>(bf16_rne(ld(T.param + k))) : uint16_t(0));
}

// ---------------------------------------------------------------- kernels

// Runs f(T, begin, end) on this workgroup's span of TILES tiles: span
// b % (8 / TILES) of chunk entry b / (8 / TILES), which names a shard and an
// element range of it.  The range is empty for spans past the end of a
// shard's last, shorter entry.  Every value here is uniform, so the entry and
// the descriptor arrive by scalar loads.
template <int TILES = 1, typename F>
__device__ __forceinline__ void for_my_tile(const TensorDesc* __restrict__ tensors,
                                            const ChunkDesc* __restrict__ chunks, F&& f) {
    static_assert(TILES >= 1 && kTilesPerChunk % TILES == 0, "spans tile a chunk entry");
    constexpr int kSpans = kTilesPerChunk / TILES;
    const uint32_t b = blockIdx.x;
    const ChunkDesc cd = chunks[b / kSpans];
    const TensorDesc T = tensors[cd.tensor];
    const int32_t lo = static_cast<int32_t>(b % kSpans) * (TILES * kTile);
    const int32_t n = std::max(0, std::min(TILES * kTile, cd.count - lo));
    f(T, cd.begin + lo, cd.begin + lo + n);
}

// Slot of workgroup b's partial result among n (a multiple of 8).  Workgroups
// are dealt to the 8 XCDs round-robin, so XCD-major slots let each XCD's L2
// gather its workgroups' small stores into whole lines before writing back.
constexpr int kXcds = 8;
static_assert(kTilesPerChunk % kXcds == 0, "plan launches hold a multiple of 8 workgroups");
__device__ __forceinline__ uint32_t xcd_slot(uint32_t b, uint32_t n) {
    return (b % kXcds) * (n / kXcds) + b / kXcds;
}

// The fused step on one tile.  GENERAL: some shard of the plan reads its
// slices through a table of pointers, or has a slice or a low-precision copy
// that is not vector-aligned; the form is then chosen per tile from the
// shard's descriptor.  Plans with neither run the plain form only, compiled
// without the others.
template <int NS, bool BF16, bool AMAX, bool FP8, bool GENERAL, int POL = kStPlain>
__device__ __forceinline__ void fused_tile(const TensorDesc& T, int64_t b, int64_t e, const StepConsts& c,
                                           uint32_t* amax = nullptr, float fp8_scale = 0.0f) {
    if constexpr (GENERAL) {
        if (T.slice_ptrs) {
            if (T.gen & kGenLoad) fused_range<NS, BF16, AMAX, FP8, true, true, true, POL>(T, b, e, c, amax, fp8_scale);
            else if (T.gen) fused_range<NS, BF16, AMAX, FP8, true, false, true, POL>(T, b, e, c, amax, fp8_scale);
            else fused_range<NS, BF16, AMAX, FP8, true, false, false, POL>(T, b, e, c, amax, fp8_scale);
            return;
        }
        if (T.gen & kGenLoad) {
            fused_range<NS, BF16, AMAX, FP8, false, true, true, POL>(T, b, e, c, amax, fp8_scale);
            return;
        }
        if (T.gen) {
            fused_range<NS, BF16, AMAX, FP8, false, false, true, POL>(T, b, e, c, amax, fp8_scale);
            return;
        }
    }
    fused_range<NS, BF16, AMAX, FP8, false, false, false, POL>(T, b, e, c, amax, fp8_scale);
}

// The step's scalars: those passed by value, or (DEVC: a step whose count is
// in device memory) those the count kernel derived at *cdev.  DEVC is a
// template argument so that the by-value kernels carry no test of cdev.
template <bool DEVC>
__device__ __forceinline__ StepConsts step_consts(const StepConsts& c, const StepConsts* cdev) {
    if constexpr (DEVC) return *cdev;
    else return c;
}

// Multi-tensor fused step: reduce, AdamW and cast for every tile.
template <int NS, bool BF16, bool GENERAL, int POL, bool DEVC>
__global__ __launch_bounds__(kBlock) void mt_step_kernel(const TensorDesc* __restrict__ tensors,
                                                         const ChunkDesc* __restrict__ chunks,
                                                         StepConsts c_arg, const StepConsts* cdev) {
    const StepConsts c = step_consts<DEVC>(c_arg, cdev);
    for_my_tile(tensors, chunks, [&](const TensorDesc& T, int64_t b, int64_t e) {
        fused_tile<NS, BF16, false, false, GENERAL, POL>(T, b, e, c);
    });
}

// The fused step on a plan whose shards lie back to back in every buffer,
// as one range T: workgroup b covers elements [b*kTile, (b+1)*kTile).  The
// elements and their arithmetic are those of mt_step_kernel; only the way a
// workgroup finds its tile differs.
template <int NS, bool BF16, int POL, bool DEVC>
__global__ __launch_bounds__(kBlock) void run_step_kernel(TensorDesc T, StepConsts c_arg,
                                                          const StepConsts* cdev) {
    const StepConsts c = step_consts<DEVC>(c_arg, cdev);
    const int64_t begin = static_cast<int64_t>(blockIdx.x) * kTile;
    fused_range<NS, BF16, false, false, false, false, false, POL>(
        T, begin, std::min<int64_t>(begin + kTile, T.shard_numel), c);
}

// Reduce (or reduce and accumulate) into grad_shard_out; SQ: also write
// this workgroup's sum of squares of the stored values to its partials slot.
template <int NS, bool BF16, bool SQ, bool GENERAL, int POL>
__global__ __launch_bounds__(kBlock) void mt_reduce_store_kernel(const TensorDesc* __restrict__ tensors,
                                                                 const ChunkDesc* __restrict__ chunks,
                                                                 StepConsts c, int32_t acc,
                                                                 double* partials) {
    double sq = 0.0;
    for_my_tile(tensors, chunks, [&](const TensorDesc& T, int64_t b, int64_t e) {
        const bool a = acc != 0;
        if (GENERAL && T.slice_ptrs)
            sq = T.gen & kGenLoad ? reduce_store_range<NS, BF16, SQ, true, true, POL>(T, b, e, c, a)
                                  : reduce_store_range<NS, BF16, SQ, true, false, POL>(T, b, e, c, a);
        else if (GENERAL && (T.gen & kGenLoad))
            sq = reduce_store_range<NS, BF16, SQ, false, true, POL>(T, b, e, c, a);
        else
            sq = reduce_store_range<NS, BF16, SQ, false, false, POL>(T, b, e, c, a);
    });
    if constexpr (SQ) {
        const double total = wave_sum(sq);
        if (threadIdx.x == 0) st(partials + xcd_slot(blockIdx.x, gridDim.x), total);
    }
}

// Workgroup b accumulates elements [b*kTile, (b+1)*kTile) of one buffer.
template <bool BF16, bool GEN, int POL>
__global__ __launch_bounds__(kBlock) void accumulate_kernel(float* a, const void* x, int64_t n,
                                                            int32_t accum, int32_t vec) {
    const int64_t begin = static_cast<int64_t>(blockIdx.x) * kTile;
    accumulate_range<BF16, GEN, POL>(a, x, begin, std::min(begin + kTile, n), accum != 0,
                                                     vec != 0);
}

// Pass 2 of a clipped step: AdamW and cast from grad_shard_out times *scale.
template <bool GENERAL, int POL, bool DEVC>
__global__ __launch_bounds__(kBlock) void mt_scaled_step_kernel(const TensorDesc* __restrict__ tensors,
                                                                const ChunkDesc* __restrict__ chunks,
                                                                StepConsts c_arg, const float* scale,
                                                                const StepConsts* cdev) {
    const StepConsts c = step_consts<DEVC>(c_arg, cdev);
    const float k = *scale;
    for_my_tile(tensors, chunks, [&](const TensorDesc& T, int64_t b, int64_t e) {
        if (GENERAL && (T.gen & kGenStore)) scaled_range<true, POL>(T, b, e, k, c);
        else scaled_range<false, POL>(T, b, e, k, c);
    });
}

// The fused step that also records, per workgroup, the largest |p'| (as
// fp32 bits, in the workgroup's slot) for the fp8 copy's per-tensor scale.
template <int NS, bool BF16, bool GENERAL, int POL, bool DEVC>
__global__ __launch_bounds__(kBlock) void mt_step_amax_kernel(const TensorDesc* __restrict__ tensors,
                                                              const ChunkDesc* __restrict__ chunks,
                                                              StepConsts c_arg, uint32_t* tile_amax,
                                                              const StepConsts* cdev) {
    const StepConsts c = step_consts<DEVC>(c_arg, cdev);
    uint32_t am = 0;
    for_my_tile(tensors, chunks, [&](const TensorDesc& T, int64_t b, int64_t e) {
        fused_tile<NS, BF16, true, false, GENERAL, POL>(T, b, e, c, &am);
    });
    const uint32_t wm = wave_max(am);
    if (threadIdx.x == 0) st(tile_amax + xcd_slot(blockIdx.x, gridDim.x), wm);
}

// The fused step that also writes the fp8 codes of p' with a per-tensor scale
// given in advance (scale_in[index], e.g. from the previous step's amax) and
// records this step's per-workgroup largest |p'|, all in the one pass.
template <int NS, bool BF16, bool GENERAL, int POL, bool DEVC>
__global__ __launch_bounds__(kBlock) void mt_step_fp8_kernel(const TensorDesc* __restrict__ tensors,
                                                             const ChunkDesc* __restrict__ chunks,
                                                             StepConsts c_arg, const float* scale_in,
                                                             uint32_t* tile_amax, const StepConsts* cdev) {
    const StepConsts c = step_consts<DEVC>(c_arg, cdev);
    uint32_t am = 0;
    for_my_tile(tensors, chunks, [&](const TensorDesc& T, int64_t b, int64_t e) {
        const float scale = ld(scale_in + T.index);
        fused_tile<NS, BF16, true, true, GENERAL, POL>(T, b, e, c, &am, scale);
    });
    const uint32_t wm = wave_max(am);
    if (threadIdx.x == 0) st(tile_amax + xcd_slot(blockIdx.x, gridDim.x), wm);
}

// First workgroup and number of workgroups of each shard, by input position
// (both multiples of 8: a shard's chunk entries are whole).
struct ShardTiles {
    int64_t first;
    int64_t count;
};

constexpr int kAmaxBlock = 1024;        // threads of the per-shard amax reduction

// Workgroup i: amax_out[i] = max over shard i's workgroups (0 if empty).
// Their slots are XCD-major (see xcd_slot): one run of count/8 in each of the
// 8 regions of `region` slots.  A large shard has tens of thousands of them:
// each lane keeps four loads in flight, then the 16 waves combine through LDS.
__global__ __launch_bounds__(kAmaxBlock) void shard_amax_kernel(const ShardTiles* sc,
                                                                const uint32_t* tile_amax,
                                                                int64_t region, float* amax_out) {
    __shared__ uint32_t s_max[kAmaxBlock / 64];
    const ShardTiles r = sc[blockIdx.x];
    const int64_t run = r.count / kXcds;
    uint32_t m = 0;
    for (int x = 0; x < kXcds; ++x) {
        const uint32_t* p = tile_amax + x * region + r.first / kXcds;
        int64_t j = threadIdx.x;
        for (; j + 3 * kAmaxBlock < run; j += 4 * kAmaxBlock) {
            const uint32_t a = ld(p + j), b = ld(p + j + kAmaxBlock);
            const uint32_t c = ld(p + j + 2 * kAmaxBlock), d = ld(p + j + 3 * kAmaxBlock);
            m = std::max(std::max(m, std::max(a, b)), std::max(c, d));
        }
        for (; j < run; j += kAmaxBlock) m = std::max(m, ld(p + j));
    }
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x / 64] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kAmaxBlock / 64; ++w) t = std::max(t, s_max[w]);
        st(amax_out + blockIdx.x, __uint_as_float(t));
    }
}

// fp8 copy of every shard: the tensor's amax is the maximum over the ranks'
// values (amax_ranks[r * n_shards + index]; NaN propagates), its scale
// 448 / max(amax, 1e-12) in fp32.  The workgroup holding a shard's first
// tile also stores the scale (both parts of a split shard store the same
// value).  GENERAL: some shard's fp8 copy is not vector-aligned.
template <bool GENERAL, int POL>
__global__ __launch_bounds__(kBlock) void mt_cast_fp8_kernel(const TensorDesc* __restrict__ tensors,
                                                             const ChunkDesc* __restrict__ chunks,
                                                             const float* amax_ranks, int32_t n_ranks,
                                                             int64_t n_shards, float* scale_out) {
    for_my_tile<RS_CAST_TILES>(tensors, chunks, [&](const TensorDesc& T, int64_t b, int64_t e) {
        uint32_t bits = 0;
        for (int32_t r = 0; r < n_ranks; ++r)
            bits = std::max(bits, __float_as_uint(ld(amax_ranks + r * n_shards + T.index)) & 0x7fffffffu);
        const float amax = __uint_as_float(bits);
        const float den = (amax > 1e-12f || amax != amax) ? amax : 1e-12f;
        const float scale = 448.0f / den;
        if (b == 0 && scale_out && threadIdx.x == 0) st(scale_out + T.index, scale);
        if (GENERAL && (T.gen & kGenStore)) fp8_range<RS_CAST_TILES, true, POL>(T, b, e, scale);
        else fp8_range<RS_CAST_TILES, false, POL>(T, b, e, scale);
    });
}

constexpr int kSumBlocks = 1024;        // workgroups of the first summation stage

// Workgroup b sums partials[b*per, min(n, (b+1)*per)) into out[b]: lane t
// adds the elements t, t+64, ... of the range (coalesced, several loads in
// flight), then the wave sum.  The order is fixed, so the sum is too.
__global__ __launch_bounds__(kBlock) void sum_partials_kernel(const double* partials, int64_t n,
                                                              int64_t per, double* out) {
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
    const int64_t hi = std::min(n, lo + per);
    double acc = 0.0;
    int64_t i = lo + threadIdx.x;
    for (; i + 3 * kBlock < hi; i += 4 * kBlock) {
        const double a = ld(partials + i), b = ld(partials + i + kBlock);
        const double c = ld(partials + i + 2 * kBlock), d = ld(partials + i + 3 * kBlock);
        acc += a;
        acc += b;
        acc += c;
        acc += d;
    }
    for (; i < hi; i += kBlock) acc += ld(partials + i);
    const double total = wave_sum(acc);
    if (threadIdx.x == 0) st(out + blockIdx.x, total);
}

// Clip coefficient from the ranks' squared norms (their all-reduce sum, taken
// here in index order): norm = sqrt(sum), coef = min(1, max_norm/(norm+1e-6)),
// NaN kept.  One thread.
__global__ void clip_coef_kernel(float* coef_out, double* norm_out, const double* sq, int32_t n,
                                 double max_norm) {
    if (threadIdx.x != 0) return;
    double total = 0.0;
    for (int32_t i = 0; i < n; ++i) total += ld(sq + i);
    const double norm = sqrt(total);
    double coef = max_norm / (norm + 1e-6);
    if (coef > 1.0) coef = 1.0;
    st(coef_out, static_cast<float>(coef));
    if (norm_out) st(norm_out, norm);
}

// A step whose count lives in device memory: advance *step_dev by one and
// derive that step's count- and learning-rate-dependent scalars into *out
// (when out is not null), the learning rate from *lr_dev when that is not
// null, the other scalars coming from the host in `c`.  One lane does it all,
// with vector memory accesses.
__global__ __launch_bounds__(kBlock) void step_count_kernel(int64_t* step_dev, const double* lr_dev,
                                                            StepConsts c, double lr, double wd,
                                                            double beta1, double beta2, StepConsts* out) {
    if (threadIdx.x != 0) return;
    const int64_t t = ld(step_dev) + 1;
    st(step_dev, t);
    if (!out) return;
    if (lr_dev) lr = ld(lr_dev);
    count_scalars(c, lr, wd, beta1, beta2, t);
    static_assert(sizeof(StepConsts) % 4 == 0, "the scalars are stored as 32-bit words");
    uint32_t w[sizeof(StepConsts) / 4];
    __builtin_memcpy(w, &c, sizeof c);
#pragma unroll
    for (size_t i = 0; i < sizeof(StepConsts) / 4; ++i) st(reinterpret_cast<uint32_t*>(out) + i, w[i]);
}

// Single-shard kernels: workgroup b covers elements [b*kTile, (b+1)*kTile).
// GEN: the slices (the gradient, for AdamW alone) or the bf16 copy start off
// a vector boundary, the fp32 buffers on it.
template <int NS, bool BF16, bool GEN, int POL>
__global__ __launch_bounds__(kBlock) void fused_single_kernel(TensorDesc T, StepConsts c) {
    const int64_t begin = static_cast<int64_t>(blockIdx.x) * kTile;
    fused_range<NS, BF16, false, false, false, GEN, false, POL>(
        T, begin, std::min<int64_t>(begin + kTile, T.shard_numel), c);
}

template <int NS, bool BF16, bool GEN, int POL>
__global__ __launch_bounds__(kBlock) void reduce_single_kernel(TensorDesc T, StepConsts c) {
    const int64_t begin = static_cast<int64_t>(blockIdx.x) * kTile;
    reduce_range<NS, BF16, GEN, POL>(T, begin, std::min<int64_t>(begin + kTile, T.shard_numel), c);
}

template <bool GEN, int POL>
__global__ __launch_bounds__(kBlock) void cast_single_kernel(TensorDesc T) {
    const int64_t begin = static_cast<int64_t>(blockIdx.x) * kTile;
    cast_range<GEN, POL>(T, begin, std::min<int64_t>(begin + kTile, T.shard_numel));
}

// Reduce one shard into grad_out and write each workgroup's sum of squares to
// its partials slot.  The grid is whole chunk entries (a multiple of 8), as a
// plan holding this one shard launches it: workgroup b covers elements
// [b*kTile, (b+1)*kTile), the same tile as the plan's tile b % 8 of entry
// b / 8, and the workgroups past the shard's end store a zero partial.
template <int NS, bool BF16, bool GEN, int POL>
__global__ __launch_bounds__(kBlock) void reduce_sqnorm_single_kernel(TensorDesc T, StepConsts c,
                                                                      double* partials) {
    const int64_t begin = static_cast<int64_t>(blockIdx.x) * kTile;
    const int64_t end = std::max(begin, std::min<int64_t>(begin + kTile, T.shard_numel));
    const double sq = reduce_store_range<NS, BF16, true, false, GEN, POL>(T, begin, end, c, false);
    const double total = wave_sum(sq);
    if (threadIdx.x == 0) st(partials + xcd_slot(blockIdx.x, gridDim.x), total);
}

// ---------------------------------------------------------------- kernel selection

using MtKernel = void (*)(const TensorDesc*, const ChunkDesc*, StepConsts, const StepConsts*);
using ReduceKernel = void (*)(TensorDesc, StepConsts);

template <bool BF16, bool GENERAL, int POL, bool DEVC>
MtKernel pick_mt(int n) {
    switch (n) {
        case 1: return mt_step_kernel<1, BF16, GENERAL, POL, DEVC>;
        case 2: return mt_step_kernel<2, BF16, GENERAL, POL, DEVC>;
        case 4: return mt_step_kernel<4, BF16, GENERAL, POL, DEVC>;
        case 8: return mt_step_kernel<8, BF16, GENERAL, POL, DEVC>;
        default: return mt_step_kernel<0, BF16, GENERAL, POL, DEVC>;
    }
}

// The fused step's store policy as a compile-time constant: the one chosen
// for the plan (write-through or its non-temporal form), or the one forced at
// build time.
template <typename Pick>
auto by_step_policy(int pol, Pick pick) {
    if constexpr (RS_ST_POLICY >= 0) {
        (void)pol;
        return pick(std::integral_constant<int, RS_ST_POLICY>{});
    } else {
        return pol == kStNtWriteThrough ? pick(std::integral_constant<int, kStNtWriteThrough>{})
                                        : pick(std::integral_constant<int, kStWriteThrough>{});
    }
}

MtKernel pick_mt(int dtype, int n, bool general, int pol, bool devc) {
    return by_step_policy(pol, [&](auto P) {
        constexpr int kPol = decltype(P)::value;
        if (devc) {
            if (dtype == FSDP_DT_BF16)
                return general ? pick_mt<true, true, kPol, true>(n) : pick_mt<true, false, kPol, true>(n);
            return general ? pick_mt<false, true, kPol, true>(n) : pick_mt<false, false, kPol, true>(n);
        }
        if (dtype == FSDP_DT_BF16)
            return general ? pick_mt<true, true, kPol, false>(n) : pick_mt<true, false, kPol, false>(n);
        return general ? pick_mt<false, true, kPol, false>(n) : pick_mt<false, false, kPol, false>(n);
    });
}

using RunKernel = void (*)(TensorDesc, StepConsts, const StepConsts*);

template <bool BF16, int POL, bool DEVC>
RunKernel pick_run(int n) {
    switch (n) {
        case 1: return run_step_kernel<1, BF16, POL, DEVC>;
        case 2: return run_step_kernel<2, BF16, POL, DEVC>;
        case 4: return run_step_kernel<4, BF16, POL, DEVC>;
        case 8: return run_step_kernel<8, BF16, POL, DEVC>;
        default: return run_step_kernel<0, BF16, POL, DEVC>;
    }
}

RunKernel pick_run(int dtype, int n, int pol, bool devc) {
    return by_step_policy(pol, [&](auto P) {
        constexpr int kPol = decltype(P)::value;
        if (devc) return dtype == FSDP_DT_BF16 ? pick_run<true, kPol, true>(n) : pick_run<false, kPol, true>(n);
        return dtype == FSDP_DT_BF16 ? pick_run<true, kPol, false>(n) : pick_run<false, kPol, false>(n);
    });
}

// The policy a pass's stores run under: the one chosen for the launch
// (write-through or its non-temporal form), or the one forced at build time.
template <typename Pick>
auto by_policy(int pol, Pick pick) {
    if constexpr (RS_ST_POLICY_PASSES >= 0) {
        (void)pol;
        return pick(std::integral_constant<int, RS_ST_POLICY_PASSES>{});
    } else {
        return pol == kStNtWriteThrough ? pick(std::integral_constant<int, kStNtWriteThrough>{})
                                        : pick(std::integral_constant<int, kStWriteThrough>{});
    }
}

using ReduceStoreKernel = void (*)(const TensorDesc*, const ChunkDesc*, StepConsts, int32_t, double*);

template <bool BF16, bool SQ, bool GENERAL, int POL>
ReduceStoreKernel pick_reduce_store(int n) {
    switch (n) {
        case 1: return mt_reduce_store_kernel<1, BF16, SQ, GENERAL, POL>;
        case 2: return mt_reduce_store_kernel<2, BF16, SQ, GENERAL, POL>;
        case 4: return mt_reduce_store_kernel<4, BF16, SQ, GENERAL, POL>;
        case 8: return mt_reduce_store_kernel<8, BF16, SQ, GENERAL, POL>;
        default: return mt_reduce_store_kernel<0, BF16, SQ, GENERAL, POL>;
    }
}

template <bool GENERAL, int POL>
ReduceStoreKernel pick_reduce_store(int dtype, int n, bool sq) {
    if (dtype == FSDP_DT_BF16)
        return sq ? pick_reduce_store<true, true, GENERAL, POL>(n) : pick_reduce_store<true, false, GENERAL, POL>(n);
    return sq ? pick_reduce_store<false, true, GENERAL, POL>(n) : pick_reduce_store<false, false, GENERAL, POL>(n);
}

ReduceStoreKernel pick_reduce_store(int dtype, int n, bool sq, bool general, int pol) {
    return by_policy(pol, [&](auto P) {
        constexpr int kPol = decltype(P)::value;
        return general ? pick_reduce_store<true, kPol>(dtype, n, sq) : pick_reduce_store<false, kPol>(dtype, n, sq);
    });
}

using AmaxKernel = void (*)(const TensorDesc*, const ChunkDesc*, StepConsts, uint32_t*, const StepConsts*);

template <bool BF16, bool GENERAL, int POL, bool DEVC>
AmaxKernel pick_amax(int n) {
    switch (n) {
        case 1: return mt_step_amax_kernel<1, BF16, GENERAL, POL, DEVC>;
        case 2: return mt_step_amax_kernel<2, BF16, GENERAL, POL, DEVC>;
        case 4: return mt_step_amax_kernel<4, BF16, GENERAL, POL, DEVC>;
        case 8: return mt_step_amax_kernel<8, BF16, GENERAL, POL, DEVC>;
        default: return mt_step_amax_kernel<0, BF16, GENERAL, POL, DEVC>;
    }
}

template <int POL, bool DEVC>
AmaxKernel pick_amax(int dtype, int n, bool general) {
    if (dtype == FSDP_DT_BF16)
        return general ? pick_amax<true, true, POL, DEVC>(n) : pick_amax<true, false, POL, DEVC>(n);
    return general ? pick_amax<false, true, POL, DEVC>(n) : pick_amax<false, false, POL, DEVC>(n);
}

AmaxKernel pick_amax(int dtype, int n, bool general, int pol, bool devc) {
    return by_policy(pol, [&](auto P) {
        constexpr int kPol = decltype(P)::value;
        return devc ? pick_amax<kPol, true>(dtype, n, general) : pick_amax<kPol, false>(dtype, n, general);
    });
}

using Fp8StepKernel = void (*)(const TensorDesc*, const ChunkDesc*, StepConsts, const float*,
                               uint32_t*, const StepConsts*);

template <bool BF16, bool GENERAL, int POL, bool DEVC>
Fp8StepKernel pick_fp8_step(int n) {
    switch (n) {
        case 1: return mt_step_fp8_kernel<1, BF16, GENERAL, POL, DEVC>;
        case 2: return mt_step_fp8_kernel<2, BF16, GENERAL, POL, DEVC>;
        case 4: return mt_step_fp8_kernel<4, BF16, GENERAL, POL, DEVC>;
        case 8: return mt_step_fp8_kernel<8, BF16, GENERAL, POL, DEVC>;
        default: return mt_step_fp8_kernel<0, BF16, GENERAL, POL, DEVC>;
    }
}

template <int POL, bool DEVC>
Fp8StepKernel pick_fp8_step(int dtype, int n, bool general) {
    if (dtype == FSDP_DT_BF16)
        return general ? pick_fp8_step<true, true, POL, DEVC>(n) : pick_fp8_step<true, false, POL, DEVC>(n);
    return general ? pick_fp8_step<false, true, POL, DEVC>(n) : pick_fp8_step<false, false, POL, DEVC>(n);
}

Fp8StepKernel pick_fp8_step(int dtype, int n, bool general, int pol, bool devc) {
    return by_policy(pol, [&](auto P) {
        constexpr int kPol = decltype(P)::value;
        return devc ? pick_fp8_step<kPol, true>(dtype, n, general) : pick_fp8_step<kPol, false>(dtype, n, general);
    });
}

using AccumulateKernel = void (*)(float*, const void*, int64_t, int32_t, int32_t);

AccumulateKernel pick_accumulate(bool bf16, bool gen, int pol) {
    return by_policy(pol, [&](auto P) -> AccumulateKernel {
        constexpr int kPol = decltype(P)::value;
        if (bf16) return gen ? accumulate_kernel<true, true, kPol> : accumulate_kernel<true, false, kPol>;
        return gen ? accumulate_kernel<false, true, kPol> : accumulate_kernel<false, false, kPol>;
    });
}

using ScaledStepKernel = void (*)(const TensorDesc*, const ChunkDesc*, StepConsts, const float*,
                                  const StepConsts*);

ScaledStepKernel pick_scaled_step(bool general, int pol, bool devc) {
    return by_policy(pol, [&](auto P) -> ScaledStepKernel {
        constexpr int kPol = decltype(P)::value;
        if (devc) return general ? mt_scaled_step_kernel<true, kPol, true> : mt_scaled_step_kernel<false, kPol, true>;
        return general ? mt_scaled_step_kernel<true, kPol, false> : mt_scaled_step_kernel<false, kPol, false>;
    });
}

template <bool BF16, bool GEN, int POL>
ReduceKernel pick_reduce(int n) {
    switch (n) {
        case 1: return reduce_single_kernel<1, BF16, GEN, POL>;
        case 2: return reduce_single_kernel<2, BF16, GEN, POL>;
        case 4: return reduce_single_kernel<4, BF16, GEN, POL>;
        case 8: return reduce_single_kernel<8, BF16, GEN, POL>;
        default: return reduce_single_kernel<0, BF16, GEN, POL>;
    }
}

ReduceKernel pick_reduce(int dtype, int n, bool gen, int pol) {
    return by_policy(pol, [&](auto P) {
        constexpr int kPol = decltype(P)::value;
        if (dtype == FSDP_DT_BF16) return gen ? pick_reduce<true, true, kPol>(n) : pick_reduce<true, false, kPol>(n);
        return gen ? pick_reduce<false, true, kPol>(n) : pick_reduce<false, false, kPol>(n);
    });
}

using SqnormSingleKernel = void (*)(TensorDesc, StepConsts, double*);

template <bool BF16, bool GEN, int POL>
SqnormSingleKernel pick_sqnorm_single(int n) {
    switch (n) {
        case 1: return reduce_sqnorm_single_kernel<1, BF16, GEN, POL>;
        case 2: return reduce_sqnorm_single_kernel<2, BF16, GEN, POL>;
        case 4: return reduce_sqnorm_single_kernel<4, BF16, GEN, POL>;
        case 8: return reduce_sqnorm_single_kernel<8, BF16, GEN, POL>;
        default: return reduce_sqnorm_single_kernel<0, BF16, GEN, POL>;
    }
}

SqnormSingleKernel pick_sqnorm_single(int dtype, int n, bool gen, int pol) {
    return by_policy(pol, [&](auto P) {
        constexpr int kPol = decltype(P)::value;
        if (dtype == FSDP_DT_BF16)
            return gen ? pick_sqnorm_single<true, true, kPol>(n) : pick_sqnorm_single<true, false, kPol>(n);
        return gen ? pick_sqnorm_single<false, true, kPol>(n) : pick_sqnorm_single<false, false, kPol>(n);
    });
}

// ---------------------------------------------------------------- host helpers

int64_t dtype_bytes(int32_t dt) { return dt == FSDP_DT_F32 ? 4 : 2; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int32_t check_hparams(const fsdp_adamw_hparams* hp) {
    if (!hp) return fail(FSDP_E_ARG, "null hyperparameters");
    const double xs[5] = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay};
    for (double x : xs)
        if (!std::isfinite(x)) return fail(FSDP_E_ARG, "hyperparameters must be finite");
    if (hp->lr < 0) return fail(FSDP_E_ARG, "lr %g < 0", hp->lr);
    if (hp->beta1 < 0 || hp->beta1 >= 1) return fail(FSDP_E_ARG, "beta1 %g outside [0, 1)", hp->beta1);
    if (hp->beta2 < 0 || hp->beta2 >= 1) return fail(FSDP_E_ARG, "beta2 %g outside [0, 1)", hp->beta2);
    if (hp->eps < 0) return fail(FSDP_E_ARG, "eps %g < 0", hp->eps);
    if (hp->weight_decay < 0) return fail(FSDP_E_ARG, "weight_decay %g < 0", hp->weight_decay);
    if (hp->step < 1) return fail(FSDP_E_ARG, "step %lld < 1", static_cast<long long>(hp->step));
    return FSDP_OK;
}

StepConsts make_consts(const fsdp_adamw_hparams* hp, int32_t n) {
    StepConsts c{};
    if (hp) {
        c.beta1 = static_cast<float>(hp->beta1);
        c.omb1 = static_cast<float>(1.0 - hp->beta1);
        c.beta2 = static_cast<float>(hp->beta2);
        c.omb2 = static_cast<float>(1.0 - hp->beta2);
        count_scalars(c, hp->lr, hp->weight_decay, hp->beta1, hp->beta2, hp->step);
        c.eps = static_cast<float>(hp->eps);
    }
    c.n = n;
    c.n_pow2 = (n & (n - 1)) == 0;
    c.inv_n = static_cast<float>(1.0 / n);
    c.n_f = static_cast<float>(n);
    return c;
}

// Bytes of one 4-element group of each buffer class: the vector path needs
// every buffer aligned to it (and slice q's start too, through the stride).
constexpr uintptr_t kF32Vec = 4 * kGroup, kBf16Vec = 2 * kGroup, kFp8Vec = kGroup;

bool slices_vec_ok(const void* slices, int32_t slice_dtype, int64_t stride, int32_t n_slices) {
    const uintptr_t a = slice_dtype == FSDP_DT_BF16 ? kBf16Vec : kF32Vec;
    if (slices && !aligned(slices, a)) return false;
    return n_slices == 1 || (stride * dtype_bytes(slice_dtype)) % static_cast<int64_t>(a) == 0;
}

int64_t tiles_for(int64_t S) { return (S + kTile - 1) / kTile; }

// Slices whose loads a tile has in flight together: all N when N is compiled
// in (1, 2, 4, 8), one batch of the runtime loop otherwise.
int64_t inflight_slices(int32_t n, int32_t slice_dtype) {
    const bool compiled = n == 1 || n == 2 || n == 4 || n == 8;
    const int64_t batch = std::max<int64_t>(1, RS_RT_BATCH_BYTES / (kGroup * dtype_bytes(slice_dtype)));
    return compiled ? n : std::min<int64_t>(n, batch);
}

// One launch covers at most 2^32 - 1 work-items in a grid dimension.
constexpr int64_t kMaxBlocks = 0xffffffffLL / kBlock;

int32_t check_grid(int64_t blocks, const char* who) {
    if (blocks > kMaxBlocks)
        return fail(FSDP_E_CAPACITY, "%s: %lld workgroups exceed one launch", who,
                    static_cast<long long>(blocks));
    return FSDP_OK;
}

int32_t launch_status(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(FSDP_E_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return FSDP_OK;
}

// Checks shared by the slice-reading calls.
int32_t check_slices(const void* slices, int32_t slice_dtype, int64_t slice_stride,
                     int32_t n_slices, int64_t S, int64_t valid, const char* who) {
    if (slice_dtype != FSDP_DT_F32 && slice_dtype != FSDP_DT_BF16)
        return fail(FSDP_E_DTYPE, "%s: unknown slice dtype %d", who, slice_dtype);
    if (n_slices < 1 || n_slices > kMaxSlices)
        return fail(FSDP_E_ARG, "%s: n_slices %d outside [1, %d]", who, n_slices, kMaxSlices);
    if (n_slices > 1 && slice_stride < S)
        return fail(FSDP_E_ARG, "%s: slice_stride %lld < shard_numel %lld", who,
                    static_cast<long long>(slice_stride), static_cast<long long>(S));
    if (valid > 0 && !slices) return fail(FSDP_E_ARG, "%s: null grad_slices", who);
    if (slices && !aligned(slices, dtype_bytes(slice_dtype)))
        return fail(FSDP_E_ALIGN, "%s: grad_slices not aligned to its element size", who);
    int64_t span;
    if (n_slices > 1 && (!fsdp::mul_i64(n_slices - 1, slice_stride, &span) ||
                         !fsdp::add_i64(span, S, &span) ||
                         !fsdp::mul_i64(span, dtype_bytes(slice_dtype), &span)))
        return fail(FSDP_E_ARG, "%s: slice extent overflows int64", who);
    return FSDP_OK;
}

// Checks of a shard's table of slice pointers (the slices of the shard in
// separate buffers): every entry set and aligned to the element size when the
// shard has data to read.
int32_t check_slice_table(const void* const* ptrs, int32_t slice_dtype, int32_t n_slices,
                          int64_t valid, const char* who) {
    if (valid == 0) return FSDP_OK;
    for (int32_t q = 0; q < n_slices; ++q) {
        if (!ptrs[q]) return fail(FSDP_E_ARG, "%s: null grad_slice_ptrs[%d]", who, q);
        if (!aligned(ptrs[q], dtype_bytes(slice_dtype)))
            return fail(FSDP_E_ALIGN, "%s: grad_slice_ptrs[%d] not aligned to its element size",
                        who, q);
    }
    int64_t bytes;
    if (!fsdp::mul_i64(valid, dtype_bytes(slice_dtype), &bytes))
        return fail(FSDP_E_ARG, "%s: slice extent overflows int64", who);
    return FSDP_OK;
}

// Whether every slice of a table is aligned for the vector path.
bool slice_table_vec_ok(const void* const* ptrs, int32_t slice_dtype, int32_t n_slices) {
    const uintptr_t a = slice_dtype == FSDP_DT_BF16 ? kBf16Vec : kF32Vec;
    for (int32_t q = 0; q < n_slices; ++q)
        if (!aligned(ptrs[q], a)) return false;
    return true;
}

// The vector path needs the fp32 buffers it reads and writes back (param,
// moments, stored gradient) 16-byte aligned; the slices and the
// low-precision copies may start at any element (they are read as two
// aligned vectors and a byte shift, or stored in narrower pieces).
bool state_vec_ok(const TensorDesc& d) {
    return aligned(d.param, kF32Vec) && aligned(d.m, kF32Vec) && aligned(d.v, kF32Vec) &&
           (!d.grad_out || aligned(d.grad_out, kF32Vec));
}

// The any-alignment forms a shard on the vector path needs: kGenLoad when a
// slice is not vector-aligned, kGenStore when a low-precision copy is not
// (or when its slices are not: that form stores at any alignment too).
int64_t plan_gen(const TensorDesc& d, int32_t slice_dtype, int32_t n_slices,
                 const void* const* table) {
    const bool slices_ok = d.valid == 0 ||
                           (table ? slice_table_vec_ok(table, slice_dtype, n_slices)
                                  : slices_vec_ok(d.slices, slice_dtype, d.slice_stride, n_slices));
    const bool copies_ok = (!d.out_bf16 || aligned(d.out_bf16, kBf16Vec)) &&
                           (!d.out_fp8 || aligned(d.out_fp8, kFp8Vec));
    return (slices_ok ? 0 : kGenLoad | kGenStore) | (copies_ok ? 0 : kGenStore);
}

// How many elements past a vector boundary the fp32 buffers of shard d
// start (0-3), or -1 when they disagree (then no split aligns them all).
int element_phase(const TensorDesc& d) {
    int phase = -1;
    bool agree = true;
    const float* const fp32_bufs[4] = {d.param, d.m, d.v, d.grad_out};
    for (const float* p : fp32_bufs) {
        if (!p) continue;
        const int ph = static_cast<int>((reinterpret_cast<uintptr_t>(p) / 4) & 3);
        if (phase < 0) phase = ph;
        else if (ph != phase) agree = false;
    }
    return agree ? phase : -1;
}

int32_t check_sizes(int64_t S, int64_t valid, const char* who) {
    if (S < 0 || valid < 0 || valid > S)
        return fail(FSDP_E_ARG, "%s: need 0 <= valid (%lld) <= shard_numel (%lld)", who,
                    static_cast<long long>(valid), static_cast<long long>(S));
    if (S > (int64_t(1) << 60)) return fail(FSDP_E_ARG, "%s: shard_numel too large", who);
    return FSDP_OK;
}

fsdp::Range range_of(const void* p, int64_t elems, int64_t esize, bool written, int32_t owner,
                     const char* what) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return fsdp::Range{lo, p ? lo + static_cast<uintptr_t>(elems * esize) : lo, written, owner, what};
}

void add_slice_ranges(std::vector<fsdp::Range>& rs, const void* slices, int32_t dt,
                      int64_t stride, int32_t n, int64_t valid, int32_t owner) {
    if (!slices || valid == 0) return;
    const int64_t es = dtype_bytes(dt);
    for (int32_t q = 0; q < n; ++q)
        rs.push_back(range_of(static_cast<const char*>(slices) + q * stride * es, valid, es, false,
                              owner, "grad_slices"));
}

}  // namespace

// ====================================================================== C ABI

struct fsdp_mt_plan {
    int device = -1;
    int32_t n_slices = 1;
    int32_t slice_dtype = FSDP_DT_F32;
    int64_t n_tensors = 0, n_chunks = 0, n_blocks = 0, total_numel = 0, total_valid = 0;
    int64_t chunk_numel = 0;
    bool all_grad_out = false;       // every non-empty shard stores its reduced gradient
    bool any_fp8 = false;            // some shard has an fp8 copy
    bool all_fp8 = false;            // every non-empty shard has one
    bool any_bf16 = false;           // some shard has a bf16 copy
    bool any_grad_out = false;       // some shard stores its reduced gradient
    bool any_general = false;        // some shard reads its slices through a table of pointers,
                                     // or has a slice or copy that is not vector-aligned
    uint32_t* d_tile_amax = nullptr;      // fp8: largest |p'| per workgroup
    ShardTiles* d_shard_tiles = nullptr;  // fp8: each input shard's run of workgroups
    TensorDesc* d_tensors = nullptr;
    ChunkDesc* d_chunks = nullptr;
    const void** d_slice_ptrs = nullptr;  // the shards' tables of slice pointers, if any
    double* d_partials = nullptr;    // clipped steps: one sum of squares per workgroup,
                                     // then kSumBlocks second-stage sums
    StepConsts* d_consts = nullptr;  // steps whose count is in device memory: that step's scalars
    fsdp::Footprint footprint;       // the shards' buffers, for checking the calls' other buffers
    int store_pol = kStPlain;        // how the fused step stores the updated state
    bool has_run = false;            // the shards lie back to back in every buffer:
    TensorDesc run{};                // then this one range covers them all
    bool pooled = false;             // the device tables come from the stream-ordered allocator
    hipEvent_t done = nullptr;       // completes with the plan's last launch outside a capture
};

namespace {

// Whether work queued on `s` now would be captured into a HIP graph (or the
// query fails, as it does for the null stream while another stream captures
// globally: then it is treated as capturing).
bool capturing(hipStream_t s) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    return cs != hipStreamCaptureStatusNone;
}

// Launch of a plan call.  The call's last launch carries the plan's
// completion event, bound to the kernel's own completion (no further queue
// entry), which fsdp_mt_plan_destroy waits on.  Launches that a HIP graph
// captures carry none: the graph's replays are the caller's to order.
template <typename K, typename... Args>
void plan_launch(const fsdp_mt_plan* plan, bool last, K k, dim3 grid, dim3 block, size_t lds,
                 hipStream_t stream, Args... args) {
    if (last && plan->done && !capturing(stream))
        hipExtLaunchKernelGGL(k, grid, block, static_cast<uint32_t>(lds), stream, nullptr, plan->done,
                              0u, args...);
    else
        hipLaunchKernelGGL(k, grid, block, lds, stream, args...);
}

// A plan's device tables come from the stream-ordered allocator where the
// device has one, so that destroying the plan frees them without the
// device-wide synchronisation that hipFree performs.
hipError_t plan_alloc(const fsdp_mt_plan* plan, void** p, size_t bytes, hipStream_t stream) {
    return plan->pooled ? hipMallocAsync(p, bytes, stream) : hipMalloc(p, bytes);
}

// One non-blocking stream per device, made on the first plan destroyed there
// and kept until the process ends: the stream-ordered frees go on it, after
// the host has waited for the plan's last launch.
std::mutex g_free_mu;
hipStream_t g_free_stream[kMaxDevices] = {};

hipError_t free_stream(int dev, hipStream_t* out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_free_mu);
    if (!g_free_stream[dev]) {
        const hipError_t e = hipStreamCreateWithFlags(&g_free_stream[dev], hipStreamNonBlocking);
        if (e != hipSuccess) return e;
    }
    *out = g_free_stream[dev];
    return hipSuccess;
}

// The plan exists and belongs to the current device.
int32_t check_plan_device(const fsdp_mt_plan* plan, const char* who) {
    if (!plan) return fail(FSDP_E_ARG, "%s: null plan", who);
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FSDP_E_HIP, "%s: %s", who, hipGetErrorString(e));
    if (dev != plan->device)
        return fail(FSDP_E_STATE, "%s: plan made on device %d used on device %d", who, plan->device,
                    dev);
    return FSDP_OK;
}

// A further device buffer of a plan call (`bytes` long at p) against the
// plan's own buffers: an input may overlap only the read-only gradient
// slices, an output none of them.
int32_t check_extra(const fsdp_mt_plan* plan, const void* p, int64_t bytes, bool output,
                    const char* who, const char* what) {
    if (!p || bytes <= 0) return FSDP_OK;
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    const uintptr_t hi = lo + static_cast<uintptr_t>(bytes);
    if (output ? plan->footprint.hits_any(lo, hi) : plan->footprint.hits_written(lo, hi))
        return fail(FSDP_E_ALIAS, "%s: %s overlaps %s buffer of the plan's shards", who, what,
                    output ? "a" : "a written");
    return FSDP_OK;
}

// Bytes per element of the plan's slices that a tile has in flight at once
// (all N for the slice counts compiled in, one batch for the others), and
// of its fused step.
int64_t slice_bytes(const fsdp_mt_plan* plan) {
    return dtype_bytes(plan->slice_dtype) * inflight_slices(plan->n_slices, plan->slice_dtype);
}
int64_t step_bytes(const fsdp_mt_plan* plan) {
    return slice_bytes(plan) + 24 + 2 * plan->any_bf16 + 4 * plan->any_grad_out;
}

// Whether the shards descs[0..) lie back to back in every buffer, so that
// one range covers them: each starts where the one before it ends in the
// state, the stored gradient, the copies and the slices (one stride for all),
// every shard but the last has no padding, and all take the plain vector
// path.  The range is written to *run.
//
// The range deals its tile j to workgroup j, hence to XCD j % 8; the chunk
// table restarts the deal at every shard, giving a shard's tile j to XCD
// j % 8.  The two agree on a shard that starts on a chunk-entry boundary of
// the range.  The deal alone moves a step by several per cent either way
// (it decides which HBM channels each XCD's L2 streams from), so the range
// is taken only where the shards off such a boundary hold at most
// 1/kRedealShare of the elements: a Llama block's last norm weight (2 of
// 98,820 tiles), but not a whole model's shard, whose 512-element norm
// weights shift every other layer's deal by four XCDs.
constexpr int64_t kRedealShare = 256;

bool merge_run(const std::vector<TensorDesc>& descs, int32_t slice_dtype, int32_t n_slices,
               TensorDesc* run) {
    if (descs.empty()) return false;
    const int64_t es = dtype_bytes(slice_dtype);
    int64_t redealt = 0;  // elements of shards that start off a chunk-entry boundary
    TensorDesc r = descs[0];
    for (size_t i = 0; i < descs.size(); ++i) {
        const TensorDesc& d = descs[i];
        if (d.slice_ptrs || !d.vec_ok || d.gen) return false;
        if (i == 0) continue;
        const TensorDesc& a = descs[i - 1];
        const int64_t n = a.shard_numel;
        if (a.valid != n) return false;
        if (d.param != a.param + n || d.m != a.m + n || d.v != a.v + n) return false;
        if ((a.grad_out == nullptr) != (d.grad_out == nullptr) || (d.grad_out && d.grad_out != a.grad_out + n))
            return false;
        if ((a.out_bf16 == nullptr) != (d.out_bf16 == nullptr) || (d.out_bf16 && d.out_bf16 != a.out_bf16 + n))
            return false;
        if ((a.out_fp8 == nullptr) != (d.out_fp8 == nullptr) || (d.out_fp8 && d.out_fp8 != a.out_fp8 + n))
            return false;
        if (d.valid > 0) {
            if (d.slices != static_cast<const char*>(a.slices) + n * es) return false;
            if (n_slices > 1 && d.slice_stride != a.slice_stride) return false;
        }
        if (r.shard_numel % kChunk != 0) redealt += d.shard_numel;
        r.shard_numel += d.shard_numel;
    }
    if (redealt > r.shard_numel / kRedealShare) return false;
    r.valid = r.shard_numel - (descs.back().shard_numel - descs.back().valid);
    r.index = 0;
    *run = r;
    return true;
}

// The store policy of a streaming pass that reads `reads` and writes
// `writes` bytes per element: write-through where it reads more than half
// again as many bytes as it writes; non-temporal write-through where writes
// come closer to half the traffic.  Measured on the 7B shard's passes
// (interleaved builds, 3 passes): the fused step at 28 : 14 and the fp8 steps
// at 28 : 12-13 gain most from write-through (5.31 -> 5.21 ms for the
// delayed-scaling step), the synchronised accumulation at 20 : 4 too (2.99 ->
// 2.94 ms, 3.05 under the non-temporal form); the 70B shard's step at 16 : 14
// and the no_sync accumulation at 6 : 4, the one tie, from the non-temporal
// form (1.291 -> 1.244 ms, 1.265 under write-through alone).
int write_policy(int64_t reads, int64_t writes) {
    return 2 * reads > 3 * writes ? kStWriteThrough : kStNtWriteThrough;
}

// Bytes per element a plan's passes read in slices (all N) and write besides
// the state.
int64_t plan_slice_read(const fsdp_mt_plan* plan) { return dtype_bytes(plan->slice_dtype) * plan->n_slices; }
int64_t plan_copy_write(const fsdp_mt_plan* plan) { return 2 * plan->any_bf16 + 4 * plan->any_grad_out; }

// The fused step's store policy for a plan: N slices at 2 or 4 bytes and 12
// bytes of state read against 12 of state, 2 of bf16 and 4 of stored
// gradient written.
int store_policy(const fsdp_mt_plan* plan) {
    if (RS_ST_POLICY >= 0) return RS_ST_POLICY;
    return write_policy(plan_slice_read(plan) + 12, 12 + plan_copy_write(plan));
}

}  // namespace

static int32_t reduce_grad_shard_impl(float* grad_shard_out, const void* grad_slices,
                                      int32_t slice_dtype, int64_t slice_stride,
                                      int32_t n_slices, int64_t shard_numel, int64_t valid,
                                      hipStream_t stream) {
    const char* who = "fsdp_reduce_grad_shard";
    int32_t st;
    if ((st = check_sizes(shard_numel, valid, who)) != FSDP_OK) return st;
    if ((st = check_slices(grad_slices, slice_dtype, slice_stride, n_slices, shard_numel, valid,
                           who)) != FSDP_OK)
        return st;
    if (shard_numel == 0) return FSDP_OK;
    if (!grad_shard_out) return fail(FSDP_E_ARG, "%s: null grad_shard_out", who);
    if (!aligned(grad_shard_out, 4)) return fail(FSDP_E_ALIGN, "%s: grad_shard_out misaligned", who);
    std::vector<fsdp::Range> rs{range_of(grad_shard_out, shard_numel, 4, true, 0, "grad_shard_out")};
    add_slice_ranges(rs, grad_slices, slice_dtype, slice_stride, n_slices, valid, 0);
    if ((st = fsdp::check_aliases(rs)) != FSDP_OK) return st;

    TensorDesc T{};
    T.slices = grad_slices;
    T.grad_out = grad_shard_out;
    T.slice_stride = slice_stride;
    T.shard_numel = shard_numel;
    T.valid = valid;
    // the vector path needs the output aligned; slices off a vector
    // boundary take the shifted loads
    T.vec_ok = aligned(grad_shard_out, kF32Vec);
    const bool gen = T.vec_ok && !slices_vec_ok(grad_slices, slice_dtype, slice_stride, n_slices);
    const StepConsts c = make_consts(nullptr, n_slices);
    if ((st = check_grid(tiles_for(shard_numel), who)) != FSDP_OK) return st;
    const ReduceKernel k =
        pick_reduce(slice_dtype, n_slices, gen, write_policy(dtype_bytes(slice_dtype) * n_slices, 4));
    hipLaunchKernelGGL(k, dim3(static_cast<uint32_t>(tiles_for(shard_numel))), dim3(kBlock),
                       lds_reserve(dtype_bytes(slice_dtype) * inflight_slices(n_slices, slice_dtype) + 4),
                       stream, T, c);
    return launch_status(who);
}

static int32_t adamw_shard_step_impl(float* param_fp32, float* exp_avg, float* exp_avg_sq,
                                     const float* grad_shard, int64_t shard_numel,
                                     int64_t valid, const fsdp_adamw_hparams* hp,
                                     hipStream_t stream) {
    const char* who = "fsdp_adamw_shard_step";
    int32_t st;
    if ((st = check_sizes(shard_numel, valid, who)) != FSDP_OK) return st;
    if ((st = check_hparams(hp)) != FSDP_OK) return st;
    if (shard_numel == 0) return FSDP_OK;
    if (!param_fp32 || !exp_avg || !exp_avg_sq)
        return fail(FSDP_E_ARG, "%s: null param / exp_avg / exp_avg_sq", who);
    if (valid > 0 && !grad_shard) return fail(FSDP_E_ARG, "%s: null grad_shard", who);
    if (!aligned(param_fp32, 4) || !aligned(exp_avg, 4) || !aligned(exp_avg_sq, 4) ||
        !aligned(grad_shard, 4))
        return fail(FSDP_E_ALIGN, "%s: fp32 buffer not 4-byte aligned", who);
    std::vector<fsdp::Range> rs{range_of(param_fp32, shard_numel, 4, true, 0, "param"),
                                range_of(exp_avg, shard_numel, 4, true, 0, "exp_avg"),
                                range_of(exp_avg_sq, shard_numel, 4, true, 0, "exp_avg_sq")};
    add_slice_ranges(rs, grad_shard, FSDP_DT_F32, shard_numel, 1, valid, 0);
    if ((st = fsdp::check_aliases(rs)) != FSDP_OK) return st;

    TensorDesc T{};
    T.param = param_fp32;
    T.m = exp_avg;
    T.v = exp_avg_sq;
    T.slices = grad_shard;
    T.slice_stride = shard_numel;
    T.shard_numel = shard_numel;
    T.valid = valid;
    // the vector path needs the state aligned; a gradient off a vector
    // boundary takes the shifted loads
    T.vec_ok = state_vec_ok(T);
    const bool gen = T.vec_ok && !aligned(grad_shard, kF32Vec);
    const StepConsts c = make_consts(hp, 1);
    if ((st = check_grid(tiles_for(shard_numel), who)) != FSDP_OK) return st;
    // 4 bytes of gradient and 12 of state read, 12 written
    const ReduceKernel k = by_policy(write_policy(16, 12), [&](auto P) -> ReduceKernel {
        constexpr int kPol = decltype(P)::value;
        return gen ? fused_single_kernel<1, false, true, kPol> : fused_single_kernel<1, false, false, kPol>;
    });
    hipLaunchKernelGGL(k, dim3(static_cast<uint32_t>(tiles_for(shard_numel))),
                       dim3(kBlock), lds_reserve(4 + 24), stream, T, c);
    return launch_status(who);
}

static int32_t cast_unshard_bf16_impl(uint16_t* unshard_bf16_out, const float* param_fp32,
                                      int64_t shard_numel, int64_t valid, hipStream_t stream) {
    const char* who = "fsdp_cast_unshard_bf16";
    int32_t st;
    if ((st = check_sizes(shard_numel, valid, who)) != FSDP_OK) return st;
    if (shard_numel == 0) return FSDP_OK;
    if (!unshard_bf16_out) return fail(FSDP_E_ARG, "%s: null unshard_bf16_out", who);
    if (valid > 0 && !param_fp32) return fail(FSDP_E_ARG, "%s: null param_fp32", who);
    if (!aligned(unshard_bf16_out, 2) || !aligned(param_fp32, 4))
        return fail(FSDP_E_ALIGN, "%s: buffer not aligned to its element size", who);
    std::vector<fsdp::Range> rs{range_of(unshard_bf16_out, shard_numel, 2, true, 0, "unshard_bf16_out")};
    if (valid > 0) rs.push_back(range_of(param_fp32, valid, 4, false, 0, "param"));
    if ((st = fsdp::check_aliases(rs)) != FSDP_OK) return st;

    TensorDesc T{};
    T.param = const_cast<float*>(param_fp32);
    T.out_bf16 = unshard_bf16_out;
    T.shard_numel = shard_numel;
    T.valid = valid;
    // the vector path needs the parameter aligned; a copy off a vector
    // boundary is stored in narrower pieces
    T.vec_ok = aligned(param_fp32, kF32Vec);
    const bool gen = T.vec_ok && !aligned(unshard_bf16_out, kBf16Vec);
    if ((st = check_grid(tiles_for(shard_numel), who)) != FSDP_OK) return st;
    // 4 bytes read per 2 written: write-through
    using CastKernel = void (*)(TensorDesc);
    const CastKernel k = by_policy(write_policy(4, 2), [&](auto P) -> CastKernel {
        constexpr int kPol = decltype(P)::value;
        return gen ? cast_single_kernel<true, kPol> : cast_single_kernel<false, kPol>;
    });
    hipLaunchKernelGGL(k, dim3(static_cast<uint32_t>(tiles_for(shard_numel))),
                       dim3(kBlock), lds_reserve(4 + 2), stream, T);
    return launch_status(who);
}

static int32_t mt_plan_create_impl(fsdp_mt_plan** plan_out, const fsdp_mt_tensor* tensors,
                                   int32_t n_tensors, int32_t n_slices, int32_t slice_dtype,
                                   hipStream_t stream) {
    const char* who = "fsdp_mt_plan_create";
    if (!plan_out) return fail(FSDP_E_ARG, "%s: null plan_out", who);
    *plan_out = nullptr;
    if (n_tensors < 0) return fail(FSDP_E_ARG, "%s: n_tensors %d < 0", who, n_tensors);
    if (n_tensors > 0 && !tensors) return fail(FSDP_E_ARG, "%s: null tensors", who);
    if (slice_dtype != FSDP_DT_F32 && slice_dtype != FSDP_DT_BF16)
        return fail(FSDP_E_DTYPE, "%s: unknown slice dtype %d", who, slice_dtype);
    if (n_slices < 1 || n_slices > kMaxSlices)
        return fail(FSDP_E_ARG, "%s: n_slices %d outside [1, %d]", who, n_slices, kMaxSlices);

    std::vector<TensorDesc> descs;
    descs.reserve(static_cast<size_t>(n_tensors));
    bool all_grad_out = true;
    bool any_fp8 = false, all_fp8 = true, any_bf16 = false, any_grad_out = false;
    std::vector<fsdp::Range> rs;
    std::vector<const void*> table_host;  // the tables of slice pointers, shard after shard
    std::vector<int64_t> table_off;       // per desc: its table's offset, or -1
    int64_t total = 0, total_valid = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        const fsdp_mt_tensor& t = tensors[i];
        char tag[64];
        snprintf(tag, sizeof tag, "%s: shard %d", who, i);
        int32_t st;
        if ((st = check_sizes(t.shard_numel, t.valid, tag)) != FSDP_OK) return st;
        const bool table = t.grad_slice_ptrs != nullptr;
        if (table) {
            if ((st = check_slice_table(t.grad_slice_ptrs, slice_dtype, n_slices, t.valid, tag)) !=
                FSDP_OK)
                return st;
        } else if ((st = check_slices(t.grad_slices, slice_dtype, t.slice_stride, n_slices,
                                      t.shard_numel, t.valid, tag)) != FSDP_OK) {
            return st;
        }
        if (t.shard_numel > 0 && (!t.param_fp32 || !t.exp_avg || !t.exp_avg_sq))
            return fail(FSDP_E_ARG, "%s: null param / exp_avg / exp_avg_sq", tag);
        if (!aligned(t.param_fp32, 4) || !aligned(t.exp_avg, 4) || !aligned(t.exp_avg_sq, 4) ||
            !aligned(t.grad_shard_out, 4) || !aligned(t.unshard_bf16_out, 2))
            return fail(FSDP_E_ALIGN, "%s: buffer not aligned to its element size", tag);
        if (!fsdp::add_i64(total, t.shard_numel, &total))
            return fail(FSDP_E_ARG, "%s: total size overflows", who);
        total_valid += t.valid;
        if (t.unshard_fp8_out) any_fp8 = true;
        if (t.shard_numel == 0) continue;
        if (!t.grad_shard_out) all_grad_out = false;
        if (!t.unshard_fp8_out) all_fp8 = false;
        if (t.grad_shard_out) any_grad_out = true;
        if (t.unshard_bf16_out) any_bf16 = true;
        rs.push_back(range_of(t.param_fp32, t.shard_numel, 4, true, i, "param"));
        rs.push_back(range_of(t.exp_avg, t.shard_numel, 4, true, i, "exp_avg"));
        rs.push_back(range_of(t.exp_avg_sq, t.shard_numel, 4, true, i, "exp_avg_sq"));
        if (t.unshard_bf16_out)
            rs.push_back(range_of(t.unshard_bf16_out, t.shard_numel, 2, true, i, "unshard_bf16_out"));
        if (t.grad_shard_out)
            rs.push_back(range_of(t.grad_shard_out, t.shard_numel, 4, true, i, "grad_shard_out"));
        if (t.unshard_fp8_out)
            rs.push_back(range_of(t.unshard_fp8_out, t.shard_numel, 1, true, i, "unshard_fp8_out"));
        if (table) {
            for (int32_t q = 0; q < n_slices && t.valid > 0; ++q)
                rs.push_back(range_of(t.grad_slice_ptrs[q], t.valid, dtype_bytes(slice_dtype), false,
                                      i, "grad_slice_ptrs"));
            table_off.push_back(static_cast<int64_t>(table_host.size()));
            table_host.insert(table_host.end(), t.grad_slice_ptrs, t.grad_slice_ptrs + n_slices);
        } else {
            add_slice_ranges(rs, t.grad_slices, slice_dtype, t.slice_stride, n_slices, t.valid, i);
            table_off.push_back(-1);
        }
        TensorDesc d{};
        d.param = t.param_fp32;
        d.m = t.exp_avg;
        d.v = t.exp_avg_sq;
        d.slices = table ? nullptr : t.grad_slices;
        d.out_bf16 = t.unshard_bf16_out;
        d.grad_out = t.grad_shard_out;
        d.out_fp8 = t.unshard_fp8_out;
        d.index = i;
        d.slice_stride = table ? 0 : t.slice_stride;
        d.shard_numel = t.shard_numel;
        d.valid = t.valid;
        const void* const* tab = table ? t.grad_slice_ptrs : nullptr;
        d.vec_ok = state_vec_ok(d);
        d.gen = d.vec_ok ? plan_gen(d, slice_dtype, n_slices, tab) : 0;
        // A shard whose fp32 buffers all start the same 1-3 elements past a
        // vector boundary (shards packed back to back after one whose size is
        // not a multiple of 4) is split in two under its index: a head of
        // those elements, which takes the element path, and the aligned rest,
        // which streams in vectors.  Their chunk entries are adjacent, so the
        // shard's workgroups stay one run.
        const int phase = d.vec_ok ? 0 : element_phase(d);
        const int64_t head = phase > 0 ? 4 - phase : 0;
        if (head > 0 && d.valid >= head + kGroup) {
            const int64_t es = dtype_bytes(slice_dtype);
            TensorDesc b = d;
            b.param += head;
            b.m += head;
            b.v += head;
            if (b.grad_out) b.grad_out += head;
            if (b.out_bf16) b.out_bf16 += head;
            if (b.out_fp8) b.out_fp8 += head;
            if (b.slices) b.slices = static_cast<const char*>(b.slices) + head * es;
            b.shard_numel -= head;
            b.valid -= head;
            d.shard_numel = head;
            d.valid = head;
            d.vec_ok = 0;
            d.gen = 0;
            b.vec_ok = state_vec_ok(b);
            if (table) {
                table_off.push_back(static_cast<int64_t>(table_host.size()));
                for (int32_t q = 0; q < n_slices; ++q)
                    table_host.push_back(static_cast<const char*>(t.grad_slice_ptrs[q]) + head * es);
                b.gen = b.vec_ok ? plan_gen(b, slice_dtype, n_slices, table_host.data() + table_off.back())
                                 : 0;
            } else {
                table_off.push_back(-1);
                b.gen = b.vec_ok ? plan_gen(b, slice_dtype, n_slices, nullptr) : 0;
            }
            descs.push_back(d);
            descs.push_back(b);
        } else {
            descs.push_back(d);
        }
    }
    if (descs.size() > static_cast<size_t>(INT32_MAX))
        return fail(FSDP_E_CAPACITY, "%s: too many shards", who);
    {
        const int32_t st = fsdp::check_aliases(rs);
        if (st != FSDP_OK) return st;
    }
    fsdp::Footprint footprint;
    footprint.build(rs);

    // Every chunk but a shard's last is kChunk elements, so every chunk and
    // every tile starts group-aligned.  Workgroup b takes tile b % 8 of entry b / 8.
    // The launch's size is checked before any table is built: a shard too
    // large for one launch is refused without building its entries.
    const int64_t chunk = kChunk;
    int64_t n_chunks = 0;
    for (const TensorDesc& d : descs) n_chunks += (d.shard_numel + chunk - 1) / chunk;
    {
        const int32_t st = check_grid(n_chunks * kTilesPerChunk, who);
        if (st != FSDP_OK) return st;
    }
    if (any_fp8) {
        // the per-shard amax pass runs one kAmaxBlock-thread workgroup per shard
        const int32_t st = check_grid(int64_t(n_tensors) * (kAmaxBlock / kBlock), who);
        if (st != FSDP_OK) return st;
    }
    std::vector<ChunkDesc> chunks;
    chunks.reserve(static_cast<size_t>(n_chunks));
    std::vector<ShardTiles> runs(static_cast<size_t>(n_tensors), ShardTiles{0, 0});
    for (size_t i = 0; i < descs.size(); ++i) {
        // a split shard's two parts are adjacent: one run of workgroups
        ShardTiles& run = runs[static_cast<size_t>(descs[i].index)];
        if (run.count == 0) run.first = static_cast<int64_t>(chunks.size()) * kTilesPerChunk;
        run.count += (descs[i].shard_numel + chunk - 1) / chunk * kTilesPerChunk;
        for (int64_t b = 0; b < descs[i].shard_numel; b += chunk) {
            ChunkDesc cd{};
            cd.begin = b;
            cd.tensor = static_cast<int32_t>(i);
            cd.count = static_cast<int32_t>(std::min(chunk, descs[i].shard_numel - b));
            chunks.push_back(cd);
        }
    }

    fsdp_mt_plan* plan = new (std::nothrow) fsdp_mt_plan();
    if (!plan) return fail(FSDP_E_CAPACITY, "%s: out of host memory", who);
    plan->n_slices = n_slices;
    plan->slice_dtype = slice_dtype;
    plan->n_tensors = n_tensors;
    plan->n_chunks = static_cast<int64_t>(chunks.size());
    plan->n_blocks = plan->n_chunks * kTilesPerChunk;
    plan->total_numel = total;
    plan->total_valid = total_valid;
    plan->chunk_numel = chunk;
    plan->all_grad_out = all_grad_out;
    plan->any_fp8 = any_fp8;
    plan->all_fp8 = all_fp8;
    plan->any_bf16 = any_bf16;
    plan->any_grad_out = any_grad_out;
    plan->any_general = !table_host.empty() ||
                        std::any_of(descs.begin(), descs.end(), [](const TensorDesc& x) { return x.gen != 0; });
    plan->footprint = std::move(footprint);
    plan->store_pol = store_policy(plan);
    plan->has_run = RS_RUN_STEP && merge_run(descs, slice_dtype, n_slices, &plan->run);
    hipError_t e = hipGetDevice(&plan->device);
    int pools = 0;
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&pools, hipDeviceAttributeMemoryPoolsSupported, plan->device);
    plan->pooled = pools != 0;
    if (e == hipSuccess && !chunks.empty()) e = hipEventCreateWithFlags(&plan->done, hipEventDisableTiming);
    auto alloc = [&](auto** p, size_t bytes) {
        return plan_alloc(plan, reinterpret_cast<void**>(p), bytes, stream);
    };
    if (e == hipSuccess && any_fp8 && n_tensors > 0) {
        e = alloc(&plan->d_shard_tiles, runs.size() * sizeof(ShardTiles));
        if (e == hipSuccess)
            e = hipMemcpyAsync(plan->d_shard_tiles, runs.data(), runs.size() * sizeof(ShardTiles),
                               hipMemcpyHostToDevice, stream);
        if (e == hipSuccess && !chunks.empty())
            e = alloc(&plan->d_tile_amax, static_cast<size_t>(plan->n_blocks) * sizeof(uint32_t));
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
    }
    if (e == hipSuccess && !chunks.empty() && !table_host.empty()) {
        e = alloc(&plan->d_slice_ptrs, table_host.size() * sizeof(const void*));
        if (e == hipSuccess)
            e = hipMemcpyAsync(plan->d_slice_ptrs, table_host.data(),
                               table_host.size() * sizeof(const void*), hipMemcpyHostToDevice,
                               stream);
        for (size_t k = 0; e == hipSuccess && k < descs.size(); ++k)
            if (table_off[k] >= 0) descs[k].slice_ptrs = plan->d_slice_ptrs + table_off[k];
    }
    if (e == hipSuccess && !chunks.empty()) {
        e = alloc(&plan->d_tensors, descs.size() * sizeof(TensorDesc));
        if (e == hipSuccess) e = alloc(&plan->d_chunks, chunks.size() * sizeof(ChunkDesc));
        if (e == hipSuccess) e = alloc(&plan->d_consts, sizeof(StepConsts));
        if (e == hipSuccess && all_grad_out)
            e = alloc(&plan->d_partials, static_cast<size_t>(plan->n_blocks + kSumBlocks) * sizeof(double));
        if (e == hipSuccess)
            e = hipMemcpyAsync(plan->d_tensors, descs.data(), descs.size() * sizeof(TensorDesc),
                               hipMemcpyHostToDevice, stream);
        if (e == hipSuccess)
            e = hipMemcpyAsync(plan->d_chunks, chunks.data(), chunks.size() * sizeof(ChunkDesc),
                               hipMemcpyHostToDevice, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
    }
    if (e != hipSuccess) {
        // uploads queued before the failure finish before their tables are freed
        (void)hipStreamSynchronize(stream);
        (void)hipGetLastError();
        fsdp_mt_plan_destroy(plan);
        return fail(FSDP_E_HIP, "%s: %s", who, hipGetErrorString(e));
    }
    *plan_out = plan;
    return FSDP_OK;
}

// A step's scalars for a plan launch: from hp on the host, or, with a device
// step count, advance the count and derive them on the device (a one-lane
// launch queued first) into the plan's slot, which *cdev then names.  hp's
// own step is not used then, nor hp's lr when lr_dev is given.
static int32_t queue_step_consts(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp, int64_t* step_dev,
                                 const double* lr_dev, hipStream_t stream, StepConsts* c,
                                 const StepConsts** cdev, const char* who) {
    *cdev = nullptr;
    *c = make_consts(hp, plan->n_slices);
    if (!step_dev) return FSDP_OK;
    hipLaunchKernelGGL(step_count_kernel, dim3(1), dim3(kBlock), 0, stream, step_dev, lr_dev, *c, hp->lr,
                       hp->weight_decay, hp->beta1, hp->beta2,
                       plan->n_chunks > 0 ? plan->d_consts : nullptr);
    *cdev = plan->d_consts;
    return launch_status(who);
}

// Two device buffers of a call on one plan may not overlap each other.
static int32_t check_disjoint(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes,
                              const char* who, const char* what) {
    if (!a || !b || a_bytes <= 0 || b_bytes <= 0) return FSDP_OK;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    if (x < y + static_cast<uintptr_t>(b_bytes) && y < x + static_cast<uintptr_t>(a_bytes))
        return fail(FSDP_E_ALIAS, "%s: %s", who, what);
    return FSDP_OK;
}

// The hyperparameter and step-count checks of the calls that take a device
// step count: hp as for a call (its step aside), step_dev a device int64
// that is no buffer of the plan's, and lr_dev (optional) a device double that
// may lie only in the plan's read-only slices and not on step_dev.
static int32_t check_step_dev(const fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp, const int64_t* step_dev,
                              const double* lr_dev, const char* who) {
    if (!hp) return fail(FSDP_E_ARG, "%s: null hyperparameters", who);
    fsdp_adamw_hparams h = *hp;
    h.step = 1;
    int32_t st;
    if ((st = check_hparams(&h)) != FSDP_OK) return st;
    if (!step_dev) return fail(FSDP_E_ARG, "%s: null step_dev", who);
    if (!aligned(step_dev, 8)) return fail(FSDP_E_ALIGN, "%s: step_dev not 8-byte aligned", who);
    if (!aligned(lr_dev, 8)) return fail(FSDP_E_ALIGN, "%s: lr_dev not 8-byte aligned", who);
    if ((st = check_extra(plan, step_dev, 8, true, who, "step_dev")) != FSDP_OK ||
        (st = check_extra(plan, lr_dev, 8, false, who, "lr_dev")) != FSDP_OK)
        return st;
    return check_disjoint(step_dev, 8, lr_dev, 8, who, "step_dev overlaps lr_dev");
}

// capturable: the count comes from step_dev (which must then be given).
static int32_t mt_step_impl(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp, bool capturable,
                            int64_t* step_dev, const double* lr_dev, hipStream_t stream, const char* who) {
    if (!plan) return fail(FSDP_E_ARG, "%s: null plan", who);
    int32_t st;
    if ((st = capturable ? check_step_dev(plan, hp, step_dev, lr_dev, who) : check_hparams(hp)) != FSDP_OK)
        return st;
    if ((st = check_plan_device(plan, who)) != FSDP_OK) return st;
    StepConsts c;
    const StepConsts* cdev;
    if ((st = queue_step_consts(plan, hp, step_dev, lr_dev, stream, &c, &cdev, who)) != FSDP_OK) return st;
    if (plan->n_chunks == 0) return FSDP_OK;
    const int64_t budget = plan->store_pol == kStWriteThrough     ? RS_INFLIGHT_KB_WT
                           : plan->store_pol == kStNtWriteThrough ? RS_INFLIGHT_KB_NTWT
                                                                  : RS_INFLIGHT_KB;
    if (plan->has_run) {
        const RunKernel k = pick_run(plan->slice_dtype, plan->n_slices, plan->store_pol, cdev != nullptr);
        // the smaller budget where a tile's slice loads are all in flight at
        // once (N compiled in); batched slice counts make several round trips
        // per wave and keep the general one
        const int32_t n = plan->n_slices;
        const bool one_batch = n == 1 || n == 2 || n == 4 || n == 8;
        const int64_t run_budget =
            plan->store_pol == kStWriteThrough && one_batch ? RS_INFLIGHT_KB_RUN : budget;
        plan_launch(plan, true, k, dim3(static_cast<uint32_t>(tiles_for(plan->run.shard_numel))),
                    dim3(kBlock), lds_reserve(step_bytes(plan), run_budget), stream, plan->run, c, cdev);
        return launch_status(who);
    }
    const size_t lds = lds_reserve(step_bytes(plan), budget);
    const MtKernel k = pick_mt(plan->slice_dtype, plan->n_slices, plan->any_general, plan->store_pol,
                               cdev != nullptr);
    plan_launch(plan, true, k, dim3(static_cast<uint32_t>(plan->n_blocks)), dim3(kBlock), lds, stream,
                plan->d_tensors, plan->d_chunks, c, cdev);
    return launch_status(who);
}

extern "C" int32_t fsdp_mt_step(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp,
                                hipStream_t stream) {
    return mt_step_impl(plan, hp, false, nullptr, nullptr, stream, "fsdp_mt_step");
}

extern "C" int32_t fsdp_mt_step_capturable(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp,
                                           int64_t* step_dev, const double* lr_dev, hipStream_t stream) {
    return mt_step_impl(plan, hp, true, step_dev, lr_dev, stream, "fsdp_mt_step_capturable");
}

extern "C" int32_t fsdp_mt_reduce_accumulate(fsdp_mt_plan* plan, int32_t accumulate,
                                             double* sqnorm_out, hipStream_t stream) {
    const char* who = "fsdp_mt_reduce_accumulate";
    if (!plan) return fail(FSDP_E_ARG, "%s: null plan", who);
    if (accumulate != 0 && accumulate != 1)
        return fail(FSDP_E_ARG, "%s: accumulate must be 0 or 1", who);
    if (sqnorm_out && !aligned(sqnorm_out, 8))
        return fail(FSDP_E_ALIGN, "%s: sqnorm_out not 8-byte aligned", who);
    if (!plan->all_grad_out)
        return fail(FSDP_E_ARG, "%s: every shard of the plan needs a grad_shard_out", who);
    int32_t st;
    if ((st = check_extra(plan, sqnorm_out, 8, true, who, "sqnorm_out")) != FSDP_OK) return st;
    if ((st = check_plan_device(plan, who)) != FSDP_OK) return st;
    const bool sq = sqnorm_out != nullptr;
    if (plan->n_chunks > 0) {
        const StepConsts c = make_consts(nullptr, plan->n_slices);
        const ReduceStoreKernel k =
            pick_reduce_store(plan->slice_dtype, plan->n_slices, sq, plan->any_general,
                              write_policy(plan_slice_read(plan) + 4 * accumulate, 4));
        plan_launch(plan, !sq, k, dim3(static_cast<uint32_t>(plan->n_blocks)), dim3(kBlock),
                    lds_reserve(slice_bytes(plan) + 4 + 4 * accumulate,
                                accumulate ? RS_INFLIGHT_KB_ACC : RS_INFLIGHT_KB), stream,
                    plan->d_tensors, plan->d_chunks, c, accumulate, plan->d_partials);
        if ((st = launch_status(who)) != FSDP_OK) return st;
    }
    if (!sq) return FSDP_OK;
    if (plan->n_chunks == 0) {
        // nothing to sum: one workgroup over an empty range writes 0
        plan_launch(plan, true, sum_partials_kernel, dim3(1), dim3(kBlock), 0, stream,
                    static_cast<const double*>(nullptr), int64_t(0), int64_t(0), sqnorm_out);
        return launch_status(who);
    }
    // two fixed-order stages: n_blocks partials -> up to kSumBlocks -> one
    const int64_t n = plan->n_blocks;
    const int64_t per = (n + kSumBlocks - 1) / kSumBlocks;
    const int64_t stage = (n + per - 1) / per;
    double* second = plan->d_partials + n;
    hipLaunchKernelGGL(sum_partials_kernel, dim3(static_cast<uint32_t>(stage)), dim3(kBlock), 0,
                       stream, static_cast<const double*>(plan->d_partials), n, per, second);
    if ((st = launch_status(who)) != FSDP_OK) return st;
    plan_launch(plan, true, sum_partials_kernel, dim3(1), dim3(kBlock), 0, stream,
                static_cast<const double*>(second), stage, stage, sqnorm_out);
    return launch_status(who);
}

extern "C" int32_t fsdp_mt_reduce_sqnorm(fsdp_mt_plan* plan, double* sqnorm_out,
                                         hipStream_t stream) {
    if (!sqnorm_out) return fail(FSDP_E_ARG, "fsdp_mt_reduce_sqnorm: null sqnorm_out");
    return fsdp_mt_reduce_accumulate(plan, 0, sqnorm_out, stream);
}

static int32_t grad_accumulate_impl(float* acc, const void* micro, int32_t micro_dtype,
                                    int64_t numel, int32_t accumulate, hipStream_t stream) {
    const char* who = "fsdp_grad_accumulate";
    int32_t st;
    if ((st = check_sizes(numel, numel, who)) != FSDP_OK) return st;
    if (micro_dtype != FSDP_DT_F32 && micro_dtype != FSDP_DT_BF16)
        return fail(FSDP_E_DTYPE, "%s: unknown micro-batch dtype %d", who, micro_dtype);
    if (accumulate != 0 && accumulate != 1)
        return fail(FSDP_E_ARG, "%s: accumulate must be 0 or 1", who);
    if (numel == 0) return FSDP_OK;
    if (!acc || !micro) return fail(FSDP_E_ARG, "%s: null acc or micro", who);
    if (!aligned(acc, 4) || !aligned(micro, dtype_bytes(micro_dtype)))
        return fail(FSDP_E_ALIGN, "%s: buffer not aligned to its element size", who);
    std::vector<fsdp::Range> rs{range_of(acc, numel, 4, true, 0, "acc"),
                                range_of(micro, numel, dtype_bytes(micro_dtype), false, 0, "micro")};
    if ((st = fsdp::check_aliases(rs)) != FSDP_OK) return st;
    const int64_t blocks = tiles_for(numel);
    if ((st = check_grid(blocks, who)) != FSDP_OK) return st;
    // the vector path needs the accumulator aligned; a micro-batch gradient
    // off a vector boundary takes the shifted loads
    const int32_t vec = aligned(acc, kF32Vec);
    const bool gen = vec && !aligned(micro, micro_dtype == FSDP_DT_BF16 ? kBf16Vec : kF32Vec);
    const AccumulateKernel k =
        pick_accumulate(micro_dtype == FSDP_DT_BF16, gen,
                        write_policy(dtype_bytes(micro_dtype) + 4 * accumulate, 4));
    hipLaunchKernelGGL(k, dim3(static_cast<uint32_t>(blocks)), dim3(kBlock),
                       lds_reserve(dtype_bytes(micro_dtype) + 4 + 4 * accumulate), stream, acc, micro,
                       numel, accumulate, vec);
    return launch_status(who);
}

static int32_t clip_coef_impl(float* coef_out, double* norm_out, const double* sqnorms,
                              int32_t n_ranks, double max_norm, hipStream_t stream) {
    const char* who = "fsdp_clip_coef";
    if (!coef_out || !sqnorms) return fail(FSDP_E_ARG, "%s: null coef_out or sqnorms", who);
    if (n_ranks < 1 || n_ranks > (1 << 20))
        return fail(FSDP_E_ARG, "%s: n_ranks %d outside [1, 2^20]", who, n_ranks);
    if (!std::isfinite(max_norm) || max_norm < 0)
        return fail(FSDP_E_ARG, "%s: max_norm must be finite and >= 0", who);
    if (!aligned(coef_out, 4) || !aligned(sqnorms, 8) || !aligned(norm_out, 8))
        return fail(FSDP_E_ALIGN, "%s: buffer not aligned to its element size", who);
    std::vector<fsdp::Range> rs{range_of(coef_out, 1, 4, true, 0, "coef_out"),
                                range_of(sqnorms, n_ranks, 8, false, 0, "sqnorms")};
    if (norm_out) rs.push_back(range_of(norm_out, 1, 8, true, 0, "norm_out"));
    int32_t st;
    if ((st = fsdp::check_aliases(rs)) != FSDP_OK) return st;
    hipLaunchKernelGGL(clip_coef_kernel, dim3(1), dim3(64), 0, stream, coef_out, norm_out, sqnorms,
                       n_ranks, max_norm);
    return launch_status(who);
}

static int32_t mt_step_clipped_impl(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp, bool capturable,
                                    int64_t* step_dev, const double* lr_dev, const float* grad_scale,
                                    hipStream_t stream, const char* who) {
    if (!plan) return fail(FSDP_E_ARG, "%s: null plan", who);
    int32_t st;
    if ((st = capturable ? check_step_dev(plan, hp, step_dev, lr_dev, who) : check_hparams(hp)) != FSDP_OK)
        return st;
    if (!grad_scale) return fail(FSDP_E_ARG, "%s: null grad_scale", who);
    if (!aligned(grad_scale, 4)) return fail(FSDP_E_ALIGN, "%s: grad_scale misaligned", who);
    if (!plan->all_grad_out)
        return fail(FSDP_E_ARG, "%s: every shard of the plan needs a grad_shard_out", who);
    if ((st = check_extra(plan, grad_scale, 4, false, who, "grad_scale")) != FSDP_OK) return st;
    if ((st = check_disjoint(step_dev, 8, grad_scale, 4, who, "step_dev overlaps grad_scale")) != FSDP_OK)
        return st;
    if ((st = check_plan_device(plan, who)) != FSDP_OK) return st;
    StepConsts c;
    const StepConsts* cdev;
    if ((st = queue_step_consts(plan, hp, step_dev, lr_dev, stream, &c, &cdev, who)) != FSDP_OK) return st;
    if (plan->n_chunks == 0) return FSDP_OK;
    const ScaledStepKernel k =
        pick_scaled_step(plan->any_general, write_policy(4 + 12, 12 + 2 * plan->any_bf16), cdev != nullptr);
    plan_launch(plan, true, k, dim3(static_cast<uint32_t>(plan->n_blocks)), dim3(kBlock),
                lds_reserve(4 + 24 + 2 * plan->any_bf16), stream, plan->d_tensors, plan->d_chunks, c,
                grad_scale, cdev);
    return launch_status(who);
}

extern "C" int32_t fsdp_mt_step_clipped(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp,
                                        const float* grad_scale, hipStream_t stream) {
    return mt_step_clipped_impl(plan, hp, false, nullptr, nullptr, grad_scale, stream,
                                "fsdp_mt_step_clipped");
}

extern "C" int32_t fsdp_mt_step_clipped_capturable(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp,
                                                   int64_t* step_dev, const double* lr_dev,
                                                   const float* grad_scale, hipStream_t stream) {
    return mt_step_clipped_impl(plan, hp, true, step_dev, lr_dev, grad_scale, stream,
                                "fsdp_mt_step_clipped_capturable");
}

static int32_t mt_step_amax_impl(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp, bool capturable,
                                 int64_t* step_dev, const double* lr_dev, float* amax_out, hipStream_t stream,
                                 const char* who) {
    if (!plan) return fail(FSDP_E_ARG, "%s: null plan", who);
    int32_t st;
    if ((st = capturable ? check_step_dev(plan, hp, step_dev, lr_dev, who) : check_hparams(hp)) != FSDP_OK)
        return st;
    if (!plan->any_fp8) return fail(FSDP_E_ARG, "%s: the plan has no fp8 outputs", who);
    if (!amax_out) return fail(FSDP_E_ARG, "%s: null amax_out", who);
    if (!aligned(amax_out, 4)) return fail(FSDP_E_ALIGN, "%s: amax_out misaligned", who);
    if ((st = check_extra(plan, amax_out, 4 * plan->n_tensors, true, who, "amax_out")) != FSDP_OK)
        return st;
    if ((st = check_disjoint(step_dev, 8, amax_out, 4 * plan->n_tensors, who,
                             "step_dev overlaps amax_out")) != FSDP_OK ||
        (st = check_disjoint(lr_dev, 8, amax_out, 4 * plan->n_tensors, who,
                             "lr_dev overlaps amax_out")) != FSDP_OK)
        return st;
    if ((st = check_plan_device(plan, who)) != FSDP_OK) return st;
    StepConsts c;
    const StepConsts* cdev;
    if ((st = queue_step_consts(plan, hp, capturable ? step_dev : nullptr, lr_dev, stream, &c, &cdev, who)) !=
        FSDP_OK)
        return st;
    if (plan->n_tensors == 0) return FSDP_OK;
    if (plan->n_chunks > 0) {
        const AmaxKernel k = pick_amax(plan->slice_dtype, plan->n_slices, plan->any_general,
                                       write_policy(plan_slice_read(plan) + 12, 12 + plan_copy_write(plan)),
                                       cdev != nullptr);
        hipLaunchKernelGGL(k, dim3(static_cast<uint32_t>(plan->n_blocks)), dim3(kBlock),
                           lds_reserve(step_bytes(plan), RS_INFLIGHT_KB_FP8), stream, plan->d_tensors,
                           plan->d_chunks, c, plan->d_tile_amax, cdev);
        if ((st = launch_status(who)) != FSDP_OK) return st;
    }
    plan_launch(plan, true, shard_amax_kernel, dim3(static_cast<uint32_t>(plan->n_tensors)),
                dim3(kAmaxBlock), 0, stream, static_cast<const ShardTiles*>(plan->d_shard_tiles),
                static_cast<const uint32_t*>(plan->d_tile_amax), plan->n_blocks / kXcds, amax_out);
    return launch_status(who);
}

extern "C" int32_t fsdp_mt_step_amax(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp,
                                     float* amax_out, hipStream_t stream) {
    return mt_step_amax_impl(plan, hp, false, nullptr, nullptr, amax_out, stream, "fsdp_mt_step_amax");
}

extern "C" int32_t fsdp_mt_step_amax_capturable(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp,
                                                int64_t* step_dev, const double* lr_dev, float* amax_out,
                                                hipStream_t stream) {
    return mt_step_amax_impl(plan, hp, true, step_dev, lr_dev, amax_out, stream,
                             "fsdp_mt_step_amax_capturable");
}

static int32_t mt_cast_fp8_impl(fsdp_mt_plan* plan, const float* amax_ranks, int32_t n_ranks,
                                float* scale_out, hipStream_t stream) {
    const char* who = "fsdp_mt_cast_fp8";
    if (!plan) return fail(FSDP_E_ARG, "%s: null plan", who);
    if (!plan->all_fp8) return fail(FSDP_E_ARG, "%s: every shard of the plan needs an fp8 output", who);
    if (n_ranks < 1 || n_ranks > (1 << 20))
        return fail(FSDP_E_ARG, "%s: n_ranks %d outside [1, 2^20]", who, n_ranks);
    if (plan->n_tensors > 0 && !amax_ranks) return fail(FSDP_E_ARG, "%s: null amax_ranks", who);
    if (!aligned(amax_ranks, 4) || !aligned(scale_out, 4))
        return fail(FSDP_E_ALIGN, "%s: buffer not aligned to its element size", who);
    if (scale_out && amax_ranks) {
        std::vector<fsdp::Range> rs{range_of(scale_out, plan->n_tensors, 4, true, 0, "scale_out"),
                                    range_of(amax_ranks, plan->n_tensors * n_ranks, 4, false, 0,
                                             "amax_ranks")};
        int32_t st;
        if ((st = fsdp::check_aliases(rs)) != FSDP_OK) return st;
    }
    int32_t st;
    if ((st = check_extra(plan, amax_ranks, 4 * plan->n_tensors * n_ranks, false, who,
                          "amax_ranks")) != FSDP_OK ||
        (st = check_extra(plan, scale_out, 4 * plan->n_tensors, true, who, "scale_out")) != FSDP_OK)
        return st;
    if ((st = check_plan_device(plan, who)) != FSDP_OK) return st;
    if (plan->n_chunks == 0) return FSDP_OK;
    // 4 bytes read per code written: write-through (the rule above)
    const auto k = by_policy(write_policy(4, 1), [&](auto P) {
        constexpr int kPol = decltype(P)::value;
        return plan->any_general ? mt_cast_fp8_kernel<true, kPol> : mt_cast_fp8_kernel<false, kPol>;
    });
    plan_launch(plan, true, k,
                dim3(static_cast<uint32_t>(plan->n_chunks * (kTilesPerChunk / RS_CAST_TILES))),
                dim3(kBlock), 0, stream, plan->d_tensors, plan->d_chunks, amax_ranks, n_ranks,
                plan->n_tensors, scale_out);
    return launch_status(who);
}

static int32_t mt_step_fp8_impl(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp, bool capturable,
                                int64_t* step_dev, const double* lr_dev, const float* scale_in, float* amax_out,
                                hipStream_t stream, const char* who) {
    if (!plan) return fail(FSDP_E_ARG, "%s: null plan", who);
    int32_t st;
    if ((st = capturable ? check_step_dev(plan, hp, step_dev, lr_dev, who) : check_hparams(hp)) != FSDP_OK)
        return st;
    if (!plan->all_fp8) return fail(FSDP_E_ARG, "%s: every shard of the plan needs an fp8 output", who);
    if (plan->n_tensors > 0 && (!scale_in || !amax_out))
        return fail(FSDP_E_ARG, "%s: null scale_in or amax_out", who);
    if (!aligned(scale_in, 4) || !aligned(amax_out, 4))
        return fail(FSDP_E_ALIGN, "%s: buffer not aligned to its element size", who);
    if (scale_in && amax_out) {
        std::vector<fsdp::Range> rs{range_of(amax_out, plan->n_tensors, 4, true, 0, "amax_out"),
                                    range_of(scale_in, plan->n_tensors, 4, false, 0, "scale_in")};
        if ((st = fsdp::check_aliases(rs)) != FSDP_OK) return st;
    }
    if ((st = check_extra(plan, scale_in, 4 * plan->n_tensors, false, who, "scale_in")) != FSDP_OK ||
        (st = check_extra(plan, amax_out, 4 * plan->n_tensors, true, who, "amax_out")) != FSDP_OK)
        return st;
    if ((st = check_disjoint(step_dev, 8, amax_out, 4 * plan->n_tensors, who,
                             "step_dev overlaps amax_out")) != FSDP_OK ||
        (st = check_disjoint(step_dev, 8, scale_in, 4 * plan->n_tensors, who,
                             "step_dev overlaps scale_in")) != FSDP_OK ||
        (st = check_disjoint(lr_dev, 8, amax_out, 4 * plan->n_tensors, who,
                             "lr_dev overlaps amax_out")) != FSDP_OK)
        return st;
    if ((st = check_plan_device(plan, who)) != FSDP_OK) return st;
    StepConsts c;
    const StepConsts* cdev;
    if ((st = queue_step_consts(plan, hp, capturable ? step_dev : nullptr, lr_dev, stream, &c, &cdev, who)) !=
        FSDP_OK)
        return st;
    if (plan->n_tensors == 0) return FSDP_OK;
    if (plan->n_chunks > 0) {
        const Fp8StepKernel k =
            pick_fp8_step(plan->slice_dtype, plan->n_slices, plan->any_general,
                          write_policy(plan_slice_read(plan) + 12, 12 + plan_copy_write(plan) + plan->any_fp8),
                          cdev != nullptr);
        hipLaunchKernelGGL(k, dim3(static_cast<uint32_t>(plan->n_blocks)), dim3(kBlock),
                           lds_reserve(step_bytes(plan) + 1, RS_INFLIGHT_KB_FP8), stream, plan->d_tensors,
                           plan->d_chunks, c, scale_in, plan->d_tile_amax, cdev);
        if ((st = launch_status(who)) != FSDP_OK) return st;
    }
    plan_launch(plan, true, shard_amax_kernel, dim3(static_cast<uint32_t>(plan->n_tensors)),
                dim3(kAmaxBlock), 0, stream, static_cast<const ShardTiles*>(plan->d_shard_tiles),
                static_cast<const uint32_t*>(plan->d_tile_amax), plan->n_blocks / kXcds, amax_out);
    return launch_status(who);
}

// ---------------------------------------------------------------- no device allocation

// Per-workgroup partial sums of fsdp_reduce_sqnorm_noalloc, then its
// kSumBlocks second-stage sums.  Device code never names this array: host
// code looks up its address on each device (hipGetSymbolAddress) and passes
// that address to the kernels, as a plan passes its own partials.
constexpr int64_t kScratchDoubles = FSDP_NOALLOC_SCRATCH_BYTES / sizeof(double);
static __device__ __align__(256) double scratch[kScratchDoubles];

namespace {

// The largest shard whose partials and second-stage sums fit the array, in
// whole chunk entries.
constexpr int64_t kNoAllocMaxBlocks = (kScratchDoubles - kSumBlocks) / kTilesPerChunk * kTilesPerChunk;
static_assert(FSDP_NOALLOC_MAX_NUMEL == kNoAllocMaxBlocks / kTilesPerChunk * kChunk,
              "the header's size limit is what the scratch array holds");

std::mutex g_scratch_mu;
double* g_scratch_dev[kMaxDevices] = {};  // the array's address on each device, once looked up

// The scratch array's address on the current device, looked up on the first
// call there with that device current.
int32_t scratch_on_current_device(double** out, const char* who) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FSDP_E_HIP, "%s: %s", who, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(FSDP_E_STATE, "%s: device %d beyond the %d this library tracks", who, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(FSDP_E_HIP, "%s: address of the scratch array on device %d: %s", who, dev,
                        hipGetErrorString(e));
        g_scratch_dev[dev] = static_cast<double*>(p);
    }
    *out = g_scratch_dev[dev];
    return FSDP_OK;
}

bool overlaps(uintptr_t a_lo, uintptr_t a_hi, uintptr_t b_lo, uintptr_t b_hi) {
    return a_lo < a_hi && b_lo < b_hi && a_lo < b_hi && b_lo < a_hi;
}

}  // namespace

extern "C" int32_t fsdp_reduce_sqnorm_noalloc(float* grad_shard_out, double* sqnorm_out,
                                              const void* grad_slices, int32_t slice_dtype,
                                              int64_t slice_stride, int32_t n_slices,
                                              int64_t shard_numel, int64_t valid, hipStream_t stream) {
    const char* who = "fsdp_reduce_sqnorm_noalloc";
    int32_t st;
    if ((st = check_sizes(shard_numel, valid, who)) != FSDP_OK) return st;
    if ((st = check_slices(grad_slices, slice_dtype, slice_stride, n_slices, shard_numel, valid,
                           who)) != FSDP_OK)
        return st;
    if (shard_numel > FSDP_NOALLOC_MAX_NUMEL)
        return fail(FSDP_E_CAPACITY, "%s: shard_numel %lld exceeds FSDP_NOALLOC_MAX_NUMEL (%lld): "
                    "the partial sums would not fit the library's %d-byte scratch array", who,
                    static_cast<long long>(shard_numel), static_cast<long long>(FSDP_NOALLOC_MAX_NUMEL),
                    FSDP_NOALLOC_SCRATCH_BYTES);
    if (!sqnorm_out) return fail(FSDP_E_ARG, "%s: null sqnorm_out", who);
    if (!aligned(sqnorm_out, 8)) return fail(FSDP_E_ALIGN, "%s: sqnorm_out not 8-byte aligned", who);
    if (shard_numel > 0 && !grad_shard_out) return fail(FSDP_E_ARG, "%s: null grad_shard_out", who);
    if (!aligned(grad_shard_out, 4)) return fail(FSDP_E_ALIGN, "%s: grad_shard_out misaligned", who);
    // overlaps, checked pairwise (nothing allocated): the two outputs against
    // each other and against every slice
    const uintptr_t g_lo = reinterpret_cast<uintptr_t>(grad_shard_out);
    const uintptr_t g_hi = g_lo + static_cast<uintptr_t>(shard_numel) * 4;
    const uintptr_t s_lo = reinterpret_cast<uintptr_t>(sqnorm_out), s_hi = s_lo + 8;
    if (overlaps(g_lo, g_hi, s_lo, s_hi))
        return fail(FSDP_E_ALIAS, "%s: sqnorm_out overlaps grad_shard_out", who);
    if (valid > 0) {
        const int64_t es = dtype_bytes(slice_dtype);
        for (int32_t q = 0; q < n_slices; ++q) {
            const uintptr_t lo = reinterpret_cast<uintptr_t>(grad_slices) +
                                 static_cast<uintptr_t>(q * slice_stride * es);
            const uintptr_t hi = lo + static_cast<uintptr_t>(valid * es);
            if (overlaps(g_lo, g_hi, lo, hi) || overlaps(s_lo, s_hi, lo, hi))
                return fail(FSDP_E_ALIAS, "%s: an output overlaps gradient slice %d", who, q);
        }
    }
    double* partials = nullptr;
    if ((st = scratch_on_current_device(&partials, who)) != FSDP_OK) return st;
    if (shard_numel == 0) {
        // nothing to sum: one workgroup over an empty range writes 0
        hipLaunchKernelGGL(sum_partials_kernel, dim3(1), dim3(kBlock), 0, stream,
                           static_cast<const double*>(nullptr), int64_t(0), int64_t(0), sqnorm_out);
        return launch_status(who);
    }
    TensorDesc T{};
    T.slices = grad_slices;
    T.grad_out = grad_shard_out;
    T.slice_stride = slice_stride;
    T.shard_numel = shard_numel;
    T.valid = valid;
    T.vec_ok = aligned(grad_shard_out, kF32Vec);
    const bool gen = T.vec_ok && !slices_vec_ok(grad_slices, slice_dtype, slice_stride, n_slices);
    const StepConsts c = make_consts(nullptr, n_slices);
    const int64_t n = (shard_numel + kChunk - 1) / kChunk * kTilesPerChunk;
    const int64_t in_flight = dtype_bytes(slice_dtype) * inflight_slices(n_slices, slice_dtype);
    hipLaunchKernelGGL(pick_sqnorm_single(slice_dtype, n_slices, gen,
                                          write_policy(dtype_bytes(slice_dtype) * n_slices, 4)),
                       dim3(static_cast<uint32_t>(n)),
                       dim3(kBlock), lds_reserve(in_flight + 4), stream, T, c, partials);
    if ((st = launch_status(who)) != FSDP_OK) return st;
    // the same two fixed-order stages as a plan's: n partials -> up to
    // kSumBlocks -> one
    const int64_t per = (n + kSumBlocks - 1) / kSumBlocks;
    const int64_t stage = (n + per - 1) / per;
    double* second = partials + n;
    hipLaunchKernelGGL(sum_partials_kernel, dim3(static_cast<uint32_t>(stage)), dim3(kBlock), 0, stream,
                       static_cast<const double*>(partials), n, per, second);
    if ((st = launch_status(who)) != FSDP_OK) return st;
    hipLaunchKernelGGL(sum_partials_kernel, dim3(1), dim3(kBlock), 0, stream,
                       static_cast<const double*>(second), stage, stage, sqnorm_out);
    return launch_status(who);
}

// ---------------------------------------------------------------- entry points that allocate
// host memory: no C++ exception crosses the ABI

extern "C" int32_t fsdp_reduce_grad_shard(float* grad_shard_out, const void* grad_slices,
                                          int32_t slice_dtype, int64_t slice_stride,
                                          int32_t n_slices, int64_t shard_numel, int64_t valid,
                                          hipStream_t stream) {
    return fsdp::guarded("fsdp_reduce_grad_shard", [&] {
        return reduce_grad_shard_impl(grad_shard_out, grad_slices, slice_dtype, slice_stride,
                                      n_slices, shard_numel, valid, stream);
    });
}

extern "C" int32_t fsdp_adamw_shard_step(float* param_fp32, float* exp_avg, float* exp_avg_sq,
                                         const float* grad_shard, int64_t shard_numel,
                                         int64_t valid, const fsdp_adamw_hparams* hp,
                                         hipStream_t stream) {
    return fsdp::guarded("fsdp_adamw_shard_step", [&] {
        return adamw_shard_step_impl(param_fp32, exp_avg, exp_avg_sq, grad_shard, shard_numel,
                                     valid, hp, stream);
    });
}

extern "C" int32_t fsdp_cast_unshard_bf16(uint16_t* unshard_bf16_out, const float* param_fp32,
                                          int64_t shard_numel, int64_t valid, hipStream_t stream) {
    return fsdp::guarded("fsdp_cast_unshard_bf16", [&] {
        return cast_unshard_bf16_impl(unshard_bf16_out, param_fp32, shard_numel, valid, stream);
    });
}

extern "C" int32_t fsdp_mt_plan_create(fsdp_mt_plan** plan_out, const fsdp_mt_tensor* tensors,
                                       int32_t n_tensors, int32_t n_slices, int32_t slice_dtype,
                                       hipStream_t stream) {
    return fsdp::guarded("fsdp_mt_plan_create", [&] {
        return mt_plan_create_impl(plan_out, tensors, n_tensors, n_slices, slice_dtype, stream);
    });
}

extern "C" int32_t fsdp_grad_accumulate(float* acc, const void* micro, int32_t micro_dtype,
                                        int64_t numel, int32_t accumulate, hipStream_t stream) {
    return fsdp::guarded("fsdp_grad_accumulate", [&] {
        return grad_accumulate_impl(acc, micro, micro_dtype, numel, accumulate, stream);
    });
}

extern "C" int32_t fsdp_clip_coef(float* coef_out, double* norm_out, const double* sqnorms,
                                  int32_t n_ranks, double max_norm, hipStream_t stream) {
    return fsdp::guarded("fsdp_clip_coef", [&] {
        return clip_coef_impl(coef_out, norm_out, sqnorms, n_ranks, max_norm, stream);
    });
}

extern "C" int32_t fsdp_mt_cast_fp8(fsdp_mt_plan* plan, const float* amax_ranks, int32_t n_ranks,
                                    float* scale_out, hipStream_t stream) {
    return fsdp::guarded("fsdp_mt_cast_fp8", [&] {
        return mt_cast_fp8_impl(plan, amax_ranks, n_ranks, scale_out, stream);
    });
}

extern "C" int32_t fsdp_mt_step_fp8(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp,
                                    const float* scale_in, float* amax_out, hipStream_t stream) {
    return fsdp::guarded("fsdp_mt_step_fp8", [&] {
        return mt_step_fp8_impl(plan, hp, false, nullptr, nullptr, scale_in, amax_out, stream,
                                "fsdp_mt_step_fp8");
    });
}

extern "C" int32_t fsdp_mt_step_fp8_capturable(fsdp_mt_plan* plan, const fsdp_adamw_hparams* hp,
                                               int64_t* step_dev, const double* lr_dev, const float* scale_in,
                                               float* amax_out, hipStream_t stream) {
    return fsdp::guarded("fsdp_mt_step_fp8_capturable", [&] {
        return mt_step_fp8_impl(plan, hp, true, step_dev, lr_dev, scale_in, amax_out, stream,
                                "fsdp_mt_step_fp8_capturable");
    });
}

extern "C" int32_t fsdp_mt_plan_get_info(const fsdp_mt_plan* plan, fsdp_mt_plan_info* info) {
    if (!plan || !info) return fail(FSDP_E_ARG, "fsdp_mt_plan_get_info: null argument");
    info->n_tensors = plan->n_tensors;
    info->n_chunks = plan->n_chunks;
    info->n_blocks = plan->n_blocks;
    info->total_numel = plan->total_numel;
    info->total_valid = plan->total_valid;
    info->chunk_numel = plan->chunk_numel;
    info->n_slices = plan->n_slices;
    info->slice_dtype = plan->slice_dtype;
    info->step_one_range = plan->has_run ? 1 : 0;
    info->store_policy = plan->store_pol;
    return FSDP_OK;
}

extern "C" int32_t fsdp_mt_plan_destroy(fsdp_mt_plan* plan) {
    if (!plan) return FSDP_OK;
    hipError_t e = hipSuccess;
    // the plan's last launch (outside a graph capture) has finished; other
    // work on the device is not waited for
    if (plan->done) {
        e = hipEventSynchronize(plan->done);
        const hipError_t d = hipEventDestroy(plan->done);
        if (e == hipSuccess) e = d;
    }
    void* const bufs[] = {plan->d_slice_ptrs, plan->d_tensors, plan->d_chunks, plan->d_partials,
                          plan->d_tile_amax, plan->d_shard_tiles, plan->d_consts};
    const bool any = std::any_of(std::begin(bufs), std::end(bufs), [](void* b) { return b != nullptr; });
    if (any && plan->pooled) {
        // stream-ordered frees on the plan's device, which wait for nothing
        int cur = -1;
        hipError_t d = hipGetDevice(&cur);
        if (d == hipSuccess && cur != plan->device) d = hipSetDevice(plan->device);
        hipStream_t fs = nullptr;
        if (d == hipSuccess) d = free_stream(plan->device, &fs);
        for (void* b : bufs)
            if (b && d == hipSuccess) d = hipFreeAsync(b, fs);
        if (cur >= 0 && cur != plan->device) (void)hipSetDevice(cur);
        if (e == hipSuccess) e = d;
    } else if (any) {
        for (void* b : bufs)
            if (b) (void)hipFree(b);
    }
    delete plan;
    if (e != hipSuccess) return fail(FSDP_E_HIP, "fsdp_mt_plan_destroy: %s", hipGetErrorString(e));
    return FSDP_OK;
}
