// Internal helpers shared by the kvc HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "kvc.h"

namespace kvc {

// ---------------------------------------------------------------- host side

// Records the message for kvc_last_error() and returns `status`.
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Checks the launch just enqueued; returns KVC_OK or KVC_ERR_HIP.
int check_launch(const char *what);

// Validates a kvc_dims for the kernels' shape limits.
int check_dims(const kvc_dims *d, const char *who);

inline int64_t n_rows(const kvc_dims *d) {
    return (int64_t)d->n_seq * d->n_layers * d->n_kv_heads;
}

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------- bounds-checked builds
//
// Built with -DKVC_CHECK, an index wrapped in KVC_IDX(i, n, site) is checked
// against [0, n): one outside records `site` in this source file's device
// check word and is replaced by 0, an index that exists, so the access is
// reported instead of made. KVC_NOTE(cond, site) records caller data that the
// kernels clamp (kept indices past the cache, counts above their buffers, page
// spans, block-table entries). Normal builds compile both away: KVC_IDX(i, n,
// site) is i. kvc_check_read collects the words of every source and clears them.
enum : unsigned {
    KVC_CHK_SCORE = 1u << 0,     // score: key, query and score indices
    KVC_CHK_SELECT = 1u << 1,    // select: token, candidate and output indices
    KVC_CHK_COMPACT = 1u << 2,   // compaction: source tokens and destination slots
    KVC_CHK_DECODE = 1u << 3,    // decode: pool slots and partial slots
    KVC_CHK_POOL = 1u << 4,      // score pooling: tokens
    KVC_CHK_PAGE = 1u << 5,      // page effects and page scores: tokens and pages
    KVC_CHK_KEPT = 1u << 8,      // caller data: a kept index at or past the cache
    KVC_CHK_COUNT = 1u << 9,     // caller data: a count above its buffer
    KVC_CHK_SPAN = 1u << 10,     // caller data: a page span outside the cache or above the page size
    KVC_CHK_BLOCK = 1u << 11,    // caller data: a block-table entry outside the storage
};

#ifdef KVC_CHECK
static __device__ unsigned kvc_check_word;   // this source file's copy

template <class I>
__device__ __forceinline__ I kvc_idx(I i, int64_t n, unsigned site) {
    if ((int64_t)i >= 0 && (int64_t)i < n) return i;
    atomicOr(&kvc_check_word, site);
    return I(0);
}
#define KVC_IDX(i, n, site) ::kvc::kvc_idx((i), (int64_t)(n), (site))
#define KVC_NOTE(cond, site)                                          \
    do {                                                              \
        if (cond) atomicOr(&::kvc::kvc_check_word, (unsigned)(site)); \
    } while (0)
// Host: this source file's check word, read and cleared.
#define KVC_CHECK_READER(fn)                                                                        \
    unsigned fn() {                                                                                 \
        unsigned v = 0u, z = 0u;                                                                    \
        if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(kvc_check_word), sizeof v) != hipSuccess) return ~0u; \
        if (hipMemcpyToSymbol(HIP_SYMBOL(kvc_check_word), &z, sizeof z) != hipSuccess) return ~0u;   \
        return v;                                                                                   \
    }
#else
#define KVC_IDX(i, n, site) (i)
#define KVC_NOTE(cond, site) \
    do {                     \
    } while (0)
#define KVC_CHECK_READER(fn) \
    unsigned fn() { return 0u; }
#endif

// ---------------------------------------------------------------- device side

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// float -> bf16 with round-to-nearest-even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Row r = (n*L + l)*Hkv + h  ->  (n, l, h).
struct RowIdx {
    int n, l, h;
};
// Row indices fit 32 bits (the argument checks cap the row count at
// INT32_MAX), so the divisions are 32-bit ones.
__device__ __forceinline__ RowIdx split_row(int64_t r, int L, int Hkv) {
    RowIdx o;
    const uint32_t rr = (uint32_t)r, nl = rr / (uint32_t)Hkv;
    o.h = (int)(rr - nl * (uint32_t)Hkv);
    o.l = (int)(nl % (uint32_t)L);
    o.n = (int)(nl / (uint32_t)L);
    return o;
}

// Where the window sits: query w is at position qbase + w and sees keys
// j <= qbase + w; keys at or beyond kend are never read. lsel >= 0 restricts a
// launch to one layer: local row rr = n*Hkv + h maps to global row
// (n*L + lsel)*Hkv + h.
struct WindowGeom {
    int64_t qbase, kend;
    int lsel;
    __device__ __forceinline__ int64_t global_row(int64_t rr, int L, int Hkv) const {
        if (lsel < 0) return rr;
        return ((rr / Hkv) * L + lsel) * Hkv + rr % Hkv;
    }
};

// Row of the 32x32 MFMA accumulator held in register i by a lane in half `hf`
// (lanes 32..63 are half 1); the column is lane & 31.
__device__ __forceinline__ int acc_row(int i, int hf) { return (i >> 2) * 8 + hf * 4 + (i & 3); }

__device__ __forceinline__ bf16x8 load8(const uint16_t *p) {
    uint4 u = *reinterpret_cast<const uint4 *>(p);
    return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }


// Enqueues the softmax statistics of a query window (score pass 1 + merge):
// mm[rr][qr] = max + log2(sum) of the log2-domain logits of query row qr of
// local row rr. `part` holds rows_local * window_chunks(kend) * QRP float2.
int launch_window_stats(const kvc_dims *d, const uint16_t *K, const uint16_t *Q, int W, WindowGeom wg,
                        int64_t rows_local, float2 *part, float *mm, hipStream_t s);
int64_t window_chunks(int64_t kend);

// The single-read score kernel (score_once.hip): the number of workgroups it
// would run with for these dims on the current device (0: not applicable), and
// its workspace bytes; its launch (after a 256-byte control block the kernel
// clears); its wait bound and the diagnostic switch that stops the merges.
int score_once_plan(const kvc_dims *d, int W, size_t *ws_bytes);
int launch_score_once(const kvc_dims *d, const uint16_t *K, const uint16_t *Q, int W, float *scores, void *ws,
                      int nwg, hipStream_t s);
void set_score_wait(int64_t wait_us, bool no_merge);

// Lane exchanges inside a row of 16 lanes through DPP (no LDS traffic):
// quad_perm [1,0,3,2] and [2,3,0,1], then half-row and row mirrors. After the
// steps for N lanes every lane of each aligned group of N holds the group's
// total (N = 2, 4, 8, 16).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int N>
__device__ __forceinline__ float group_sum(float v) {
    if (N >= 2) v += dpp_f<0xB1>(v);
    if (N >= 4) v += dpp_f<0x4E>(v);
    if (N >= 8) v += dpp_f<0x141>(v);
    if (N >= 16) v += dpp_f<0x140>(v);
    return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
    if (N >= 2) v = fmaxf(v, dpp_f<0xB1>(v));
    if (N >= 4) v = fmaxf(v, dpp_f<0x4E>(v));
    if (N >= 8) v = fmaxf(v, dpp_f<0x141>(v));
    if (N >= 16) v = fmaxf(v, dpp_f<0x140>(v));
    return v;
}

// Exchanges across rows with gfx950's lane swaps: permlane16_swap of a value
// with itself gives, between its two results, the value of every lane and of
// the lane 16 away (xor 16); permlane32_swap likewise for xor 32. All lanes
// of the wave must be active.
__device__ __forceinline__ float xor16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace kvc
