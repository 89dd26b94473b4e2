// kvc_select: top-B selection under the budget.
//
// One workgroup (1024 threads) per row. Every token gets a 32-bit key that
// orders it: protected tokens (sink, recent window, table floor) get
// 0xFFFFFFFF; the others the order-preserving bit image of
// total = score + bonus[tag][group] (NaN lowest). The budget-th largest key
// tau is found by an MSB-first radix select (four 8-bit digits, LDS histogram
// per digit with wave-aggregated atomics when a wave agrees on a digit), which
// also yields `need`, the number of tau-valued tokens to keep. A final ordered
// pass keeps key > tau, plus the first `need` tokens with key == tau in index
// order -- the earlier position wins ties (PASK Appendix B.4) -- and writes
// their indices ascending through a block-wide scan. Special cases: T <= B
// keeps every token; if the protected tokens alone reach B they are all kept
// (floors take precedence over the budget, PASK §3.5) and n_kept reports the
// excess.
#include "kvc_internal.h"

namespace kvc {

static constexpr int SEL_THREADS = 1024;
static constexpr int SEL_WAVES = SEL_THREADS / 64;
static constexpr uint32_t KEY_PROTECTED = 0xFFFFFFFFu;

__device__ __forceinline__ uint32_t order_key(float x) {
    if (x != x) return 0u;
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ int32_t device_layer_group(int32_t layer, int32_t n_layers, int32_t n_groups) {
    int32_t g = 0;
    for (int32_t c = 1; c < n_groups; ++c)
        if (layer >= (int32_t)(((int64_t)c * n_layers + n_groups - 1) / n_groups)) ++g;
    return g;
}

// Exclusive block scan over SEL_THREADS threads; *total receives the sum.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t *total, uint32_t *s_wave) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    if (wave == 0) {
        const uint32_t w = lane < SEL_WAVES ? s_wave[lane] : 0u;
        uint32_t c = w;
#pragma unroll
        for (int off = 1; off < SEL_WAVES; off <<= 1) {
            const uint32_t y = __shfl_up(c, off);
            if (lane >= off) c += y;
        }
        if (lane < SEL_WAVES) s_wave[lane] = c - w;
        if (lane == SEL_WAVES - 1) s_wave[SEL_WAVES] = c;
    }
    __syncthreads();
    const uint32_t res = s_wave[wave] + x - v;
    *total = s_wave[SEL_WAVES];
    __syncthreads();
    return res;
}

__global__ void __launch_bounds__(SEL_THREADS)
    select_kernel(const float *__restrict__ scores, const uint8_t *__restrict__ tags,
                  const float *__restrict__ bonus, const uint8_t *__restrict__ floor_tbl, int64_t T,
                  int L, int Hkv, int n_groups, int layer_base, int n_layers_model, int n_tags,
                  int n_sink, int n_recent, int B, int32_t *__restrict__ kept, int kept_stride,
                  int32_t *__restrict__ n_kept) {
    __shared__ float s_bonus[256];
    __shared__ uint8_t s_floor[256];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t s_wave[SEL_WAVES + 1];
    __shared__ uint32_t s_pick[2];

    const int64_t r = blockIdx.x;
    const RowIdx ri = split_row(r, L, Hkv);
    const int tid = threadIdx.x, lane = tid & 63;
    const int grp = device_layer_group(layer_base + ri.l, n_layers_model, n_groups);
    for (int t = tid; t < 256; t += SEL_THREADS) {
        s_bonus[t] = (bonus && t < n_tags) ? bonus[t * n_groups + grp] : 0.f;
        s_floor[t] = (floor_tbl && t < n_tags) ? floor_tbl[t * n_groups + grp] : 0;
    }
    __syncthreads();
    const float *sr = scores + (size_t)r * T;
    const uint8_t *tr = tags ? tags + (size_t)ri.n * T : nullptr;
    auto key_of = [&](int64_t j) -> uint32_t {
        int tg = tr ? tr[j] : 0;
        if (tg >= n_tags) tg = 0;
        if (j < n_sink || j >= T - n_recent || s_floor[tg]) return KEY_PROTECTED;
        return order_key(sr[j] + s_bonus[tg]);
    };
    const int64_t trips = (T + SEL_THREADS - 1) / SEL_THREADS;

    uint32_t tau;
    int64_t need;
    if (T <= B) {
        tau = 0u;
        need = T;
    } else {
        uint32_t cnt = 0;
        for (int64_t it = 0; it < trips; ++it) {
            const int64_t j = it * SEL_THREADS + tid;
            if (j < T && key_of(j) == KEY_PROTECTED) ++cnt;
        }
        uint32_t nprot;
        block_excl_scan(cnt, &nprot, s_wave);
        if ((int64_t)nprot >= B) {
            tau = KEY_PROTECTED;
            need = nprot;
        } else {
            uint32_t prefix = 0u;
            uint32_t k = (uint32_t)B;
            for (int pass = 0; pass < 4; ++pass) {
                const int shift = 24 - 8 * pass;
                for (int t = tid; t < 256; t += SEL_THREADS) hist[t] = 0u;
                __syncthreads();
                for (int64_t it = 0; it < trips; ++it) {
                    const int64_t j = it * SEL_THREADS + tid;
                    uint32_t key = 0u;
                    bool active = false;
                    if (j < T) {
                        key = key_of(j);
                        active = pass == 0 || (key >> (shift + 8)) == prefix;
                    }
                    const uint32_t digit = (key >> shift) & 0xFFu;
                    const uint64_t am = __ballot(active);
                    if (am) {
                        const int first = __ffsll((unsigned long long)am) - 1;
                        const uint32_t d0 = __shfl(digit, first);
                        const uint64_t same = __ballot(active && digit == d0);
                        if (same == am) {
                            if (lane == first) atomicAdd(&hist[d0], (uint32_t)__popcll(am));
                        } else if (active) {
                            atomicAdd(&hist[digit], 1u);
                        }
                    }
                }
                __syncthreads();
                // Scan the bins from the top digit down; the bin where the count
                // crosses k holds the k-th largest key.
                const uint32_t v = tid < 256 ? hist[255 - tid] : 0u;
                uint32_t tot;
                const uint32_t ex = block_excl_scan(v, &tot, s_wave);
                if (tid < 256 && ex < k && k <= ex + v) {
                    s_pick[0] = 255u - (uint32_t)tid;
                    s_pick[1] = k - ex;
                }
                __syncthreads();
                prefix = (prefix << 8) | s_pick[0];
                k = s_pick[1];
                __syncthreads();
            }
            tau = prefix;
            need = k;
        }
    }

    // Ordered compaction: keep key > tau, and the first `need` keys == tau.
    int64_t carry_gt = 0, carry_eq = 0;
    int32_t *kr = kept + (size_t)r * kept_stride;
    for (int64_t it = 0; it < trips; ++it) {
        const int64_t j = it * SEL_THREADS + tid;
        bool gt = false, eq = false;
        if (j < T) {
            const uint32_t key = key_of(j);
            gt = key > tau;
            eq = key == tau;
        }
        uint32_t tot;
        const uint32_t ex = block_excl_scan((uint32_t)gt | ((uint32_t)eq << 16), &tot, s_wave);
        const int64_t gt_before = carry_gt + (ex & 0xFFFFu);
        const int64_t eq_before = carry_eq + (ex >> 16);
        if (gt || (eq && eq_before < need)) {
            const int64_t pos = gt_before + (eq_before < need ? eq_before : need);
            if (pos < kept_stride) kr[pos] = (int32_t)j;
        }
        carry_gt += tot & 0xFFFFu;
        carry_eq += tot >> 16;
    }
    if (tid == 0) n_kept[r] = (int32_t)(carry_gt + (carry_eq < need ? carry_eq : need));
}

}  // namespace kvc

using namespace kvc;

extern "C" int kvc_select(const kvc_dims *dims, const float *scores, const kvc_policy *p,
                          int32_t *kept_idx, int32_t kept_stride, int32_t *n_kept, void *ws,
                          size_t ws_bytes, void *stream) {
    (void)ws;
    (void)ws_bytes;
    int st = check_dims(dims, "kvc_select");
    if (st != KVC_OK) return st;
    if (!scores || !p || !kept_idx || !n_kept) return fail(KVC_ERR_ARG, "kvc_select: NULL pointer");
    const int64_t T = dims->n_tokens;
    if (p->budget <= 0) return fail(KVC_ERR_ARG, "kvc_select: budget %d must be positive", p->budget);
    if (p->n_sink < 0 || p->n_recent < 0) return fail(KVC_ERR_ARG, "kvc_select: negative sink/recent");
    if (p->n_tags < 1 || p->n_tags > 256 || p->n_groups < 1 || p->n_tags * p->n_groups > 256 * 64)
        return fail(KVC_ERR_ARG, "kvc_select: table %d x %d out of range (tags 1..256)", p->n_tags,
                    p->n_groups);
    if (p->reserved != 0) return fail(KVC_ERR_ARG, "kvc_select: reserved field must be 0");
    if (p->n_layers_model <= 0 || p->layer_base < 0 || p->layer_base + dims->n_layers > p->n_layers_model)
        return fail(KVC_ERR_ARG, "kvc_select: layers [%d, %d) outside a %d-layer model", p->layer_base,
                    p->layer_base + dims->n_layers, p->n_layers_model);
    const int64_t want = T < p->budget ? T : p->budget;
    if (kept_stride < want)
        return fail(KVC_ERR_ARG, "kvc_select: kept_stride %d < min(budget, T) = %lld", kept_stride,
                    (long long)want);
    select_kernel<<<dim3((unsigned)n_rows(dims)), dim3(SEL_THREADS), 0, as_stream(stream)>>>(
        scores, p->tags, p->tag_bonus, p->tag_floor, T, dims->n_layers, dims->n_kv_heads, p->n_groups,
        p->layer_base, p->n_layers_model, p->n_tags, p->n_sink, p->n_recent, p->budget, kept_idx,
        kept_stride, n_kept);
    if ((st = check_launch("kvc_select")) != KVC_OK) return st;
    const int64_t sink_recent = (int64_t)p->n_sink + p->n_recent;
    if (T > p->budget && (sink_recent < T ? sink_recent : T) > p->budget) {
        fail(KVC_WARN_FLOOR_EXCESS, "kvc_select: %lld sink+recent tokens exceed the budget %d",
             (long long)sink_recent, p->budget);
        return KVC_WARN_FLOOR_EXCESS;
    }
    return KVC_OK;
}
