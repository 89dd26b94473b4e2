// kvc_select: top-B selection under the budget.
//
// One workgroup (1024 threads) per row. Every token gets a 32-bit key that
// orders it: protected tokens (sink, recent window, table floor) get
// 0xFFFFFFFF; the others the order-preserving bit image of
// total = score + bonus[tag][group] (NaN lowest). The budget-th largest key
// tau is found by an MSB-first radix select over three digits (11, 11 and 10
// bits) with an LDS histogram per digit, which also yields `need`, the number
// of tau-valued tokens to keep. Finite totals never reach the top 11-bit
// digit (+inf maps to 0x7FC), so the first histogram's top bin counts the
// protected tokens. A final ordered pass keeps key > tau, plus the first
// `need` tokens with key == tau in index order -- the earlier position wins
// ties (PASK Appendix B.4) -- and writes their indices ascending through a
// block-wide scan. Special cases: T <= B keeps every token; if the protected
// tokens alone reach B they are all kept (floors take precedence over the
// budget, PASK §3.5) and n_kept reports the excess.
//
// Each thread handles four consecutive tokens per step (one float4 of scores
// and four tag bytes when the row is 4-aligned); histogram increments are
// aggregated per wave over equal digits, since the leading digits of a row's
// scores fall into a handful of bins.
#include "kvc_internal.h"

namespace kvc {

static constexpr int SEL_THREADS = 1024;
static constexpr int SEL_WAVES = SEL_THREADS / 64;
static constexpr int SEL_VEC = 4;  // tokens per thread per step
static constexpr uint32_t KEY_PROTECTED = 0xFFFFFFFFu;
static constexpr int SEL_BINS = 2048;

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

// Adds one to hist[digit] for every active lane, one atomic per distinct digit
// present in the wave (all lanes of the wave must call it together).
__device__ __forceinline__ void wave_hist_add(uint32_t *hist, bool active, uint32_t digit) {
    uint64_t todo = __ballot(active);
    while (todo) {
        const int first = __ffsll((unsigned long long)todo) - 1;
        const uint32_t d0 = __shfl(digit, first);
        const uint64_t same = __ballot(active && digit == d0);
        if ((threadIdx.x & 63) == first) atomicAdd(&hist[d0], (uint32_t)__popcll(same));
        todo &= ~same;
    }
}

struct SelRow {
    const float *sr;
    const uint8_t *tr;
    int64_t T;
    int n_sink, n_recent, n_tags;
    const float *s_bonus;
    const uint8_t *s_floor;

    __device__ __forceinline__ uint32_t key(int64_t j, float score, int tag) const {
        if (tag >= n_tags) tag = 0;
        if (j < n_sink || j >= T - n_recent || s_floor[tag]) return KEY_PROTECTED;
        return order_key(score + s_bonus[tag]);
    }
    // Keys of tokens base..base+3 (those >= T are reported invalid).
    template <bool VEC>
    __device__ __forceinline__ void keys4(int64_t base, uint32_t *k, bool *valid) const {
        if (VEC && base + SEL_VEC <= T) {
            const float4 s = *reinterpret_cast<const float4 *>(sr + base);
            uint32_t t4 = 0;
            if (tr) t4 = *reinterpret_cast<const uint32_t *>(tr + base);
            const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
            for (int e = 0; e < SEL_VEC; ++e) {
                k[e] = key(base + e, sv[e], (int)((t4 >> (8 * e)) & 0xFF));
                valid[e] = true;
            }
        } else {
#pragma unroll
            for (int e = 0; e < SEL_VEC; ++e) {
                const int64_t j = base + e;
                valid[e] = j < T;
                k[e] = valid[e] ? key(j, sr[j], tr ? tr[j] : 0) : 0u;
            }
        }
    }
};

template <bool VEC>
__global__ void __launch_bounds__(SEL_THREADS)
    select_kernel(const float *__restrict__ scores, const uint8_t *__restrict__ tags,
                  const float *__restrict__ bonus, const uint8_t *__restrict__ floor_tbl, int64_t T,
                  int L, int Hkv, int n_groups, int layer_base, int n_layers_model, int n_tags,
                  int n_sink, int n_recent, int B, int32_t *__restrict__ kept, int kept_stride,
                  int32_t *__restrict__ n_kept) {
    __shared__ float s_bonus[256];
    __shared__ uint8_t s_floor[256];
    __shared__ uint32_t hist[SEL_BINS];
    __shared__ uint32_t s_wave[SEL_WAVES + 1];
    __shared__ uint32_t s_pick[2];

    const int64_t r = blockIdx.x;
    const RowIdx ri = split_row(r, L, Hkv);
    const int tid = threadIdx.x;
    const int grp = device_layer_group(layer_base + ri.l, n_layers_model, n_groups);
    for (int t = tid; t < 256; t += SEL_THREADS) {
        s_bonus[t] = (bonus && t < n_tags) ? bonus[t * n_groups + grp] : 0.f;
        s_floor[t] = (floor_tbl && t < n_tags) ? floor_tbl[t * n_groups + grp] : 0;
    }
    __syncthreads();
    SelRow row{scores + (size_t)r * T, tags ? tags + (size_t)ri.n * T : nullptr, T, n_sink, n_recent, n_tags,
               s_bonus, s_floor};
    const int64_t step = (int64_t)SEL_THREADS * SEL_VEC;
    const int64_t trips = (T + step - 1) / step;

    uint32_t tau;
    int64_t need;
    if (T <= B) {
        tau = 0u;
        need = T;
    } else {
        // Radix select: digits [31:21], [20:10], [9:0].
        uint32_t prefix = 0u, k = (uint32_t)B;
        bool all_protected = false;
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
            const int width = pass == 2 ? 10 : 11;
            const uint32_t mask = (1u << width) - 1u;
            const int nbins = 1 << width;
            for (int t = tid; t < SEL_BINS; t += SEL_THREADS) hist[t] = 0u;
            __syncthreads();
            for (int64_t it = 0; it < trips; ++it) {
                uint32_t kk[SEL_VEC];
                bool valid[SEL_VEC];
                row.keys4<VEC>((it * SEL_THREADS + tid) * SEL_VEC, kk, valid);
#pragma unroll
                for (int e = 0; e < SEL_VEC; ++e) {
                    const bool active = valid[e] && (pass == 0 || (kk[e] >> (shift + width)) == prefix);
                    const uint32_t digit = (kk[e] >> shift) & mask;
                    if (pass == 0)
                        wave_hist_add(hist, active, digit);
                    else if (active)
                        atomicAdd(&hist[digit], 1u);
                }
            }
            __syncthreads();
            if (pass == 0 && hist[SEL_BINS - 1] >= (uint32_t)B) {  // protected tokens fill the budget
                all_protected = true;
                break;
            }
            // Scan the bins from the top digit down; the bin where the count
            // crosses k holds the k-th largest key.
            uint32_t v[2];
            v[0] = 2 * tid < nbins ? hist[nbins - 1 - 2 * tid] : 0u;
            v[1] = 2 * tid + 1 < nbins ? hist[nbins - 2 - 2 * tid] : 0u;
            uint32_t tot;
            const uint32_t ex = block_excl_scan(v[0] + v[1], &tot, s_wave);
            if (ex < k && k <= ex + v[0]) {
                s_pick[0] = (uint32_t)(nbins - 1 - 2 * tid);
                s_pick[1] = k - ex;
            } else if (ex + v[0] < k && k <= ex + v[0] + v[1]) {
                s_pick[0] = (uint32_t)(nbins - 2 - 2 * tid);
                s_pick[1] = k - ex - v[0];
            }
            __syncthreads();
            prefix = (prefix << width) | s_pick[0];
            k = s_pick[1];
            __syncthreads();
        }
        if (all_protected) {
            tau = KEY_PROTECTED;
            need = T;  // keep every protected token
        } else {
            tau = prefix;
            need = k;
        }
    }

    // Ordered compaction: keep key > tau, and the first `need` keys == tau.
    int64_t carry_gt = 0, carry_eq = 0;
    int32_t *kr = kept + (size_t)r * kept_stride;
    for (int64_t it = 0; it < trips; ++it) {
        const int64_t base = (it * SEL_THREADS + tid) * SEL_VEC;
        uint32_t kk[SEL_VEC];
        bool valid[SEL_VEC];
        row.keys4<VEC>(base, kk, valid);
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int e = 0; e < SEL_VEC; ++e) {
            ngt += valid[e] && kk[e] > tau;
            neq += valid[e] && kk[e] == tau;
        }
        uint32_t tot;
        const uint32_t ex = block_excl_scan(ngt | (neq << 16), &tot, s_wave);
        int64_t gt_before = carry_gt + (ex & 0xFFFFu);
        int64_t eq_before = carry_eq + (ex >> 16);
#pragma unroll
        for (int e = 0; e < SEL_VEC; ++e) {
            const bool gt = valid[e] && kk[e] > tau;
            const bool eq = valid[e] && kk[e] == tau;
            if (gt || (eq && eq_before < need)) {
                const int64_t pos = gt_before + (eq_before < need ? eq_before : need);
                if (pos < kept_stride) kr[pos] = (int32_t)(base + e);
            }
            gt_before += gt;
            eq_before += eq;
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
    // float4 score loads and 4-byte tag loads need every row start 16-byte aligned.
    const bool vec = (T % 4 == 0) && (reinterpret_cast<uintptr_t>(scores) % 16 == 0) &&
                     (!p->tags || reinterpret_cast<uintptr_t>(p->tags) % 4 == 0);
    const dim3 grid((unsigned)n_rows(dims)), block(SEL_THREADS);
    hipStream_t s = as_stream(stream);
    if (vec)
        select_kernel<true><<<grid, block, 0, s>>>(scores, p->tags, p->tag_bonus, p->tag_floor, T, dims->n_layers,
                                                    dims->n_kv_heads, p->n_groups, p->layer_base,
                                                    p->n_layers_model, p->n_tags, p->n_sink, p->n_recent,
                                                    p->budget, kept_idx, kept_stride, n_kept);
    else
        select_kernel<false><<<grid, block, 0, s>>>(scores, p->tags, p->tag_bonus, p->tag_floor, T, dims->n_layers,
                                                     dims->n_kv_heads, p->n_groups, p->layer_base,
                                                     p->n_layers_model, p->n_tags, p->n_sink, p->n_recent,
                                                     p->budget, kept_idx, kept_stride, n_kept);
    if ((st = check_launch("kvc_select")) != KVC_OK) return st;
    const int64_t sink_recent = (int64_t)p->n_sink + p->n_recent;
    if (T > p->budget && (sink_recent < T ? sink_recent : T) > p->budget) {
        fail(KVC_WARN_FLOOR_EXCESS, "kvc_select: %lld sink+recent tokens exceed the budget %d",
             (long long)sink_recent, p->budget);
        return KVC_WARN_FLOOR_EXCESS;
    }
    return KVC_OK;
}
