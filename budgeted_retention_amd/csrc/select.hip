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
#include <type_traits>

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

// Cross-lane moves through DPP (VALU, no LDS round trip). Lanes whose source
// falls outside the row read 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, true);
}
static constexpr int DPP_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
static constexpr int DPP_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
static constexpr int DPP_HALF_MIRROR = 0x141;
static constexpr int DPP_SHR1 = 0x111, DPP_SHR2 = 0x112, DPP_SHR4 = 0x114, DPP_SHR8 = 0x118;
static constexpr int DPP_BCAST15 = 0x142, DPP_BCAST31 = 0x143;

// Inclusive scan of x over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += dpp<DPP_SHR1>(x);
    x += dpp<DPP_SHR2>(x);
    x += dpp<DPP_SHR4>(x);
    x += dpp<DPP_SHR8>(x);
    x += dpp<DPP_BCAST15, 0xA>(x);  // row r-1's last lane into rows 1 and 3
    x += dpp<DPP_BCAST31, 0xC>(x);  // lane 31 into rows 2 and 3
    return x;
}

// Exclusive block scan over SEL_THREADS threads; *total receives the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *total, uint32_t *s_wave) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan(v);
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    if (wave == 0) {
        const uint32_t w = lane < SEL_WAVES ? s_wave[lane] : 0u;
        const uint32_t c = wave_incl_scan(w);
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
                  int tag_rows, int n_sink, int n_recent, int B, int32_t *__restrict__ kept, int kept_stride,
                  int32_t *__restrict__ n_kept, const uint32_t *__restrict__ only) {
    __shared__ float s_bonus[256];
    __shared__ uint8_t s_floor[256];
    __shared__ uint32_t hist[SEL_BINS];
    __shared__ uint32_t s_wave[SEL_WAVES + 1];
    __shared__ uint32_t s_pick[2];

    const int64_t r = blockIdx.x;
    if (only && !only[r]) return;   // a row mask: only the flagged rows
    const RowIdx ri = split_row(r, L, Hkv);
    const int tid = threadIdx.x;
    const int grp = device_layer_group(layer_base + ri.l, n_layers_model, n_groups);
    for (int t = tid; t < 256; t += SEL_THREADS) {
        s_bonus[t] = (bonus && t < n_tags) ? bonus[t * n_groups + grp] : 0.f;
        s_floor[t] = (floor_tbl && t < n_tags) ? floor_tbl[t * n_groups + grp] : 0;
    }
    __syncthreads();
    SelRow row{scores + (size_t)r * T, tags ? tags + (size_t)(tag_rows ? r : ri.n) * T : nullptr, T, n_sink,
               n_recent, n_tags, s_bonus, s_floor};
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
                if (pos < kept_stride) kr[KVC_IDX(pos, kept_stride, KVC_CHK_SELECT)] = (int32_t)(base + e);
            }
            gt_before += gt;
            eq_before += eq;
        }
        carry_gt += tot & 0xFFFFu;
        carry_eq += tot >> 16;
    }
    if (tid == 0) n_kept[r] = (int32_t)(carry_gt + (carry_eq < need ? carry_eq : need));
}

// Candidate variant for rows whose decision bitmaps fit in LDS (T a multiple
// of 4, 16-byte aligned rows). Every kept token is found among a short
// candidate list, so the row's scores are streamed once instead of once per
// radix digit:
//   S. a sample (one 128-byte line in eight) places a lower-bound top digit
//      d_lo whose tokens should number about 1.5 B;
//   F. one pass over the row: the tokens with top digit >= d_lo are counted
//      in the exact top-digit histogram and appended to an LDS candidate list;
//   R. if they are at least B and fit the list, the histogram gives the bin of
//      the budget-th key and the two low digits are resolved on the
//      candidates alone; the kept candidates get bits in two LDS bitmaps
//      ("above" tau, "equal" to tau);
//   X. otherwise (a misleading sample, many equal scores) the exact path runs:
//      a full histogram pass, the threshold bin's tokens as candidates (or
//      streaming passes when they overflow), "above" bits written for whole
//      words;
//   D. each wave scans its contiguous bitmap words and expands the non-zero
//      ones with 32 lanes per word: every "above" token and the first `need`
//      "equal" tokens in index order, ascending.
// Instances: CAP candidates, U float4 loads per thread per trip (two trips in
// flight), WPE waves per SIMD the registers must allow. With budgets up to
// 2048 and rows up to ~110,000 tokens the small instance's LDS (under 80 KB)
// and registers (64) let two workgroups share a CU, so a call of a few more
// rows than CUs runs in one round instead of two.
static constexpr int SEL_CAND = 8192;
static constexpr int SEL_CAND_SMALL = 5632;
static constexpr size_t SEL_CAND_SMALL_LDS = 80 * 1024;   // per workgroup, static LDS included

// ORs this lane's 4-bit nibble (tokens 4*lane .. 4*lane+3 of the wave's 256)
// with those of its 8-lane group; lane 8g ends with the group's 32-bit word.
__device__ __forceinline__ uint32_t group8_word(uint32_t nib, int lane) {
    uint32_t w = nib << (4 * (lane & 7));
    w |= dpp<DPP_XOR1>(w);
    w |= dpp<DPP_XOR2>(w);
    w |= dpp<DPP_HALF_MIRROR>(w);  // lane i <-> 7 - i: the other quad of the group
    return w;
}

// Finds the bin where the count of keys from the top reaches `krank` (block-wide,
// nbins <= 2*SEL_THREADS bins of hist); returns the bin and the rank within it.
__device__ __forceinline__ void pick_bin(const uint32_t *hist, int nbins, uint32_t krank, uint32_t *s_wave,
                                         uint32_t *s_pick, uint32_t &bin, uint32_t &rank) {
    const int tid = threadIdx.x;
    uint32_t cnt[2];
    cnt[0] = 2 * tid < nbins ? hist[nbins - 1 - 2 * tid] : 0u;
    cnt[1] = 2 * tid + 1 < nbins ? hist[nbins - 2 - 2 * tid] : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan(cnt[0] + cnt[1], &tot, s_wave);
    if (tid == 0) {
        s_pick[0] = 0u;  // not reached: bin 0
        s_pick[1] = krank;
    }
    __syncthreads();
    if (ex < krank && krank <= ex + cnt[0]) {
        s_pick[0] = (uint32_t)(nbins - 1 - 2 * tid);
        s_pick[1] = krank - ex;
    } else if (ex + cnt[0] < krank && krank <= ex + cnt[0] + cnt[1]) {
        s_pick[0] = (uint32_t)(nbins - 2 - 2 * tid);
        s_pick[1] = krank - ex - cnt[0];
    }
    __syncthreads();
    bin = s_pick[0];
    rank = s_pick[1];
    __syncthreads();
}

template <int CAP, int U, int WPE>
__global__ void __launch_bounds__(SEL_THREADS) __attribute__((amdgpu_waves_per_eu(WPE)))
    select_cand(const float *__restrict__ scores, const uint8_t *__restrict__ tags,
                const float *__restrict__ bonus, const uint8_t *__restrict__ floor_tbl, int64_t T, int L, int Hkv,
                int n_groups, int layer_base, int n_layers_model, int n_tags, int tag_rows, int n_sink,
                int n_recent, int B, int32_t *__restrict__ kept, int kept_stride, int32_t *__restrict__ n_kept) {
    __shared__ uint32_t hist[SEL_BINS];
    __shared__ uint32_t s_wave[SEL_WAVES + 1];
    __shared__ uint32_t s_wave2[SEL_WAVES + 1];
    __shared__ uint32_t s_pick[2];
    __shared__ uint32_t s_ncand;
    __shared__ uint32_t s_tab[256];  // per tag: all ones = protected, else the bonus's float bits
    extern __shared__ uint32_t s_dyn[];
    const int Ti = (int)T, mwords = (Ti + 31) >> 5;
    uint32_t *c_key = s_dyn;                    // [CAP]
    uint32_t *c_idx = s_dyn + CAP;         // [CAP]
    uint32_t *m_gt = s_dyn + 2 * CAP;      // [mwords] kept: above tau
    uint32_t *m_eq = m_gt + mwords;             // [mwords] tie: equal to tau

    const int64_t r = blockIdx.x;
    const RowIdx ri = split_row(r, L, Hkv);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = device_layer_group(layer_base + ri.l, n_layers_model, n_groups);
    for (int t = tid; t < 256; t += SEL_THREADS) {
        const bool fl = floor_tbl && t < n_tags && floor_tbl[t * n_groups + grp];
        const float bo = (bonus && t < n_tags) ? bonus[t * n_groups + grp] : 0.f;
        s_tab[t] = fl ? KEY_PROTECTED : __float_as_uint(bo);
    }
    for (int t = tid; t < SEL_BINS; t += SEL_THREADS) hist[t] = 0u;
    for (int t = tid; t < mwords; t += SEL_THREADS) {
        m_gt[t] = 0u;
        m_eq[t] = 0u;
    }
    if (tid == 0) s_ncand = 0u;
    __syncthreads();
    const float *sr = scores + (size_t)r * T;
    const uint8_t *tr = tags ? tags + (size_t)(tag_rows ? r : ri.n) * T : nullptr;
    const int lo_prot = n_sink, hi_prot = Ti - n_recent;
    // Keys of n groups of four tokens: all table lookups first (no branches
    // between them), then the keys.
    auto keys_of = [&](auto Nc, const float4 *sv, const uint32_t *tv, const int *base, uint32_t (*k)[SEL_VEC]) {
        constexpr int N = decltype(Nc)::value;
        uint32_t tab[N][SEL_VEC];
#pragma unroll
        for (int u = 0; u < N; ++u)
#pragma unroll
            for (int e = 0; e < SEL_VEC; ++e) {
                uint32_t tg = (tv[u] >> (8 * e)) & 0xFFu;
                tg = tg < (uint32_t)n_tags ? tg : 0u;
                tab[u][e] = s_tab[tg];
            }
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const float x[SEL_VEC] = {sv[u].x, sv[u].y, sv[u].z, sv[u].w};
#pragma unroll
            for (int e = 0; e < SEL_VEC; ++e) {
                const int j = base[u] + e;
                const bool prot = j < lo_prot || j >= hi_prot || tab[u][e] == KEY_PROTECTED;
                k[u][e] = prot ? KEY_PROTECTED : order_key(x[e] + __uint_as_float(tab[u][e]));
            }
        }
    };
    const int stride = SEL_THREADS * SEL_VEC;  // tokens per block step
    // Streams the row: fn(base[U], keys[U][4]) once per trip of U
    // 4-token groups per thread (groups with base >= T are padding); the next trip's scores and tags are loaded
    // before this trip is processed (always issued, re-reading the last group
    // past the end, so the loads in flight per wait are the same on every path).
    // Every lane of a wave runs the same number of trips (fn may use wave-wide
    // operations).
    const int trips = (Ti + U * stride - 1) / (U * stride);
    auto stream = [&](auto fn) {
        float4 sa[U], sb[U];
        uint32_t ta[U], tb[U];
        auto fetch = [&](int it, float4 (&sv)[U], uint32_t (&tv)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                int b = it * U * stride + u * stride + tid * SEL_VEC;
                if (b >= Ti) b = Ti - SEL_VEC;
                b = KVC_IDX(b, Ti - SEL_VEC + 1, KVC_CHK_SELECT);
                sv[u] = *reinterpret_cast<const float4 *>(sr + b);
                tv[u] = tr ? *reinterpret_cast<const uint32_t *>(tr + b) : 0u;
            }
        };
        auto consume = [&](int it, const float4 (&sv)[U], const uint32_t (&tv)[U]) {
            int base[U];
#pragma unroll
            for (int u = 0; u < U; ++u) base[u] = it * U * stride + u * stride + tid * SEL_VEC;
            uint32_t k[U][SEL_VEC];
            keys_of(std::integral_constant<int, U>(), sv, tv, base, k);
            fn(base, k);
        };
        fetch(0, sa, ta);
        for (int it = 0; it < trips; it += 2) {
            fetch(it + 1, sb, tb);
            consume(it, sa, ta);
            if (it + 1 >= trips) break;
            fetch(it + 2, sa, ta);
            consume(it + 1, sb, tb);
        }
    };
    // per-group view of a trip: fn(base, ok, keys[4])
    auto per_group = [&](auto fn) {
        return [=](const int *base, uint32_t (*k)[SEL_VEC]) {
#pragma unroll
            for (int u = 0; u < U; ++u) fn(base[u], base[u] < Ti, k[u]);
        };
    };
    // Appends a trip's flagged tokens (bit 4u+e of cmask) to the candidate
    // list: a wave prefix sum over the lanes' counts and one LDS atomic per wave.
    auto append = [&](const int *base, uint32_t cmask, uint32_t (*k)[SEL_VEC]) {
        const uint32_t n = (uint32_t)__popc(cmask);
        const uint64_t any = __ballot(n != 0u);
        if (!any) return;
        const uint32_t incl = wave_incl_scan(n);
        uint32_t slot0 = 0;
        if (lane == 63) slot0 = atomicAdd(&s_ncand, incl);
        slot0 = __builtin_amdgcn_readlane(slot0, 63);
        uint32_t slot = slot0 + incl - n;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < SEL_VEC; ++e)
                if ((cmask >> (SEL_VEC * u + e)) & 1u) {
                    if (slot < CAP) {
                        c_key[slot] = k[u][e];
                        c_idx[slot] = (uint32_t)(base[u] + e);
                    }
                    ++slot;
                }
    };
    // Resolves digits [20:10] and [9:0] below the top digit pick0 and returns
    // tau and the number of tau-valued tokens to keep; over the candidates, or
    // over the stream when they overflowed.
    auto low_digits = [&](uint32_t pick0, uint32_t krank, bool from_cands, uint32_t ncand, uint32_t &tau_out,
                          int &need_out) {
        uint32_t prefix = pick0;
        for (int pass = 1; pass < 3; ++pass) {
            const int shift = pass == 1 ? 10 : 0;
            const int width = pass == 1 ? 11 : 10;
            const uint32_t mask = (1u << width) - 1u;
            for (int t = tid; t < SEL_BINS; t += SEL_THREADS) hist[t] = 0u;
            __syncthreads();
            if (from_cands) {
                for (uint32_t c = tid; c < ncand; c += SEL_THREADS) {
                    const uint32_t kv = c_key[c];
                    if ((kv >> (shift + width)) == prefix) atomicAdd(&hist[(kv >> shift) & mask], 1u);
                }
            } else {
                stream(per_group([&](int, bool ok, const uint32_t *k) {
#pragma unroll
                    for (int e = 0; e < SEL_VEC; ++e)
                        if (ok && (k[e] >> (shift + width)) == prefix) atomicAdd(&hist[(k[e] >> shift) & mask], 1u);
                }));
            }
            __syncthreads();
            uint32_t bin;
            pick_bin(hist, 1 << width, krank, s_wave, s_pick, bin, krank);
            prefix = (prefix << width) | bin;
        }
        tau_out = prefix;
        need_out = (int)krank;
    };

    uint32_t tau = 0u;
    int need = Ti;
    if (T <= B) {
        // every token is kept
        for (int w = tid; w < mwords; w += SEL_THREADS) {
            const int left = Ti - 32 * w;
            m_gt[w] = left >= 32 ? 0xFFFFFFFFu : ((1u << left) - 1u);
        }
        __syncthreads();
    } else {
        // S: sample one 128-byte line (32 tokens) in eight into the histogram
        bool fast = false;
        uint32_t d_lo = 0u;
        {
            const int lines = (Ti + 255) / 256;  // sampled lines start at 256*i
            for (int g0 = 0; g0 < lines * 8; g0 += U * SEL_THREADS) {
                float4 sv[U];
                uint32_t tv[U];
                int base[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int g = g0 + u * SEL_THREADS + tid;
                    base[u] = (g >> 3) * 256 + (g & 7) * SEL_VEC;
                    const int b = KVC_IDX(base[u] < Ti ? base[u] : Ti - SEL_VEC, Ti - SEL_VEC + 1, KVC_CHK_SELECT);
                    sv[u] = *reinterpret_cast<const float4 *>(sr + b);
                    tv[u] = tr ? *reinterpret_cast<const uint32_t *>(tr + b) : 0u;
                }
                uint32_t k[U][SEL_VEC];
                keys_of(std::integral_constant<int, U>(), sv, tv, base, k);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (base[u] >= Ti) continue;
                    uint32_t c0 = 1;
#pragma unroll
                    for (int e = 1; e < SEL_VEC; ++e) c0 += (k[u][e] >> 21) == (k[u][0] >> 21);
                    atomicAdd(&hist[k[u][0] >> 21], c0);
#pragma unroll
                    for (int e = 1; e < SEL_VEC; ++e)
                        if ((k[u][e] >> 21) != (k[u][0] >> 21)) atomicAdd(&hist[k[u][e] >> 21], 1u);
                }
            }
            __syncthreads();
            // aim at about 1.5 B tokens at or above d_lo (the sample holds one in eight)
            const uint32_t target = (uint32_t)((3 * (int64_t)B + 15) / 16) + 8;
            uint32_t rank;
            pick_bin(hist, SEL_BINS, target, s_wave, s_pick, d_lo, rank);
            for (int t = tid; t < SEL_BINS; t += SEL_THREADS) hist[t] = 0u;
            __syncthreads();
        }
        // F: exact histogram of the tokens at or above d_lo, appended as candidates
        stream([&](const int *base, uint32_t (*k)[SEL_VEC]) {
            uint32_t cmask = 0;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < SEL_VEC; ++e) {
                    const uint32_t d = k[u][e] >> 21;
                    if (base[u] < Ti && d >= d_lo) {
                        atomicAdd(&hist[d], 1u);
                        cmask |= 1u << (SEL_VEC * u + e);
                    }
                }
            append(base, cmask, k);
        });
        __syncthreads();
        const uint32_t ncand = s_ncand;
        fast = ncand >= (uint32_t)B && ncand <= (uint32_t)CAP;
        if (fast) {
            // R: every kept token is a candidate
            const bool all_protected = hist[SEL_BINS - 1] >= (uint32_t)B;
            uint32_t pick0 = 0u, krank = (uint32_t)B;
            if (all_protected) {
                tau = KEY_PROTECTED;
            } else {
                pick_bin(hist, SEL_BINS, (uint32_t)B, s_wave, s_pick, pick0, krank);
                low_digits(pick0, krank, true, ncand, tau, need);
            }
            for (uint32_t c = tid; c < ncand; c += SEL_THREADS) {
                const uint32_t kv = c_key[c], j = c_idx[c];
                if (all_protected) {
                    if (kv == KEY_PROTECTED) atomicOr(&m_gt[j >> 5], 1u << (j & 31));
                } else if (kv > tau) {
                    atomicOr(&m_gt[j >> 5], 1u << (j & 31));
                } else if (kv == tau) {
                    atomicOr(&m_eq[j >> 5], 1u << (j & 31));
                }
            }
            __syncthreads();
        } else {
            // X: the exact path over the whole row
            for (int t = tid; t < SEL_BINS; t += SEL_THREADS) hist[t] = 0u;
            if (tid == 0) s_ncand = 0u;
            __syncthreads();
            stream(per_group([&](int, bool ok, const uint32_t *k) {
                if (!ok) return;
                uint32_t d[SEL_VEC];
#pragma unroll
                for (int e = 0; e < SEL_VEC; ++e) d[e] = k[e] >> 21;
                uint32_t c0 = 1;
#pragma unroll
                for (int e = 1; e < SEL_VEC; ++e) c0 += d[e] == d[0];
                atomicAdd(&hist[d[0]], c0);
#pragma unroll
                for (int e = 1; e < SEL_VEC; ++e)
                    if (d[e] != d[0]) atomicAdd(&hist[d[e]], 1u);
            }));
            __syncthreads();
            const bool all_protected = hist[SEL_BINS - 1] >= (uint32_t)B;
            uint32_t pick0 = 0u, krank = (uint32_t)B;
            if (!all_protected) pick_bin(hist, SEL_BINS, (uint32_t)B, s_wave, s_pick, pick0, krank);
            // "above" bits for whole words, the threshold bin's tokens as candidates
            stream([&](const int *base, uint32_t (*k)[SEL_VEC]) {
                uint32_t cmask = 0;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const bool ok = base[u] < Ti;
                    uint32_t nib = 0;
                    if (ok) {
#pragma unroll
                        for (int e = 0; e < SEL_VEC; ++e) {
                            bool f;
                            if (all_protected)
                                f = k[u][e] == KEY_PROTECTED;
                            else {
                                const uint32_t d0 = k[u][e] >> 21;
                                f = d0 > pick0;
                                cmask |= (uint32_t)(d0 == pick0) << (SEL_VEC * u + e);
                            }
                            nib |= (uint32_t)f << e;
                        }
                    }
                    // the wave's 256 tokens of group u are 8 consecutive words; past T nothing is written
                    const uint32_t w = group8_word(nib, lane);
                    if ((lane & 7) == 0 && ok) m_gt[base[u] >> 5] = w;
                }
                append(base, cmask, k);
            });
            __syncthreads();
            if (all_protected) {
                tau = KEY_PROTECTED;
            } else {
                const uint32_t nc = s_ncand;
                const bool fits = nc <= (uint32_t)CAP;
                low_digits(pick0, krank, fits, nc, tau, need);
                if (fits) {
                    for (uint32_t c = tid; c < nc; c += SEL_THREADS) {
                        const uint32_t kv = c_key[c], j = c_idx[c];
                        if (kv > tau) atomicOr(&m_gt[j >> 5], 1u << (j & 31));
                        else if (kv == tau) atomicOr(&m_eq[j >> 5], 1u << (j & 31));
                    }
                } else {
                    stream(per_group([&](int base, bool ok, const uint32_t *k) {
                        // an opaque base keeps the compiler from hoisting every
                        // group's bitmap addresses out of the stream (registers)
                        asm volatile("" : "+v"(base));
#pragma unroll
                        for (int e = 0; e < SEL_VEC; ++e) {
                            const int j = base + e;
                            if (ok && (k[e] >> 21) == pick0) {
                                if (k[e] > tau) atomicOr(&m_gt[j >> 5], 1u << (j & 31));
                                else if (k[e] == tau) atomicOr(&m_eq[j >> 5], 1u << (j & 31));
                            }
                        }
                    }));
                }
            }
            __syncthreads();
        }
    }

    // D: wave w owns the contiguous words [w*WPW, (w+1)*WPW), taken 64 at a time
    const int WPW = (mwords + SEL_WAVES - 1) / SEL_WAVES;
    const int wbeg = wave * WPW, wend = wbeg + WPW < mwords ? wbeg + WPW : mwords;
    const int rounds = (WPW + 63) / 64;
    uint32_t cg = 0, ce = 0;
    for (int rr = 0; rr < rounds; ++rr) {
        const int w = wbeg + rr * 64 + lane;
        if (w < wend) {
            cg += __popc(m_gt[w]);
            ce += __popc(m_eq[w]);
        }
    }
    const uint32_t wsum_g = __builtin_amdgcn_readlane(wave_incl_scan(cg), 63);
    const uint32_t wsum_e = __builtin_amdgcn_readlane(wave_incl_scan(ce), 63);
    if (lane == 0) {
        s_wave[wave] = wsum_g;
        s_wave2[wave] = wsum_e;
    }
    __syncthreads();
    uint32_t base_g = 0, base_e = 0, tot_g = 0, tot_e = 0;
    for (int v = 0; v < SEL_WAVES; ++v) {
        if (v < wave) {
            base_g += s_wave[v];
            base_e += s_wave2[v];
        }
        tot_g += s_wave[v];
        tot_e += s_wave2[v];
    }
    int32_t *kr = kept + (size_t)r * kept_stride;
    for (int rr = 0; rr < rounds; ++rr) {
        const int w = wbeg + rr * 64 + lane;
        const uint32_t g = w < wend ? m_gt[w] : 0u, q = w < wend ? m_eq[w] : 0u;
        const uint32_t ig = wave_incl_scan((uint32_t)__popc(g)), ie = wave_incl_scan((uint32_t)__popc(q));
        const uint32_t gb = base_g + ig - __popc(g), eb = base_e + ie - __popc(q);  // before this word
        uint64_t live = __ballot((g | q) != 0u);
        while (live) {
            const int src = __ffsll((unsigned long long)live) - 1;
            live &= live - 1ull;
            const uint32_t G = __builtin_amdgcn_readlane(g, src), E = __builtin_amdgcn_readlane(q, src);
            const int GB = (int)__builtin_amdgcn_readlane(gb, src), EB = (int)__builtin_amdgcn_readlane(eb, src);
            const int W = __builtin_amdgcn_readlane(w, src);
            if (lane < 32) {
                const uint32_t bit = 1u << lane, below = bit - 1u;
                const int gpos = GB + __popc(G & below), erank = EB + __popc(E & below);
                if (G & bit) {
                    const int pos = gpos + (erank < need ? erank : need);
                    if (pos < kept_stride) kr[KVC_IDX(pos, kept_stride, KVC_CHK_SELECT)] = 32 * W + lane;
                } else if ((E & bit) && erank < need) {
                    const int pos = gpos + erank;
                    if (pos < kept_stride) kr[KVC_IDX(pos, kept_stride, KVC_CHK_SELECT)] = 32 * W + lane;
                }
            }
        }
        base_g += __builtin_amdgcn_readlane(ig, 63);
        base_e += __builtin_amdgcn_readlane(ie, 63);
    }
    if (tid == 0) n_kept[r] = (int32_t)(tot_g + (tot_e < (uint32_t)need ? tot_e : (uint32_t)need));
}


// ---------------------------------------------------------------- long rows
//
// Rows too long for one workgroup (a million-token session compacts a few
// rows per call) are split into chunks of SPLIT_CHUNK tokens, each its own
// workgroup. The same three radix digits are resolved in turn: every chunk
// adds its digit histogram into the row's histogram in the workspace, and one
// workgroup per row picks the bin where the budget-th key lies. With tau and
// `need` fixed, every chunk counts its keys above and equal to tau, one
// workgroup per row turns the counts into each chunk's first output slot and
// first tie rank, and every chunk writes its kept indices in index order.
// The decisions are those of the one-workgroup kernels (same keys, ties to the
// lower index, floors before the budget).
static constexpr int SPLIT_CHUNK = SEL_THREADS * SEL_VEC * 4;   // 16384 tokens per workgroup

struct SplitState {
    uint32_t prefix;   // digits resolved so far; after the last pick: tau
    uint32_t k;        // rank of the budget-th key among keys with that prefix
    uint32_t done;     // 1: tau/need final (every token, or every protected one)
    uint32_t pad;
    int64_t need;      // tau-valued tokens to keep (lowest indices first)
};

struct SplitWs {
    uint32_t *hist;      // [rows][3][SEL_BINS]
    SplitState *state;   // [rows]
    uint32_t *cnt;       // [rows][chunks][2]  keys above / equal to tau
    int64_t *base;       // [rows][chunks][2]  first output slot, tau-valued tokens before the chunk
};

static size_t align256s(size_t x) { return (x + 255) & ~(size_t)255; }

// Short rows (T <= 8192): one wave per row, four rows per workgroup, no
// workgroup barriers. Lane l holds the keys of tokens 256k + 4l .. 256k + 4l + 3
// (k < NPL4) in registers; the budget-th key is found with the same three
// radix digits (11, 11, 10 bits) over the wave's own LDS histogram, the
// crossing bin by a wave scan of per-lane bin sums; the ordered write walks
// the 256-token blocks in order with wave scans of the per-lane counts.
// Each tag's bonus and floor are one 32-bit table entry: the bonus, or the
// bit pattern SW_FLOOR for a floored tag (a NaN bonus is stored as the
// canonical NaN, so it still ranks lowest).
static constexpr int SW_WAVES = 4;
static constexpr uint32_t SW_FLOOR = 0x7FFFFFFFu;

// A wave's LDS operations execute in issue order; this keeps the compiler from
// moving LDS accesses of one lane across accesses of the other lanes.
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t sw_key(int j, float score, float bt, int lo, uint32_t span) {
    if ((uint32_t)(j - lo) >= span || __float_as_uint(bt) == SW_FLOOR) return KEY_PROTECTED;
    return order_key(score + bt);
}

// Rows that are not float4-aligned load their keys one by one, which takes a
// few more registers: their instances allow one wave fewer per SIMD rather
// than spill (a kernel with scratch pays for it at every launch).
template <int NPL4, bool VEC>
__global__ void __launch_bounds__(SW_WAVES * 64) __attribute__((amdgpu_waves_per_eu(NPL4 <= 16 ? (VEC ? 4 : 3) : (VEC ? 2 : 1))))
    select_wave(const float *__restrict__ scores, const uint8_t *__restrict__ tags,
                const float *__restrict__ bonus, const uint8_t *__restrict__ floor_tbl, int Ti, int64_t rows,
                int L, int Hkv, int n_groups, int layer_base, int n_layers_model, int n_tags, int tag_rows,
                int n_sink, int n_recent, int B, int32_t *__restrict__ kept, int kept_stride,
                int32_t *__restrict__ n_kept) {
    __shared__ __align__(16) uint32_t s_hist[SW_WAVES][SEL_BINS];
    __shared__ float s_tab[SW_WAVES][256];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: row pointers stay scalar
    const int64_t r = (int64_t)blockIdx.x * SW_WAVES + wave;
    if (r >= rows) return;
    const RowIdx ri = split_row(r, L, Hkv);
    const int grp = device_layer_group(layer_base + ri.l, n_layers_model, n_groups);
    float *tab = s_tab[wave];
    uint32_t *hist = s_hist[wave];
    for (int t = lane; t < 256; t += 64) {
        const int u = t < n_tags ? t : 0;   // tags beyond the table read tag 0
        float b = 0.f;
        if (u < n_tags) {
            b = bonus ? bonus[u * n_groups + grp] : 0.f;
            if (b != b) b = __uint_as_float(0x7FC00000u);
            if (floor_tbl && floor_tbl[u * n_groups + grp]) b = __uint_as_float(SW_FLOOR);
        }
        tab[t] = b;
    }
    wave_lds_order();
    const float *sr = scores + (size_t)r * Ti;
    const uint8_t *tr = tags ? tags + (size_t)(tag_rows ? r : ri.n) * Ti : nullptr;
    const int lo = n_sink;
    const int hi = Ti - n_recent;
    const uint32_t span = hi > lo ? (uint32_t)(hi - lo) : 0u;
    const float b0 = tab[0];

    // All loads first (score bits into key[][], four tags per word), then the
    // keys in place. Tokens past T get key 0 (the key of a NaN total): they
    // sit after every real token in index order, so the ordered write never
    // reaches them, and `pads` of them are taken out of histogram bin 0.
    uint32_t key[NPL4][SEL_VEC], tg[NPL4];
#pragma unroll
    for (int k = 0; k < NPL4; ++k) {
        const int base = k * 256 + 4 * lane;
        if (VEC && base + SEL_VEC <= Ti) {
            const uint4 sv = *reinterpret_cast<const uint4 *>(sr + base);
            key[k][0] = sv.x;
            key[k][1] = sv.y;
            key[k][2] = sv.z;
            key[k][3] = sv.w;
            tg[k] = tr ? *reinterpret_cast<const uint32_t *>(tr + base) : 0u;
        } else {
            tg[k] = 0u;
#pragma unroll
            for (int e = 0; e < SEL_VEC; ++e) {
                const int j = base + e;
                key[k][e] = j < Ti ? __float_as_uint(sr[j]) : 0u;
                if (tr && j < Ti) tg[k] |= (uint32_t)tr[j] << (8 * e);
            }
        }
    }
    // Protected tokens are kept whatever the budget; the histograms rank only
    // the others ("real" tokens) by d = key - kmin, so that the first digit's
    // 2048 bins span the range of real keys actually present (score totals sit
    // within a few octaves, and a fixed top digit would put most of them in a
    // handful of bins). kmax1 tracks max(key + 1): a protected key wraps to 0.
    const bool b0_floor = __float_as_uint(b0) == SW_FLOOR;
    auto inner = [&](int k) { return k * 256 >= lo && k * 256 + 256 <= hi; };
    auto plain = [&](int k) { return inner(k) && !tr && !b0_floor; };
    uint32_t nprot = 0u, kmin = 0xFFFFFFFFu, kmax1 = 0u;
#pragma unroll
    for (int k = 0; k < NPL4; ++k) {
        if (plain(k)) {
#pragma unroll
            for (int e = 0; e < SEL_VEC; ++e) {
                const uint32_t kk = order_key(__uint_as_float(key[k][e]) + b0);
                key[k][e] = kk;
                kmin = min(kmin, kk);
                kmax1 = max(kmax1, kk + 1u);
            }
        } else if (inner(k) && !tr) {   // a floored tag 0 protects every token
#pragma unroll
            for (int e = 0; e < SEL_VEC; ++e) key[k][e] = KEY_PROTECTED;
            nprot += SEL_VEC;
        } else {
#pragma unroll
            for (int e = 0; e < SEL_VEC; ++e) {
                const int j = k * 256 + 4 * lane + e;
                const float bt = tr ? tab[(tg[k] >> (8 * e)) & 0xFF] : b0;
                const uint32_t kk = j < Ti ? sw_key(j, __uint_as_float(key[k][e]), bt, lo, span) : 0u;
                key[k][e] = kk;
                nprot += (j < Ti && kk == KEY_PROTECTED) ? 1u : 0u;
                kmin = min(kmin, j < Ti ? kk : 0xFFFFFFFFu);
                kmax1 = max(kmax1, j < Ti ? kk + 1u : 0u);
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the live range to one block of keys
    }
    const uint32_t pads = (uint32_t)(NPL4 * 256 - Ti);

    uint32_t tau = 0u;
    int need;
    if (Ti <= B) {
        // keep every real token: all keys above 0, and the real tokens with key 0
        uint32_t zeros = 0u;
#pragma unroll
        for (int k = 0; k < NPL4; ++k)
#pragma unroll
            for (int e = 0; e < SEL_VEC; ++e) zeros += (uint32_t)__popcll(__ballot(key[k][e] == 0u));
        need = (int)(zeros - pads);
    } else {
        nprot = __builtin_amdgcn_readlane(wave_incl_scan(nprot), 63);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
            kmax1 = max(kmax1, (uint32_t)__shfl_xor((int)kmax1, o));
        }
        if (nprot >= (uint32_t)B) {   // protected tokens fill the budget: keep them all
            tau = KEY_PROTECTED;
            need = Ti;
        } else {
            uint4 *h4 = reinterpret_cast<uint4 *>(hist);
            auto clear = [&]() {
#pragma unroll
                for (int t = 0; t < SEL_BINS / 256; ++t) h4[t * 64 + lane] = make_uint4(0u, 0u, 0u, 0u);
                wave_lds_order();
            };
            // In the order from the top bin down, lane l owns the `per` bins
            // l*per .. l*per + per - 1 (read four at a time, starting at a
            // lane-rotated offset to spread the reads over the banks); the
            // first lane whose running count reaches kr holds the wanted key,
            // and its bins are then resolved one per lane.
            auto pick = [&](int nbins, uint32_t kr, uint32_t &bin, uint32_t &rank) {
                const int per = nbins / 64;
                const uint4 *mine = reinterpret_cast<const uint4 *>(hist + nbins - (lane + 1) * per);
                uint32_t sum = 0u;
                for (int q = 0; q < per / 4; ++q) {
                    const uint4 v = mine[(q + lane) & (per / 4 - 1)];
                    sum += v.x + v.y + v.z + v.w;
                }
                const uint32_t incl = wave_incl_scan(sum);
                const int src = __ffsll((unsigned long long)__ballot(incl >= kr)) - 1;
                const uint32_t before = __shfl(incl - sum, src);
                const uint32_t c = lane < per ? hist[nbins - 1 - src * per - lane] : 0u;
                const uint32_t incl2 = before + wave_incl_scan(c);
                const int at = __ffsll((unsigned long long)__ballot(incl2 >= kr)) - 1;
                bin = (uint32_t)(nbins - 1 - src * per - at);
                rank = kr - __shfl(incl2 - c, at);
                wave_lds_order();
            };
            // adds one to hist[digit(d)] for every real key with match(d)
            auto count = [&](auto match, auto digit) {
                clear();
#pragma unroll
                for (int k = 0; k < NPL4; ++k) {
                    if (plain(k)) {
#pragma unroll
                        for (int e = 0; e < SEL_VEC; ++e) {
                            const uint32_t d = key[k][e] - kmin;
                            if (match(d)) atomicAdd(&hist[digit(d)], 1u);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < SEL_VEC; ++e) {
                            const uint32_t d = key[k][e] - kmin;
                            const bool real = key[k][e] != KEY_PROTECTED && k * 256 + 4 * lane + e < Ti;
                            if (real && match(d)) atomicAdd(&hist[digit(d)], 1u);
                        }
                    }
                }
                wave_lds_order();
            };
            const uint32_t range = kmax1 - 1u - kmin;
            const int bl = range ? 32 - __clz(range) : 0;   // bits of d
            const int s0 = bl > 11 ? bl - 11 : 0;           // first digit: d >> s0 (< 2048)
            const int w1 = s0 < 11 ? s0 : 11, s1 = s0 - w1;  // then bits [s0-1 : s1], then [s1-1 : 0]
            uint32_t kr = (uint32_t)B - nprot;
            uint32_t dt;
            count([](uint32_t) { return true; }, [&](uint32_t d) { return d >> s0; });
            pick(SEL_BINS, kr, dt, kr);
            const uint32_t nbin = hist[dt];   // real keys in the top digit's bin
            if (w1 && nbin <= 64u) {
                // At most one of the bin's keys per lane: gather them into
                // hist[0..nbin) and take the kr-th largest directly (lane l
                // counts the keys above and at its own), instead of two more
                // histogram passes over the row.
                wave_lds_order();
                if (lane == 0) hist[64] = 0u;
                wave_lds_order();
#pragma unroll
                for (int k = 0; k < NPL4; ++k)
#pragma unroll
                    for (int e = 0; e < SEL_VEC; ++e) {
                        const uint32_t kk = key[k][e];
                        const bool real = plain(k) || (kk != KEY_PROTECTED && k * 256 + 4 * lane + e < Ti);
                        if (real && ((kk - kmin) >> s0) == dt) hist[atomicAdd(&hist[64], 1u)] = kk;
                    }
                wave_lds_order();
                const uint32_t x = (uint32_t)lane < nbin ? hist[lane] : 0u;
                uint32_t gt = 0u, ge = 0u;
                for (uint32_t j = 0; j < nbin; ++j) {
                    const uint32_t y = hist[j];
                    gt += y > x ? 1u : 0u;
                    ge += y >= x ? 1u : 0u;
                }
                const uint64_t hit = __ballot((uint32_t)lane < nbin && gt < kr && kr <= ge);
                const int at = __ffsll((unsigned long long)hit) - 1;
                tau = __builtin_amdgcn_readlane(x, at);
                need = (int)(kr - __builtin_amdgcn_readlane(gt, at));
                wave_lds_order();
            } else {
                if (w1) {
                    count([&](uint32_t d) { return (d >> s0) == dt; },
                          [&](uint32_t d) { return (d >> s1) & ((1u << w1) - 1u); });
                    uint32_t b1;
                    pick(w1 >= 8 ? 1 << w1 : 256, kr, b1, kr);
                    dt = (dt << w1) | b1;
                }
                if (s1) {
                    count([&](uint32_t d) { return (d >> s1) == dt; },
                          [&](uint32_t d) { return d & ((1u << s1) - 1u); });
                    uint32_t b2;
                    pick(s1 >= 8 ? 1 << s1 : 256, kr, b2, kr);
                    dt = (dt << s1) | b2;
                }
                tau = kmin + dt;
                need = (int)kr;
            }
        }
    }
    // ordered write: key > tau, and the first `need` keys == tau by index
    int32_t *out = kept + (size_t)r * kept_stride;
    // stores through a buffer resource: the row base stays scalar, a store
    // takes a 32-bit byte offset (no 64-bit address arithmetic per token)
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        out, (short)0, (kept_stride < (1 << 20) ? kept_stride : (1 << 20)) * 4, 0x00020000);
    auto put = [&](int pos, int j) {
        if (pos < kept_stride) __builtin_amdgcn_raw_buffer_store_b32(j, orsrc, pos * 4, 0, 0);
    };
    int gt_run = 0, eq_run = 0;
    int lane4 = 4 * lane;
    asm volatile("" : "+v"(lane4));   // token indices are recomputed here, not kept live from the loads
#pragma unroll
    for (int k = 0; k < NPL4; ++k) {
        const int base = k * 256 + lane4;
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int e = 0; e < SEL_VEC; ++e) {
            ngt += key[k][e] > tau;
            neq += key[k][e] == tau;
        }
        if (__ballot(neq != 0u) == 0ull) {
            // no key of this block equals tau: keep exactly the keys above it
            const uint32_t incl = wave_incl_scan(ngt);
            const int tot = (int)__builtin_amdgcn_readlane(incl, 63);
            int pos = gt_run + (eq_run < need ? eq_run : need) + (int)(incl - ngt);
#pragma unroll
            for (int e = 0; e < SEL_VEC; ++e)
                if (key[k][e] > tau) {
                    put(pos, base + e);
                    ++pos;
                }
            gt_run += tot;
        } else {
            const uint32_t packed = ngt | (neq << 16);
            const uint32_t incl = wave_incl_scan(packed);
            const uint32_t tot = __builtin_amdgcn_readlane(incl, 63);
            int gt_before = gt_run + (int)((incl - packed) & 0xFFFFu);
            int eq_before = eq_run + (int)((incl - packed) >> 16);
#pragma unroll
            for (int e = 0; e < SEL_VEC; ++e) {
                const bool gt = key[k][e] > tau;
                const bool eq = key[k][e] == tau;
                if (gt || (eq && eq_before < need)) put(gt_before + (eq_before < need ? eq_before : need), base + e);
                gt_before += gt;
                eq_before += eq;
            }
            gt_run += (int)(tot & 0xFFFFu);
            eq_run += (int)(tot >> 16);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (lane == 0) n_kept[r] = gt_run + (eq_run < need ? eq_run : need);
}

// ---------------------------------------------------------------- sampled threshold
//
// Rows of more than 8192 tokens, when the protected tokens (sinks and recent
// window; no floor table) fit in the budget and B <= min(2048, T/5):
//   cand_sample   one wave per row draws 8192 keys (2048 evenly spaced groups
//                 of four tokens) and takes the r_s-th largest, r_s chosen so
//                 that about 2.5 B of the row's keys should be at or above it:
//                 that key is the row's threshold k_lo;
//   cand_filter   segments of 16384 tokens, one 1024-thread workgroup each,
//                 append every token whose key is at least k_lo, with its
//                 key, in index order to the segment's own region of the
//                 workspace, and count them;
//   cand_resolve  one workgroup per row gathers the segments' candidates in
//                 order (if there are at least B and at most CAND_CAP of them;
//                 every kept token is then a candidate, since the row's top B
//                 are all at or above its B-th key, which is at least k_lo),
//                 finds the budget-th key among them and writes the kept
//                 indices in order; otherwise it flags the row, and the exact
//                 one-workgroup kernel then runs for the flagged rows only.
// The decisions are those of the other kernels: same keys, ties to the lower
// index.
static constexpr int CS_SAMPLE_GROUPS = 2048;            // 8192 sampled keys per row
static constexpr int CF_THREADS = 1024;
static constexpr int CF_SEG = CF_THREADS * 4 * 4;        // 16384 tokens per filter workgroup
static constexpr int CR_THREADS = 512;
static constexpr int CAND_CAP = 8192;

template <int WAVES>
__device__ __forceinline__ uint32_t blk_excl_scan(uint32_t v, uint32_t &total, uint32_t *s_w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_scan(v);
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    uint32_t before = 0u, tot = 0u;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        const uint32_t x = s_w[w];
        before += w < wave ? x : 0u;
        tot += x;
    }
    __syncthreads();
    total = tot;
    return before + incl - v;
}

struct CandArgs {
    const float *scores;
    const uint8_t *tags;
    const float *bonus;
    int64_t T, rows;
    int L, Hkv, n_groups, layer_base, n_layers_model, n_tags, tag_rows, n_sink, n_recent, B, nseg;
    uint32_t *k_lo;     // [rows]
    uint32_t *flag;     // [rows] 1 = resolve by the exact kernel
    uint32_t *cnt;      // [rows][nseg]
    uint32_t *c_key;    // [rows][T]: segment s's candidates from s*CF_SEG
    int32_t *c_idx;
    int32_t *kept;
    int kept_stride;
    int32_t *n_kept;
};

// The row's bonus per tag (tags beyond the table read tag 0), into tab[256].
__device__ __forceinline__ void cand_table(const CandArgs &a, int64_t r, float *tab, int tid, int nthreads) {
    const RowIdx ri = split_row(r, a.L, a.Hkv);
    const int grp = device_layer_group(a.layer_base + ri.l, a.n_layers_model, a.n_groups);
    for (int t = tid; t < 256; t += nthreads) {
        const int u = t < a.n_tags ? t : 0;
        tab[t] = (a.bonus && u < a.n_tags) ? a.bonus[u * a.n_groups + grp] : 0.f;
    }
}

__device__ __forceinline__ uint32_t cand_key_of(int64_t j, float x, float bt, int64_t lo, int64_t hi) {
    return (j < lo || j >= hi) ? KEY_PROTECTED : order_key(x + bt);
}

// hist[digit] += 1 for every active lane; the lanes that share the first
// active lane's digit add together (one atomic instead of a same-address
// conflict), which is where skewed totals put most of them.
__device__ __forceinline__ void hist_add_agg(uint32_t *hist, bool active, uint32_t digit) {
    const uint64_t act = __ballot(active);
    if (!act) return;
    const int first = __ffsll((unsigned long long)act) - 1;
    const uint32_t d0 = __builtin_amdgcn_readlane(digit, first);
    const uint64_t same = __ballot(active && digit == d0);
    if ((int)(threadIdx.x & 63) == first) atomicAdd(&hist[d0], (uint32_t)__popcll(same));
    if (active && digit != d0) atomicAdd(&hist[digit], 1u);
}

// Block-level radix pick helpers of the sampled-threshold kernels (one shared
// LDS histogram; thread t owns the bins t*PER .. t*PER + PER - 1 from the top).
template <int THREADS>
struct BlkRadix {
    static constexpr int WAVES = THREADS / 64, PER = SEL_BINS / THREADS;
    uint32_t *hist, *s_w, *s_pick;
    __device__ void clear() {
        for (int t = threadIdx.x; t < SEL_BINS; t += THREADS) hist[t] = 0u;
        __syncthreads();
    }
    __device__ void pick(uint32_t kr, uint32_t &bin, uint32_t &rank) {
        const int tid = threadIdx.x;
        uint32_t c[PER], sum = 0u;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            c[i] = hist[SEL_BINS - 1 - tid * PER - i];
            sum += c[i];
        }
        uint32_t tot;
        const uint32_t ex = blk_excl_scan<WAVES>(sum, tot, s_w);
        if (ex < kr && kr <= ex + sum) {
            uint32_t acc = ex;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                if (acc < kr && kr <= acc + c[i]) {
                    s_pick[0] = (uint32_t)(SEL_BINS - 1 - tid * PER - i);
                    s_pick[1] = kr - acc;
                }
                acc += c[i];
            }
        }
        __syncthreads();
        bin = s_pick[0];
        rank = s_pick[1];
        __syncthreads();
    }
};

static constexpr int CS_THREADS = 256;

__global__ void __launch_bounds__(CS_THREADS) cand_sample(CandArgs a) {
    constexpr int NG = CS_SAMPLE_GROUPS / CS_THREADS;   // 8 groups of four per thread
    constexpr int WAVES = CS_THREADS / 64;
    __shared__ __align__(16) uint32_t hist[SEL_BINS];
    __shared__ float s_tab[256];
    __shared__ uint32_t s_w[WAVES];
    __shared__ uint32_t s_r[3][WAVES];
    __shared__ uint32_t s_pick[2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t r = blockIdx.x;
    cand_table(a, r, s_tab, tid, CS_THREADS);
    const RowIdx ri = split_row(r, a.L, a.Hkv);
    const float *sr = a.scores + (size_t)r * a.T;
    const uint8_t *tr = a.tags ? a.tags + (size_t)(a.tag_rows ? r : ri.n) * a.T : nullptr;
    const int64_t groups = a.T / 4, lo = a.n_sink, hi = a.T - a.n_recent;
    uint32_t key[NG][4], tg[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        const int64_t j0 = 4 * ((int64_t)(k * CS_THREADS + tid) * groups / CS_SAMPLE_GROUPS);
        const uint4 v = *reinterpret_cast<const uint4 *>(sr + j0);
        tg[k] = tr ? *reinterpret_cast<const uint32_t *>(tr + j0) : 0u;
        key[k][0] = v.x;
        key[k][1] = v.y;
        key[k][2] = v.z;
        key[k][3] = v.w;
    }
    __syncthreads();   // s_tab
    uint32_t nprot = 0u, kmin = 0xFFFFFFFFu, kmax1 = 0u;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        const int64_t j0 = 4 * ((int64_t)(k * CS_THREADS + tid) * groups / CS_SAMPLE_GROUPS);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t kk =
                cand_key_of(j0 + e, __uint_as_float(key[k][e]), s_tab[(tg[k] >> (8 * e)) & 0xFF], lo, hi);
            key[k][e] = kk;
            nprot += kk == KEY_PROTECTED ? 1u : 0u;
            kmin = min(kmin, kk);             // a protected key never lowers kmin
            kmax1 = max(kmax1, kk + 1u);      // and wraps to 0 here
        }
    }
    nprot = __builtin_amdgcn_readlane(wave_incl_scan(nprot), 63);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
        kmax1 = max(kmax1, (uint32_t)__shfl_xor((int)kmax1, o));
    }
    if (lane == 0) {
        s_r[0][wave] = nprot;
        s_r[1][wave] = kmin;
        s_r[2][wave] = kmax1;
    }
    __syncthreads();
    nprot = 0u;
    kmin = 0xFFFFFFFFu;
    kmax1 = 0u;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        nprot += s_r[0][w];
        kmin = min(kmin, s_r[1][w]);
        kmax1 = max(kmax1, s_r[2][w]);
    }
    const int ns = CS_SAMPLE_GROUPS * 4;
    int64_t rs = (int64_t)(((double)a.B * 2.5 * ns + (double)a.T - 1) / (double)a.T) + 4;
    rs = rs > ns ? ns : rs;
    uint32_t k_lo;
    if (nprot >= (uint32_t)rs) {
        k_lo = KEY_PROTECTED;
    } else {
        BlkRadix<CS_THREADS> rx{hist, s_w, s_pick};
        auto count = [&](auto match, auto digit) {
            rx.clear();
#pragma unroll
            for (int k = 0; k < NG; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t kk = key[k][e], d = kk - kmin;
                    hist_add_agg(hist, kk != KEY_PROTECTED && match(d), digit(d));
                }
            __syncthreads();
        };
        const uint32_t range = kmax1 - 1u - kmin;
        const int bl = range ? 32 - __clz(range) : 0;
        const int s0 = bl > 11 ? bl - 11 : 0;
        const int w1 = s0 < 11 ? s0 : 11, s1 = s0 - w1;
        uint32_t kr = (uint32_t)rs - nprot, dt;
        count([](uint32_t) { return true; }, [&](uint32_t d) { return d >> s0; });
        rx.pick(kr, dt, kr);
        if (w1) {
            count([&](uint32_t d) { return (d >> s0) == dt; }, [&](uint32_t d) { return (d >> s1) & ((1u << w1) - 1u); });
            uint32_t b1;
            rx.pick(kr, b1, kr);
            dt = (dt << w1) | b1;
        }
        if (s1) {
            count([&](uint32_t d) { return (d >> s1) == dt; }, [&](uint32_t d) { return d & ((1u << s1) - 1u); });
            uint32_t b2;
            rx.pick(kr, b2, kr);
            dt = (dt << s1) | b2;
        }
        k_lo = kmin + dt;
    }
    if (tid == 0) a.k_lo[r] = k_lo;
}

__global__ void __launch_bounds__(CF_THREADS) cand_filter(CandArgs a) {
    constexpr int WAVES = CF_THREADS / 64;
    __shared__ float s_tab[256];
    __shared__ uint32_t s_w[WAVES];
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x / a.nseg;
    const int sg = (int)(blockIdx.x % a.nseg);
    const int64_t p0 = (int64_t)sg * CF_SEG;
    const int nv = (int)(a.T - p0 < CF_SEG ? a.T - p0 : CF_SEG);
    cand_table(a, r, s_tab, tid, CF_THREADS);
    const RowIdx ri = split_row(r, a.L, a.Hkv);
    const float *sr = a.scores + (size_t)r * a.T + p0;
    const uint8_t *tr = a.tags ? a.tags + (size_t)(a.tag_rows ? r : ri.n) * a.T + p0 : nullptr;
    uint4 v[4];
    uint32_t t4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int base = k * CF_THREADS * 4 + 4 * tid;
        v[k] = make_uint4(0u, 0u, 0u, 0u);
        t4[k] = 0u;
        if (base < nv) {   // T % 4 == 0: a group is wholly inside or outside
            v[k] = *reinterpret_cast<const uint4 *>(sr + base);
            if (tr) t4[k] = *reinterpret_cast<const uint32_t *>(tr + base);
        }
    }
    const uint32_t k_lo = a.k_lo[r];
    const int64_t lo = a.n_sink, hi = a.T - a.n_recent;
    __syncthreads();   // s_tab
    uint32_t *ck = a.c_key + (size_t)r * a.T + p0;
    int32_t *ci = a.c_idx + (size_t)r * a.T + p0;
    uint32_t run = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int base = k * CF_THREADS * 4 + 4 * tid;
        const uint32_t x[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
        uint32_t kk[4], n = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kk[e] = cand_key_of(p0 + base + e, __uint_as_float(x[e]), s_tab[(t4[k] >> (8 * e)) & 0xFF], lo, hi);
            n += (base < nv && kk[e] >= k_lo) ? 1u : 0u;
        }
        uint32_t tot;
        uint32_t pos = run + blk_excl_scan<WAVES>(n, tot, s_w);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (base < nv && kk[e] >= k_lo) {
                ck[pos] = kk[e];
                ci[pos] = (int32_t)(p0 + base + e);
                ++pos;
            }
        run += tot;
    }
    if (tid == 0) a.cnt[(size_t)r * a.nseg + sg] = run;
}

__global__ void __launch_bounds__(CR_THREADS) cand_resolve(CandArgs a) {
    constexpr int WAVES = CR_THREADS / 64;
    __shared__ uint32_t c_key[CAND_CAP];
    __shared__ int32_t c_idx[CAND_CAP];
    __shared__ __align__(16) uint32_t hist[SEL_BINS];
    __shared__ uint32_t s_w[WAVES];
    __shared__ uint32_t s_r[3][WAVES];
    __shared__ uint32_t s_pick[2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t r = blockIdx.x;
    const uint32_t *cnt = a.cnt + (size_t)r * a.nseg;
    uint32_t total = 0u;
    for (int s0 = 0; s0 < a.nseg; s0 += CR_THREADS) {
        uint32_t t;
        blk_excl_scan<WAVES>(s0 + tid < a.nseg ? cnt[s0 + tid] : 0u, t, s_w);
        total += t;
    }
    const int B = a.B;
    if (total < (uint32_t)B || total > (uint32_t)CAND_CAP) {   // the sample misled: exact kernel
        if (tid == 0) a.flag[r] = 1u;
        return;
    }
    if (tid == 0) a.flag[r] = 0u;
    // gather the segments' candidates in order
    uint32_t base = 0u;
    for (int sg = 0; sg < a.nseg; ++sg) {
        const uint32_t c = cnt[sg];
        const uint32_t *ck = a.c_key + (size_t)r * a.T + (size_t)sg * CF_SEG;
        const int32_t *ci = a.c_idx + (size_t)r * a.T + (size_t)sg * CF_SEG;
        for (uint32_t i = tid; i < c; i += CR_THREADS) {
            c_key[base + i] = ck[i];
            c_idx[base + i] = ci[i];
        }
        base += c;
    }
    __syncthreads();
    const int n = (int)total;
    // protected count and the range of the other keys
    uint32_t nprot = 0u, kmin = 0xFFFFFFFFu, kmax1 = 0u;
    for (int p = tid; p < n; p += CR_THREADS) {
        const uint32_t kk = c_key[p];
        nprot += kk == KEY_PROTECTED ? 1u : 0u;
        kmin = min(kmin, kk);
        kmax1 = max(kmax1, kk + 1u);
    }
    nprot = __builtin_amdgcn_readlane(wave_incl_scan(nprot), 63);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
        kmax1 = max(kmax1, (uint32_t)__shfl_xor((int)kmax1, o));
    }
    if (lane == 0) {
        s_r[0][wave] = nprot;
        s_r[1][wave] = kmin;
        s_r[2][wave] = kmax1;
    }
    __syncthreads();
    nprot = 0u;
    kmin = 0xFFFFFFFFu;
    kmax1 = 0u;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        nprot += s_r[0][w];
        kmin = min(kmin, s_r[1][w]);
        kmax1 = max(kmax1, s_r[2][w]);
    }
    uint32_t tau;
    int need;
    if (nprot >= (uint32_t)B) {   // only when exactly B: every protected token
        tau = KEY_PROTECTED;
        need = B;
    } else {
        BlkRadix<CR_THREADS> rx{hist, s_w, s_pick};
        auto count = [&](auto match, auto digit) {
            rx.clear();
            for (int p0 = 0; p0 < n; p0 += CR_THREADS) {   // every lane of a wave takes the same trips
                const int p = p0 + tid;
                const uint32_t kk = p < n ? c_key[p] : KEY_PROTECTED, d = kk - kmin;
                hist_add_agg(hist, kk != KEY_PROTECTED && match(d), digit(d));
            }
            __syncthreads();
        };
        auto pick = [&](uint32_t kr, uint32_t &bin, uint32_t &rank) { rx.pick(kr, bin, rank); };
        const uint32_t range = kmax1 - 1u - kmin;
        const int bl = range ? 32 - __clz(range) : 0;
        const int s0 = bl > 11 ? bl - 11 : 0;
        const int w1 = s0 < 11 ? s0 : 11, s1 = s0 - w1;
        uint32_t kr = (uint32_t)B - nprot, dt;
        count([](uint32_t) { return true; }, [&](uint32_t d) { return d >> s0; });
        pick(kr, dt, kr);
        if (w1) {
            count([&](uint32_t d) { return (d >> s0) == dt; }, [&](uint32_t d) { return (d >> s1) & ((1u << w1) - 1u); });
            uint32_t b1;
            pick(kr, b1, kr);
            dt = (dt << w1) | b1;
        }
        if (s1) {
            count([&](uint32_t d) { return (d >> s1) == dt; }, [&](uint32_t d) { return d & ((1u << s1) - 1u); });
            uint32_t b2;
            pick(kr, b2, kr);
            dt = (dt << s1) | b2;
        }
        tau = kmin + dt;
        need = (int)kr;
    }
    // ordered write: key > tau, and the first `need` keys == tau in list (= index) order
    int32_t *out = a.kept + (size_t)r * a.kept_stride;
    uint32_t gt_run = 0u, eq_run = 0u;
    for (int c0 = 0; c0 < n; c0 += CR_THREADS * 4) {
        const int pb = c0 + 4 * tid;
        uint32_t ngt = 0u, neq = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool v = pb + e < n;
            const uint32_t kk = v ? c_key[pb + e] : 0u;
            ngt += (v && kk > tau) ? 1u : 0u;
            neq += (v && kk == tau) ? 1u : 0u;
        }
        uint32_t tot;
        const uint32_t ex = blk_excl_scan<WAVES>(ngt | (neq << 16), tot, s_w);
        int gt_before = (int)(gt_run + (ex & 0xFFFFu)), eq_before = (int)(eq_run + (ex >> 16));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool v = pb + e < n;
            const uint32_t kk = v ? c_key[pb + e] : 0u;
            const bool gt = v && kk > tau, eq = v && kk == tau;
            if (gt || (eq && eq_before < need)) {
                const int pos = gt_before + (eq_before < need ? eq_before : need);
                if (pos < a.kept_stride) out[KVC_IDX(pos, a.kept_stride, KVC_CHK_SELECT)] = c_idx[pb + e];
            }
            gt_before += gt ? 1 : 0;
            eq_before += eq ? 1 : 0;
        }
        gt_run += tot & 0xFFFFu;
        eq_run += tot >> 16;
    }
    if (tid == 0) a.n_kept[r] = (int32_t)(gt_run + (eq_run < (uint32_t)need ? eq_run : (uint32_t)need));
}

KVC_CHECK_READER(check_read_select)

static bool select_use_split(const kvc_dims *d) {
    const int64_t T = d->n_tokens, rows = n_rows(d);
    return T >= 262144 || (rows < 128 && T >= 32768);
}

// The sampled path serves the rows that would otherwise be split over
// several workgroups (long rows, or few rows of at least 32,768 tokens); with
// many rows of moderate length one workgroup per row streams as fast.
static bool cand_eligible(const kvc_dims *d, const kvc_policy *p, bool vec) {
    const int64_t T = d->n_tokens;
    return vec && select_use_split(d) && !p->tag_floor && p->budget <= 2048 && 5 * (int64_t)p->budget <= T &&
           (int64_t)p->n_sink + p->n_recent <= p->budget;
}

static size_t cand_workspace_bytes(int64_t rows, int64_t T) {
    const int64_t nseg = (T + CF_SEG - 1) / CF_SEG;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return al(rows * 4) * 2 + al(rows * nseg * 4) + al((size_t)rows * T * 4) * 2;
}

static int launch_select_cand(const kvc_dims *dims, const kvc_policy *p, const float *scores, int32_t *kept,
                              int kept_stride, int32_t *n_kept, void *ws, hipStream_t s) {
    const int64_t rows = n_rows(dims), T = dims->n_tokens;
    const int nseg = (int)((T + CF_SEG - 1) / CF_SEG);
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    char *w = reinterpret_cast<char *>(ws);
    CandArgs a;
    a.scores = scores;
    a.tags = p->tags;
    a.bonus = p->tag_bonus;
    a.T = T;
    a.rows = rows;
    a.L = dims->n_layers;
    a.Hkv = dims->n_kv_heads;
    a.n_groups = p->n_groups;
    a.layer_base = p->layer_base;
    a.n_layers_model = p->n_layers_model;
    a.n_tags = p->n_tags;
    a.tag_rows = p->tag_rows;
    a.n_sink = p->n_sink;
    a.n_recent = p->n_recent;
    a.B = p->budget;
    a.nseg = nseg;
    a.k_lo = reinterpret_cast<uint32_t *>(w);
    a.flag = reinterpret_cast<uint32_t *>(w + al(rows * 4));
    a.cnt = reinterpret_cast<uint32_t *>(w + 2 * al(rows * 4));
    a.c_key = reinterpret_cast<uint32_t *>(w + 2 * al(rows * 4) + al(rows * nseg * 4));
    a.c_idx = reinterpret_cast<int32_t *>(w + 2 * al(rows * 4) + al(rows * nseg * 4) + al((size_t)rows * T * 4));
    a.kept = kept;
    a.kept_stride = kept_stride;
    a.n_kept = n_kept;
    if (rows * nseg > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "kvc_select: grid too large");
    cand_sample<<<dim3((unsigned)rows), dim3(CS_THREADS), 0, s>>>(a);
    cand_filter<<<dim3((unsigned)(rows * nseg)), dim3(CF_THREADS), 0, s>>>(a);
    cand_resolve<<<dim3((unsigned)rows), dim3(CR_THREADS), 0, s>>>(a);
    // rows whose sample misled: the exact one-workgroup kernel, only for them
    select_kernel<true><<<dim3((unsigned)rows), dim3(SEL_THREADS), 0, s>>>(
        scores, p->tags, p->tag_bonus, nullptr, T, dims->n_layers, dims->n_kv_heads, p->n_groups, p->layer_base,
        p->n_layers_model, p->n_tags, p->tag_rows, p->n_sink, p->n_recent, p->budget, kept, kept_stride, n_kept,
        a.flag);
    return check_launch("kvc_select (sampled threshold)");
}

template <int NPL4>
static void launch_select_wave(bool vec, int64_t rows, hipStream_t s, const float *scores, const kvc_policy *p,
                               const kvc_dims *dims, int32_t *kept, int kept_stride, int32_t *n_kept) {
    const dim3 grid((unsigned)((rows + SW_WAVES - 1) / SW_WAVES)), block(SW_WAVES * 64);
    if (vec)
        select_wave<NPL4, true><<<grid, block, 0, s>>>(scores, p->tags, p->tag_bonus, p->tag_floor, (int)dims->n_tokens,
                                                       rows, dims->n_layers, dims->n_kv_heads, p->n_groups,
                                                       p->layer_base, p->n_layers_model, p->n_tags, p->tag_rows,
                                                       p->n_sink, p->n_recent, p->budget, kept, kept_stride, n_kept);
    else
        select_wave<NPL4, false><<<grid, block, 0, s>>>(scores, p->tags, p->tag_bonus, p->tag_floor, (int)dims->n_tokens,
                                                        rows, dims->n_layers, dims->n_kv_heads, p->n_groups,
                                                        p->layer_base, p->n_layers_model, p->n_tags, p->tag_rows,
                                                        p->n_sink, p->n_recent, p->budget, kept, kept_stride, n_kept);
}


static size_t split_bytes(int64_t rows, int64_t chunks) {
    return align256s((size_t)rows * 3 * SEL_BINS * sizeof(uint32_t)) + align256s((size_t)rows * sizeof(SplitState)) +
           align256s((size_t)rows * chunks * 2 * sizeof(uint32_t)) + align256s((size_t)rows * chunks * 2 * sizeof(int64_t));
}

static SplitWs split_layout(void *ws, int64_t rows, int64_t chunks) {
    char *p = reinterpret_cast<char *>(ws);
    SplitWs w;
    w.hist = reinterpret_cast<uint32_t *>(p);
    p += align256s((size_t)rows * 3 * SEL_BINS * sizeof(uint32_t));
    w.state = reinterpret_cast<SplitState *>(p);
    p += align256s((size_t)rows * sizeof(SplitState));
    w.cnt = reinterpret_cast<uint32_t *>(p);
    p += align256s((size_t)rows * chunks * 2 * sizeof(uint32_t));
    w.base = reinterpret_cast<int64_t *>(p);
    return w;
}

struct SplitArgs {
    const float *scores;
    const uint8_t *tags;
    const float *bonus;
    const uint8_t *floor_tbl;
    int64_t T;
    int L, Hkv, n_groups, layer_base, n_layers_model, n_tags, n_sink, n_recent, B;
    int tag_rows;
    int32_t *kept;
    int kept_stride;
    int32_t *n_kept;
    int64_t chunks;
};

// Per-workgroup bonus/floor table of the row's layer group, and the row view.
__device__ __forceinline__ SelRow split_row_view(const SplitArgs &a, int64_t r, float *s_bonus, uint8_t *s_floor) {
    const RowIdx ri = split_row(r, a.L, a.Hkv);
    const int grp = device_layer_group(a.layer_base + ri.l, a.n_layers_model, a.n_groups);
    for (int t = threadIdx.x; t < 256; t += SEL_THREADS) {
        s_bonus[t] = (a.bonus && t < a.n_tags) ? a.bonus[t * a.n_groups + grp] : 0.f;
        s_floor[t] = (a.floor_tbl && t < a.n_tags) ? a.floor_tbl[t * a.n_groups + grp] : 0;
    }
    __syncthreads();
    return SelRow{a.scores + (size_t)r * a.T, a.tags ? a.tags + (size_t)(a.tag_rows ? r : ri.n) * a.T : nullptr,
                  a.T, a.n_sink, a.n_recent, a.n_tags, s_bonus, s_floor};
}

__global__ void __launch_bounds__(SEL_THREADS) split_init(SplitWs w, int64_t rows) {
    const int64_t n = rows * 3 * SEL_BINS;
    for (int64_t i = (int64_t)blockIdx.x * SEL_THREADS + threadIdx.x; i < n; i += (int64_t)gridDim.x * SEL_THREADS)
        w.hist[i] = 0u;
    for (int64_t i = (int64_t)blockIdx.x * SEL_THREADS + threadIdx.x; i < rows; i += (int64_t)gridDim.x * SEL_THREADS)
        w.state[i] = SplitState{0u, 0u, 0u, 0u, 0};
}

// Histogram of digit `pass` over one chunk, for the keys whose higher digits
// equal the row's prefix.
template <bool VEC>
__global__ void __launch_bounds__(SEL_THREADS) split_hist(SplitArgs a, SplitWs w, int pass) {
    __shared__ float s_bonus[256];
    __shared__ uint8_t s_floor[256];
    __shared__ uint32_t hist[SEL_BINS];
    const int64_t r = blockIdx.x / a.chunks, c = blockIdx.x % a.chunks;
    const SplitState st = w.state[r];
    if (st.done) return;
    const SelRow row = split_row_view(a, r, s_bonus, s_floor);
    for (int t = threadIdx.x; t < SEL_BINS; t += SEL_THREADS) hist[t] = 0u;
    __syncthreads();
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int width = pass == 2 ? 10 : 11;
    const uint32_t mask = (1u << width) - 1u;
    const int64_t c0 = c * SPLIT_CHUNK, c1 = c0 + SPLIT_CHUNK < a.T ? c0 + SPLIT_CHUNK : a.T;
    for (int64_t base = c0 + (int64_t)threadIdx.x * SEL_VEC; base < c0 + SPLIT_CHUNK;
         base += (int64_t)SEL_THREADS * SEL_VEC) {
        uint32_t kk[SEL_VEC];
        bool valid[SEL_VEC];
        if (base < c1) {
            row.keys4<VEC>(base, kk, valid);
        } else {
#pragma unroll
            for (int e = 0; e < SEL_VEC; ++e) valid[e] = false, kk[e] = 0u;
        }
#pragma unroll
        for (int e = 0; e < SEL_VEC; ++e) {
            const bool active = valid[e] && (pass == 0 || (kk[e] >> (shift + width)) == st.prefix);
            const uint32_t digit = (kk[e] >> shift) & mask;
            if (pass == 0)
                wave_hist_add(hist, active, digit);  // leading digits cluster in a few bins
            else if (active)
                atomicAdd(&hist[digit], 1u);
        }
    }
    __syncthreads();
    uint32_t *g = w.hist + ((size_t)r * 3 + pass) * SEL_BINS;
    for (int t = threadIdx.x; t < (1 << width); t += SEL_THREADS)
        if (hist[t]) atomicAdd(&g[t], hist[t]);
}

// One workgroup per row: the bin of digit `pass` holding the budget-th key.
__global__ void __launch_bounds__(SEL_THREADS) split_pick(SplitArgs a, SplitWs w, int pass) {
    __shared__ uint32_t hist[SEL_BINS];
    __shared__ uint32_t s_wave[SEL_WAVES + 1];
    __shared__ uint32_t s_pick[2];
    const int64_t r = blockIdx.x;
    SplitState st = w.state[r];
    if (st.done) return;
    const uint32_t *g = w.hist + ((size_t)r * 3 + pass) * SEL_BINS;
    for (int t = threadIdx.x; t < SEL_BINS; t += SEL_THREADS) hist[t] = g[t];
    __syncthreads();
    if (pass == 0) {
        if (a.T <= a.B) {  // every token is kept
            st = SplitState{0u, 0u, 1u, 0u, a.T};
        } else if (hist[SEL_BINS - 1] >= (uint32_t)a.B) {  // protected tokens fill the budget: keep them all
            st = SplitState{KEY_PROTECTED, 0u, 1u, 0u, a.T};
        }
        if (st.done) {
            if (threadIdx.x == 0) w.state[r] = st;
            return;
        }
        st.k = (uint32_t)a.B;
    }
    const int width = pass == 2 ? 10 : 11;
    uint32_t bin, rank;
    pick_bin(hist, 1 << width, st.k, s_wave, s_pick, bin, rank);
    st.prefix = (st.prefix << width) | bin;
    st.k = rank;
    if (pass == 2) {
        st.done = 1u;
        st.need = rank;
    }
    if (threadIdx.x == 0) w.state[r] = st;
}

// Keys above and equal to tau in one chunk.
template <bool VEC>
__global__ void __launch_bounds__(SEL_THREADS) split_count(SplitArgs a, SplitWs w) {
    __shared__ float s_bonus[256];
    __shared__ uint8_t s_floor[256];
    __shared__ uint32_t s_wave[SEL_WAVES + 1];
    const int64_t r = blockIdx.x / a.chunks, c = blockIdx.x % a.chunks;
    const SplitState st = w.state[r];
    const uint32_t tau = st.prefix;
    const SelRow row = split_row_view(a, r, s_bonus, s_floor);
    const int64_t c0 = c * SPLIT_CHUNK, c1 = c0 + SPLIT_CHUNK < a.T ? c0 + SPLIT_CHUNK : a.T;
    uint32_t ngt = 0, neq = 0;
    for (int64_t base = c0 + (int64_t)threadIdx.x * SEL_VEC; base < c1; base += (int64_t)SEL_THREADS * SEL_VEC) {
        uint32_t kk[SEL_VEC];
        bool valid[SEL_VEC];
        row.keys4<VEC>(base, kk, valid);
#pragma unroll
        for (int e = 0; e < SEL_VEC; ++e) {
            ngt += valid[e] && kk[e] > tau;
            neq += valid[e] && kk[e] == tau;
        }
    }
    uint32_t tg, te;
    block_excl_scan(ngt, &tg, s_wave);
    block_excl_scan(neq, &te, s_wave);
    if (threadIdx.x == 0) {
        w.cnt[((size_t)r * a.chunks + c) * 2] = tg;
        w.cnt[((size_t)r * a.chunks + c) * 2 + 1] = te;
    }
}

// One workgroup per row: each chunk's first output slot and the number of
// tau-valued tokens before it; the row's kept count.
__global__ void __launch_bounds__(SEL_THREADS) split_scan(SplitArgs a, SplitWs w) {
    __shared__ uint32_t s_wave[SEL_WAVES + 1];
    const int64_t r = blockIdx.x;
    const int64_t need = w.state[r].need;
    int64_t carry_g = 0, carry_e = 0;
    for (int64_t c0 = 0; c0 < a.chunks; c0 += SEL_THREADS) {
        const int64_t c = c0 + threadIdx.x;
        const uint32_t g = c < a.chunks ? w.cnt[((size_t)r * a.chunks + c) * 2] : 0u;
        const uint32_t e = c < a.chunks ? w.cnt[((size_t)r * a.chunks + c) * 2 + 1] : 0u;
        // counts per chunk are at most SPLIT_CHUNK, so 1024 of them sum below 2^32
        uint32_t tg, te;
        const uint32_t eg = block_excl_scan(g, &tg, s_wave);
        const uint32_t ee = block_excl_scan(e, &te, s_wave);
        if (c < a.chunks) {
            const int64_t eq_before = carry_e + ee;
            w.base[((size_t)r * a.chunks + c) * 2] = carry_g + eg + (eq_before < need ? eq_before : need);
            w.base[((size_t)r * a.chunks + c) * 2 + 1] = eq_before;
        }
        carry_g += tg;
        carry_e += te;
    }
    if (threadIdx.x == 0) a.n_kept[r] = (int32_t)(carry_g + (carry_e < need ? carry_e : need));
}

// Every chunk writes its kept indices in index order from its first slot.
template <bool VEC>
__global__ void __launch_bounds__(SEL_THREADS) split_write(SplitArgs a, SplitWs w) {
    __shared__ float s_bonus[256];
    __shared__ uint8_t s_floor[256];
    __shared__ uint32_t s_wave[SEL_WAVES + 1];
    const int64_t r = blockIdx.x / a.chunks, c = blockIdx.x % a.chunks;
    const SplitState st = w.state[r];
    const uint32_t tau = st.prefix;
    const int64_t need = st.need;
    const SelRow row = split_row_view(a, r, s_bonus, s_floor);
    const int64_t c0 = c * SPLIT_CHUNK, c1 = c0 + SPLIT_CHUNK < a.T ? c0 + SPLIT_CHUNK : a.T;
    const int64_t slot0 = w.base[((size_t)r * a.chunks + c) * 2];
    const int64_t eq0 = w.base[((size_t)r * a.chunks + c) * 2 + 1];
    int32_t *kr = a.kept + (size_t)r * a.kept_stride;
    // running counts from the chunk start: slot = slot0 + gt_seen + taken ties seen
    int64_t carry_gt = 0, carry_eq = 0;
    for (int64_t it = c0; it < c1; it += (int64_t)SEL_THREADS * SEL_VEC) {
        const int64_t base = it + (int64_t)threadIdx.x * SEL_VEC;
        uint32_t kk[SEL_VEC];
        bool valid[SEL_VEC];
        if (base < c1) {
            row.keys4<VEC>(base, kk, valid);
        } else {
#pragma unroll
            for (int e = 0; e < SEL_VEC; ++e) valid[e] = false, kk[e] = 0u;
        }
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int e = 0; e < SEL_VEC; ++e) {
            ngt += valid[e] && kk[e] > tau;
            neq += valid[e] && kk[e] == tau;
        }
        uint32_t tot;
        const uint32_t ex = block_excl_scan(ngt | (neq << 16), &tot, s_wave);
        int64_t gt_before = carry_gt + (ex & 0xFFFFu);
        int64_t eq_before = eq0 + carry_eq + (ex >> 16);
#pragma unroll
        for (int e = 0; e < SEL_VEC; ++e) {
            const bool gt = valid[e] && kk[e] > tau;
            const bool eq = valid[e] && kk[e] == tau;
            if (gt || (eq && eq_before < need)) {
                // slot0 already counts the ties taken before the chunk
                const int64_t taken = (eq_before < need ? eq_before : need) - (eq0 < need ? eq0 : need);
                const int64_t pos = slot0 + gt_before + taken;
                if (pos < a.kept_stride) kr[KVC_IDX(pos, a.kept_stride, KVC_CHK_SELECT)] = (int32_t)(base + e);
            }
            gt_before += gt;
            eq_before += eq;
        }
        carry_gt += tot & 0xFFFFu;
        carry_eq += tot >> 16;
    }
}

static int launch_select_split(const SplitArgs &a, int64_t rows, void *ws, bool vec, hipStream_t s) {
    const SplitWs w = split_layout(ws, rows, a.chunks);
    const int64_t grid_c = rows * a.chunks;
    if (grid_c > (int64_t)INT32_MAX || rows > (int64_t)INT32_MAX)
        return fail(KVC_ERR_UNSUPPORTED, "kvc_select: grid too large");
    const dim3 block(SEL_THREADS);
    const int64_t init_blocks = (rows * 3 * SEL_BINS + SEL_THREADS - 1) / SEL_THREADS;
    split_init<<<dim3((unsigned)(init_blocks < 1024 ? init_blocks : 1024)), block, 0, s>>>(w, rows);
    for (int pass = 0; pass < 3; ++pass) {
        if (vec)
            split_hist<true><<<dim3((unsigned)grid_c), block, 0, s>>>(a, w, pass);
        else
            split_hist<false><<<dim3((unsigned)grid_c), block, 0, s>>>(a, w, pass);
        split_pick<<<dim3((unsigned)rows), block, 0, s>>>(a, w, pass);
    }
    if (vec)
        split_count<true><<<dim3((unsigned)grid_c), block, 0, s>>>(a, w);
    else
        split_count<false><<<dim3((unsigned)grid_c), block, 0, s>>>(a, w);
    split_scan<<<dim3((unsigned)rows), block, 0, s>>>(a, w);
    if (vec)
        split_write<true><<<dim3((unsigned)grid_c), block, 0, s>>>(a, w);
    else
        split_write<false><<<dim3((unsigned)grid_c), block, 0, s>>>(a, w);
    return check_launch("kvc_select (long rows)");
}

// Workspace of kvc_select: the long-row path's histograms, per-row state and
// per-chunk counts; 0 when the rows take the one-workgroup kernels.
size_t select_workspace_bytes(const kvc_dims *d, int32_t B) {
    size_t n = 0;
    if (select_use_split(d)) {
        const int64_t chunks = (d->n_tokens + SPLIT_CHUNK - 1) / SPLIT_CHUNK;
        n = split_bytes(n_rows(d), chunks);
    }
    if (select_use_split(d) && B > 0 && B <= 2048 && 5 * (int64_t)B <= d->n_tokens) {
        const size_t m = cand_workspace_bytes(n_rows(d), d->n_tokens);
        n = m > n ? m : n;
    }
    return n;
}

}  // namespace kvc

using namespace kvc;

extern "C" int kvc_select(const kvc_dims *dims, const float *scores, const kvc_policy *p,
                          int32_t *kept_idx, int32_t kept_stride, int32_t *n_kept, void *ws,
                          size_t ws_bytes, void *stream) {
    int st = check_dims(dims, "kvc_select");
    if (st != KVC_OK) return st;
    if (!scores || !p || !kept_idx || !n_kept) return fail(KVC_ERR_ARG, "kvc_select: NULL pointer");
    const int64_t T = dims->n_tokens;
    if (p->budget <= 0) return fail(KVC_ERR_ARG, "kvc_select: budget %d must be positive", p->budget);
    if (p->n_sink < 0 || p->n_recent < 0) return fail(KVC_ERR_ARG, "kvc_select: negative sink/recent");
    if (p->n_tags < 1 || p->n_tags > 256 || p->n_groups < 1 || p->n_tags * p->n_groups > 256 * 64)
        return fail(KVC_ERR_ARG, "kvc_select: table %d x %d out of range (tags 1..256)", p->n_tags,
                    p->n_groups);
    if (p->tag_rows != 0 && p->tag_rows != 1)
        return fail(KVC_ERR_ARG, "kvc_select: tag_rows must be 0 or 1 (got %d)", p->tag_rows);
    if (p->n_layers_model <= 0 || p->layer_base < 0 || p->layer_base + dims->n_layers > p->n_layers_model)
        return fail(KVC_ERR_ARG, "kvc_select: layers [%d, %d) outside a %d-layer model", p->layer_base,
                    p->layer_base + dims->n_layers, p->n_layers_model);
    const int64_t want = T < p->budget ? T : p->budget;
    if (kept_stride < want)
        return fail(KVC_ERR_ARG, "kvc_select: kept_stride %d < min(budget, T) = %lld", kept_stride,
                    (long long)want);
    // Table floors may protect any token, and every protected token is kept
    // (floors take precedence over the budget): only a full-length list is
    // sure to hold them all.
    if (p->tag_floor && T > p->budget && kept_stride < T)
        return fail(KVC_ERR_ARG, "kvc_select: with a floor table kept_stride %d must be >= T = %lld", kept_stride,
                    (long long)T);
    // float4 score loads and 4-byte tag loads need every row start 16-byte aligned.
    const bool vec = (T % 4 == 0) && (reinterpret_cast<uintptr_t>(scores) % 16 == 0) &&
                     (!p->tags || reinterpret_cast<uintptr_t>(p->tags) % 4 == 0);
    const dim3 grid((unsigned)n_rows(dims)), block(SEL_THREADS);
    hipStream_t s = as_stream(stream);
    // rows whose decision map fits in LDS next to the candidate list
    const size_t cand_lds = (size_t)2 * SEL_CAND * sizeof(uint32_t) + (size_t)2 * ((T + 31) / 32) * sizeof(uint32_t);
    if (T <= 8192) {
        const int64_t rows = n_rows(dims);
        if (T <= 1024)
            launch_select_wave<4>(vec, rows, s, scores, p, dims, kept_idx, kept_stride, n_kept);
        else if (T <= 2048)
            launch_select_wave<8>(vec, rows, s, scores, p, dims, kept_idx, kept_stride, n_kept);
        else if (T <= 4096)
            launch_select_wave<16>(vec, rows, s, scores, p, dims, kept_idx, kept_stride, n_kept);
        else
            launch_select_wave<32>(vec, rows, s, scores, p, dims, kept_idx, kept_stride, n_kept);
    } else if (cand_eligible(dims, p, vec) && ws && ws_bytes >= cand_workspace_bytes(n_rows(dims), T)) {
        if ((st = launch_select_cand(dims, p, scores, kept_idx, kept_stride, n_kept, ws, s)) != KVC_OK) return st;
    } else if (select_use_split(dims)) {
        const size_t need = select_workspace_bytes(dims, 0);
        if (!ws || ws_bytes < need)
            return fail(KVC_ERR_WORKSPACE, "kvc_select: workspace %zu < %zu bytes (long rows)", ws_bytes, need);
        SplitArgs a{scores, p->tags, p->tag_bonus, p->tag_floor, T, dims->n_layers, dims->n_kv_heads, p->n_groups,
                    p->layer_base, p->n_layers_model, p->n_tags, p->n_sink, p->n_recent, p->budget, p->tag_rows,
                    kept_idx, kept_stride, n_kept, (T + SPLIT_CHUNK - 1) / SPLIT_CHUNK};
        if ((st = launch_select_split(a, n_rows(dims), ws, vec, s)) != KVC_OK) return st;
    } else if (vec && cand_lds <= 144 * 1024) {
        const size_t small_lds = (size_t)2 * SEL_CAND_SMALL * sizeof(uint32_t) +
                                 (size_t)2 * ((T + 31) / 32) * sizeof(uint32_t);
        static size_t small_static = 0;   // the small instance's static LDS, asked once
        if (!small_static) {
            hipFuncAttributes fa;
            if (hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(&select_cand<SEL_CAND_SMALL, 2, 8>)) !=
                hipSuccess)
                return fail(KVC_ERR_HIP, "kvc_select: cannot read the candidate kernel's attributes");
            small_static = fa.sharedSizeBytes > 0 ? fa.sharedSizeBytes : 1;
        }
        const bool small = p->budget <= 2048 && small_lds + small_static <= SEL_CAND_SMALL_LDS;
        auto launch = [&](auto kern, size_t lds) -> int {
            static bool lds_set[2] = {false, false};
            if (!lds_set[small]) {
                if (hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, 144 * 1024) != hipSuccess)
                    return fail(KVC_ERR_HIP, "kvc_select: cannot raise the LDS limit");
                lds_set[small] = true;
            }
            kern<<<grid, block, lds, s>>>(scores, p->tags, p->tag_bonus, p->tag_floor, T, dims->n_layers,
                                          dims->n_kv_heads, p->n_groups, p->layer_base, p->n_layers_model,
                                          p->n_tags, p->tag_rows, p->n_sink, p->n_recent, p->budget, kept_idx,
                                          kept_stride, n_kept);
            return KVC_OK;
        };
        st = small ? launch(select_cand<SEL_CAND_SMALL, 2, 8>, small_lds) : launch(select_cand<SEL_CAND, 4, 4>, cand_lds);
        if (st != KVC_OK) return st;
    } else if (vec) {
        select_kernel<true><<<grid, block, 0, s>>>(scores, p->tags, p->tag_bonus, p->tag_floor, T, dims->n_layers,
                                                    dims->n_kv_heads, p->n_groups, p->layer_base,
                                                    p->n_layers_model, p->n_tags, p->tag_rows, p->n_sink,
                                                    p->n_recent, p->budget, kept_idx, kept_stride, n_kept, nullptr);
    } else {
        select_kernel<false><<<grid, block, 0, s>>>(scores, p->tags, p->tag_bonus, p->tag_floor, T, dims->n_layers,
                                                     dims->n_kv_heads, p->n_groups, p->layer_base,
                                                     p->n_layers_model, p->n_tags, p->tag_rows, p->n_sink,
                                                     p->n_recent, p->budget, kept_idx, kept_stride, n_kept, nullptr);
    }
    if ((st = check_launch("kvc_select")) != KVC_OK) return st;
    const int64_t sink_recent = (int64_t)p->n_sink + p->n_recent;
    if (T > p->budget && (sink_recent < T ? sink_recent : T) > p->budget) {
        fail(KVC_WARN_FLOOR_EXCESS, "kvc_select: %lld sink+recent tokens exceed the budget %d",
             (long long)sink_recent, p->budget);
        return KVC_WARN_FLOOR_EXCESS;
    }
    return KVC_OK;
}
