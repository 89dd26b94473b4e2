// kvc_score with one read of the keys: a persistent kernel for long rows.
//
// The score of key j sums, over the G*W window queries of its row, the
// softmax weight exp(s_qj - M_q) / L_q (PASK §3.1 Eq. 1 attention, window
// queries as in CommitKV §3.1 Eq. 5, causal rule of CommitKV Eq. 6). The
// normaliser of query row q needs every key of the row, so a key's weight is
// only known once the whole row has been seen. Instead of streaming the keys
// twice, every workgroup here keeps what it computed from its keys on chip
// until the row's normalisers are known:
//
// * One workgroup per CU, four waves; all workgroups walk the rows in order
//   and share each row's 32-key tiles: wave v (of NWAVE) takes tiles v,
//   v + NWAVE, v + 2*NWAVE; the few tiles beyond 3*NWAVE go one per
//   workgroup, rotating with the row, and its four waves split that tile by
//   query block.
// * A tile's logits come from v_mfma_f32_32x32x16_bf16 as C[key][qrow] (a lane
//   owns one query row of each block and 16 keys). Each lane takes the
//   integer ceiling m of its 16 log2-domain logits per block and keeps
//   e = exp2(x - m) in fp16 (RNE, e <= 1) with m as int16, and folds the
//   tile into its running (M, l) per query row with exact power-of-two
//   rescaling.
// * A row's per-lane statistics are folded over the workgroup into one
//   log-sum-exp per query row and published; one wave per query row merges
//   the workgroups' values into the row's log-sum-exp LSE_q; every
//   workgroup fetches the 128 merged values. Each value travels as a 64-bit
//   word (value, row tag) written and read with agent-scope relaxed atomics,
//   so a reader knows from the tag alone that the value is there: no fence,
//   no counter, no float atomics (the merge order is fixed: the result does
//   not depend on timing).
// * Two rows after a row's tiles, its kept exponentials are finished:
//   score_j = sum over blocks and lanes of e * exp2(m - LSE_q), summed across
//   the 32 query-row lanes by a transposing reduction. Three rows are held
//   on chip: two in registers, one in LDS.
//
// Every wait is bounded (a realtime-clock limit); a wait that runs out sets
// an abort word all workgroups watch, so the grid drains and the call's
// status word reports it (the scores of unfinished rows are then undefined).
// The launch is cooperative, so all workgroups are resident together.
#include <cmath>
#include <mutex>
#include <vector>

#include <algorithm>

#include "kvc_internal.h"

namespace kvc {
namespace once {

constexpr int WAVES = 4, THREADS = WAVES * 64;
constexpr int NB = 4;               // query blocks of 32 rows: 128 query rows
constexpr int D = 128, S = D / 16;  // head dim, 16-dim k-steps
constexpr int TPW = 3;              // base tiles per wave per row
constexpr int RING = 8;             // rows of exchange words in flight
constexpr int SLOT_V = 28;          // uint4 per lane of one row's kept state
constexpr int NWG_MAX = 256;
constexpr int REF_EMPTY = -30000;   // reference of a block with no visible key
constexpr int M_EMPTY = -30001;     // running maximum before any key

// LDS layout (bytes)
constexpr int LDS_Q = 4 * S * 64 * 16;                       // query fragments, 32 KB
constexpr int LDS_SLOT = WAVES * SLOT_V * 64 * 16;           // one row's kept state
constexpr int LDS_PART = WAVES * 128 * 8;                    // per-wave (M, l) per query row
constexpr int LDS_FIN = 2 * 128 * 4;                         // merged LSE, two rows
constexpr int LDS_XS = 2 * WAVES * 32 * 4;                   // split-tile partial scores
constexpr int LDS_CTL = 16;
constexpr int LDS_BYTES = LDS_Q + LDS_SLOT + LDS_PART + LDS_FIN + LDS_XS + LDS_CTL;

struct Args {
    const uint16_t *K;
    const uint16_t *Q;
    float *scores;
    int64_t T;
    int W, G, L, Hkv, Hq, R;
    int NT, NT0, X;     // tiles per row, base tiles (< 3*NWAVE), split tiles per row
    int NWG, MD;        // workgroups; mergers per query row (NWAVE / 128)
    float c2;
    unsigned long long *P1;   // [RING][NWG][128] workgroup log-sum-exp words
    unsigned long long *P2;   // [RING][128] merged words
    unsigned *ctl;            // [0] status (0 ok), [1] abort
    long long wait_ticks;     // realtime ticks (100 MHz) one wait may last
    int no_merge;             // diagnostics: the merge duty publishes nothing
};

__device__ __forceinline__ unsigned long long ll_word(float v, unsigned tag) {
    return ((unsigned long long)tag << 32) | __float_as_uint(v);
}
__device__ __forceinline__ void ll_store(unsigned long long *p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ll_load(const unsigned long long *p) {
    return __hip_atomic_load(const_cast<unsigned long long *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ll_tag(unsigned long long w) { return (unsigned)(w >> 32); }
__device__ __forceinline__ float ll_val(unsigned long long w) { return __uint_as_float((unsigned)w); }

__device__ __forceinline__ bool aborted(const Args &a) {
    return __hip_atomic_load(a.ctl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}
__device__ __forceinline__ void give_up(const Args &a, unsigned code) {
    __hip_atomic_store(a.ctl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.ctl + 0, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Full-wave reductions (every lane gets the result).
__device__ __forceinline__ float wave_max(float v) { return xor32_max(xor16_max(group_max<16>(v))); }
__device__ __forceinline__ float wave_sum(float v) { return xor32_sum(xor16_sum(group_sum<16>(v))); }

// Which 32-key tiles a wave owns in row i: base tile k is gw + k*NWAVE when
// below NT0; the split tile (NT0 + e) goes to workgroup c when
// e = (c - i*X) mod NWG is below X, and each of its waves takes one query block.
struct RowTiles {
    int base[TPW];
    int split;   // tile index or -1
};
__device__ __forceinline__ RowTiles row_tiles(const Args &a, int i, int c, int gw) {
    RowTiles r;
    const int nwave = a.NWG * WAVES;
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        const int t = gw + k * nwave;
        r.base[k] = t < a.NT0 ? t : -1;
    }
    r.split = -1;
    if (a.X > 0) {
        const int off = (int)(((int64_t)i * a.X) % a.NWG);
        const int e = (c - off + a.NWG) % a.NWG;
        if (e < a.X) r.split = a.NT0 + e;
    }
    return r;
}

// Keys of tile t of row i: lane l loads key 32t + (l & 31), dims 8*(l >> 5) +
// 16 s; keys at or past T read key T-1 (masked later). With t < 0 (no tile)
// every lane reads the same 16 bytes instead: the same eight load
// instructions are issued either way, so the compiler counts the loads in
// flight exactly and waits for a tile without draining the later ones.
__device__ __forceinline__ void load_tile(const Args &a, int i, int t, int lane, bf16x8 (&kf)[S]) {
    int64_t key = (int64_t)t * 32 + (lane & 31);
    if (key >= a.T) key = a.T - 1;
    const uint16_t *p = a.K + ((size_t)i * a.T + key) * D + 8 * (lane >> 5);
    const int step = t >= 0 ? 16 : 0;
    if (t < 0) p = a.K;
#pragma unroll
    for (int s = 0; s < S; ++s) kf[s] = load8(p + step * s);
}

// Window queries of row i (G*W = 128 rows, qr = g*W + w).
__device__ __forceinline__ const uint16_t *row_queries(const Args &a, int i) {
    const RowIdx ri = split_row(i, a.L, a.Hkv);
    return a.Q + ((size_t)(ri.n * a.L + ri.l) * a.Hq + (size_t)ri.h * a.G) * a.W * D;
}

// Fragment entry e of the staged queries: the 16 bytes lane (e & 63) feeds
// for block b, k-step s, where (b*S + s) = e >> 6.
__device__ __forceinline__ uint4 query_entry(const uint16_t *Qg, int e) {
    const int lane = e & 63, bs = e >> 6, s = bs % S, b = bs / S;
    const int qr = b * 32 + (lane & 31);
    return *reinterpret_cast<const uint4 *>(Qg + (size_t)qr * D + 16 * s + 8 * (lane >> 5));
}

// One row's kept state of one lane: e of base tiles k (entries 8k + 2b, 8k +
// 2b + 1: 16 fp16 of block b), references (entry 24: tiles 0, 1 as int16
// pairs; entry 25: tile 2 and the split tile), split-tile exponentials
// (entries 26, 27).
struct RegSlot {
    uint4 v[SLOT_V];
};

template <bool IN_LDS>
struct SlotRef;

template <>
struct SlotRef<false> {
    RegSlot &s;
    __device__ __forceinline__ uint4 get(int j) const { return s.v[j]; }
    __device__ __forceinline__ void put(int j, uint4 x) { s.v[j] = x; }
};

template <>
struct SlotRef<true> {
    uint4 *base;   // entry j of this lane at base[j * 64]
    __device__ __forceinline__ uint4 get(int j) const { return base[j * 64]; }
    __device__ __forceinline__ void put(int j, uint4 x) { base[j * 64] = x; }
};

__device__ __forceinline__ unsigned pack_ref(int a, int b) {
    return ((unsigned)a & 0xffffu) | ((unsigned)b << 16);
}
__device__ __forceinline__ int ref_lo(unsigned w) { return (int)(short)(w & 0xffffu); }
__device__ __forceinline__ int ref_hi(unsigned w) { return (int)(short)(w >> 16); }

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ unsigned pk_f16(float x, float y) {
    const half2_t h = {(_Float16)x, (_Float16)y};   // v_cvt_pk_f16_f32: round to nearest even
    return __builtin_bit_cast(unsigned, h);
}
__device__ __forceinline__ float lo_f16(unsigned w) { return (float)__builtin_bit_cast(half2_t, w)[0]; }
__device__ __forceinline__ float hi_f16(unsigned w) { return (float)__builtin_bit_cast(half2_t, w)[1]; }

// Running (M, l) of one lane and block: l = sum of exp2(x - M) with integer M.
__device__ __forceinline__ void fold_stats(int &M, float &l, int m, float s) {
    const int d = m - M;
    l = d > 0 ? __builtin_ldexpf(l, -d) + s : l + __builtin_ldexpf(s, d);
    M = d > 0 ? m : M;
}

// Logits of block b of a tile into acc (C[key][qrow]); masked entries -inf.
template <bool MASKED>
__device__ __forceinline__ f32x16 block_logits(const bf16x8 (&kf)[S], const uint4 *sq, int b, int lane, int qoff,
                                               int64_t j0, const Args &a) {
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const bf16x8 qf = __builtin_bit_cast(bf16x8, sq[(b * S + s) * 64 + qoff]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf, acc, 0, 0, 0);
    }
    if (MASKED) {
        // key j0 + acc_row(i, hf) is visible to query row qr = g*W + w when
        // it is at most T - W + w and below T
        const int hf = lane >> 5, col = lane & 31;
        const int w = (b * 32 + col) % a.W;
        const int64_t lim = a.T - a.W + w;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (j0 + acc_row(i, hf) > lim) acc[i] = -INFINITY;
    }
    return acc;
}

// Exponentials of one block against its integer reference: returns the
// reference and the 8 packed fp16 words; adds the block to (M, l).
__device__ __forceinline__ int block_exps(const f32x16 &acc, float c2, uint4 &lo, uint4 &hi, int &M, float &l) {
    float mx = acc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, acc[i]);
    int m = REF_EMPTY;
    if (mx > -INFINITY) {
        const float c = ceilf(mx * c2);
        m = (int)fminf(fmaxf(c, (float)(REF_EMPTY + 1)), 30000.f);
    }
    const float mf = (float)m;
    float e[16];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        e[i] = __builtin_amdgcn_exp2f(fmaf(acc[i], c2, -mf));
        s += e[i];
    }
    lo = make_uint4(pk_f16(e[0], e[1]), pk_f16(e[2], e[3]), pk_f16(e[4], e[5]), pk_f16(e[6], e[7]));
    hi = make_uint4(pk_f16(e[8], e[9]), pk_f16(e[10], e[11]), pk_f16(e[12], e[13]), pk_f16(e[14], e[15]));
    fold_stats(M, l, m, s);
    return m;
}

// A base tile: all four blocks; e into the slot entries 8k .. 8k+7.
template <bool MASKED, typename Slot>
__device__ __forceinline__ void base_tile(const Args &a, const bf16x8 (&kf)[S], const uint4 *sq, int lane, int qoff,
                                          int64_t j0, int k, Slot &slot, int (&refs)[NB], int (&M)[NB],
                                          float (&l)[NB]) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const f32x16 acc = block_logits<MASKED>(kf, sq, b, lane, qoff, j0, a);
        uint4 lo, hi;
        refs[b] = block_exps(acc, a.c2, lo, hi, M[b], l[b]);
        slot.put(8 * k + 2 * b, lo);
        slot.put(8 * k + 2 * b + 1, hi);
    }
}

// Transposing sum over the 32 lanes of a half-wave: lane (h, c) holds v[0..15]
// (keys i of its half); on return lanes with c even hold, for key index
// i = c >> 1, the sum over the 32 lanes (lanes c and c+1 hold the same).
__device__ __forceinline__ float transpose_sum16(float (&v)[16], int lane) {
    // xor 16 through the row swap: x + y is own + partner for the half kept
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[j]), __float_as_uint(v[j + 8]), false, false);
        v[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    // lanes of row 0 now hold keys 0..7, of row 1 keys 8..15; halve within rows
    const bool b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1, b1 = (lane >> 1) & 1;
    float u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float keep = b3 ? v[j + 4] : v[j];
        const float send = b3 ? v[j] : v[j + 4];
        u[j] = keep + dpp_f<0x140>(send);   // row_mirror: lane 15 - x, bit 3 flipped
    }
    float t2[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const float keep = b2 ? u[j + 2] : u[j];
        const float send = b2 ? u[j] : u[j + 2];
        t2[j] = keep + dpp_f<0x141>(send);  // row_half_mirror: lane 7 - x, bit 2 flipped
    }
    const float keep = b1 ? t2[1] : t2[0];
    const float send = b1 ? t2[0] : t2[1];
    float r = keep + dpp_f<0x4E>(send);     // quad_perm [2,3,0,1]: bit 1 flipped
    return r + dpp_f<0xB1>(r);              // quad_perm [1,0,3,2]: bit 0 flipped
}

// Finishes a base tile: score of each key = sum over blocks of e * exp2(m - LSE).
template <typename Slot>
__device__ __forceinline__ void finish_base(const Args &a, float *out, int64_t j0, int k, const Slot &slot,
                                            const int (&refs)[NB], const float (&f)[NB], const int (&n)[NB],
                                            int lane) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const float c = __builtin_ldexpf(f[b], refs[b] - n[b]);
        const uint4 lo = slot.get(8 * k + 2 * b), hi = slot.get(8 * k + 2 * b + 1);
        const unsigned w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v[2 * j] = fmaf(lo_f16(w[j]), c, v[2 * j]);
            v[2 * j + 1] = fmaf(hi_f16(w[j]), c, v[2 * j + 1]);
        }
    }
    const float r = transpose_sum16(v, lane);
    const int hf = lane >> 5, cc = lane & 31;
    const int64_t key = j0 + acc_row(cc >> 1, hf);
    if (!(cc & 1) && key < a.T) out[key] = r;
}

// The split tile of one wave (its block b = wave): partial sums over the
// block's 32 query rows of the tile's keys, into xs[key slot].
template <typename Slot>
__device__ __forceinline__ void finish_split(const Slot &slot, int ref, float f, int n, int lane, float *xs) {
    const float c = __builtin_ldexpf(f, ref - n);
    const uint4 lo = slot.get(26), hi = slot.get(27);
    const unsigned w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    float v[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        v[2 * j] = lo_f16(w[j]) * c;
        v[2 * j + 1] = hi_f16(w[j]) * c;
    }
    const float r = transpose_sum16(v, lane);
    const int hf = lane >> 5, cc = lane & 31;
    if (!(cc & 1)) xs[acc_row(cc >> 1, hf)] = r;
}

// Bounded wait helper: true while the deadline has not passed.
__device__ __forceinline__ bool keep_waiting(const Args &a, long long t0) {
    return (long long)__builtin_amdgcn_s_memrealtime() - t0 < a.wait_ticks && !aborted(a);
}

// Merge duty: wave gw owns query row q = gw / MD of the rows j with j % MD ==
// gw % MD. issue() loads the NWG workgroup words of (j, q) into registers;
// check() (a later point, so the loads are back) merges and publishes them
// when every tag says row j, and reports whether it did.
struct Merge {
    unsigned long long w[NWG_MAX / 64];
    int j;
    bool due, done;

    // Always issues the same loads (the first exchange word when there is
    // nothing to load), so the loads in flight stay countable.
    __device__ __forceinline__ void issue(const Args &a, int q, int lane) {
        const bool live = due && !done;
        const unsigned long long *src = a.P1 + ((size_t)((live ? j : 0) % RING) * a.NWG) * 128 + (live ? q : 0);
#pragma unroll
        for (int k = 0; k < NWG_MAX / 64; ++k) {
            const int c = lane + 64 * k;
            w[k] = ll_load(src + (live && c < a.NWG ? (size_t)c * 128 : 0));
        }
    }
    __device__ __forceinline__ void check(const Args &a, int q, int lane) {
        if (!due || done) return;
        const unsigned tag = (unsigned)j + 1u;
        bool ok = true;
        float v[NWG_MAX / 64];
#pragma unroll
        for (int k = 0; k < NWG_MAX / 64; ++k) {
            const bool real = lane + 64 * k < a.NWG;   // lanes past the workgroups hold a dummy word
            ok &= !real || ll_tag(w[k]) == tag;
            v[k] = real ? ll_val(w[k]) : -INFINITY;
        }
        if (__builtin_amdgcn_ballot_w64(!ok) != 0) return;
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < NWG_MAX / 64; ++k) mx = fmaxf(mx, v[k]);
        mx = wave_max(mx);
        float s = 0.f;
        if (mx > -INFINITY) {
#pragma unroll
            for (int k = 0; k < NWG_MAX / 64; ++k)
                if (v[k] > -INFINITY) s += __builtin_amdgcn_exp2f(v[k] - mx);
        }
        s = wave_sum(s);
        const float lse = mx > -INFINITY ? mx + __builtin_amdgcn_logf(s) : -INFINITY;
        if (lane == 0) ll_store(a.P2 + (size_t)(j % RING) * 128 + q, ll_word(lse, tag));
        done = true;
    }
};

// Fetch of row j's 128 merged values (wave 1 of each workgroup) into fin.
struct Fetch {
    unsigned long long w0, w1;
    int j;
    bool due, done;

    __device__ __forceinline__ void issue(const Args &a, int lane) {
        const bool live = due && !done;
        const unsigned long long *src = a.P2 + (size_t)((live ? j : 0) % RING) * 128;
        w0 = ll_load(src + (live ? lane : 0));
        w1 = ll_load(src + (live ? lane + 64 : 0));
    }
    __device__ __forceinline__ void check(int lane, float *fin) {
        if (!due || done) return;
        const unsigned tag = (unsigned)j + 1u;
        const bool ok = ll_tag(w0) == tag && ll_tag(w1) == tag;
        if (__builtin_amdgcn_ballot_w64(!ok) != 0) return;
        fin[lane] = ll_val(w0);
        fin[lane + 64] = ll_val(w1);
        done = true;
    }
};

// Per-lane state carried through a row.
struct RowState {
    int M[NB];
    float l[NB];
    int refs[TPW][NB];
    int xref;
};

__device__ __forceinline__ void reset_stats(RowState &st) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        st.M[b] = M_EMPTY;
        st.l[b] = 0.f;
    }
}

template <typename Slot>
__device__ __forceinline__ void store_refs(Slot &slot, const RowState &st) {
    slot.put(24, make_uint4(pack_ref(st.refs[0][0], st.refs[0][1]), pack_ref(st.refs[0][2], st.refs[0][3]),
                            pack_ref(st.refs[1][0], st.refs[1][1]), pack_ref(st.refs[1][2], st.refs[1][3])));
    slot.put(25, make_uint4(pack_ref(st.refs[2][0], st.refs[2][1]), pack_ref(st.refs[2][2], st.refs[2][3]),
                            (unsigned)st.xref, 0u));
}

template <typename Slot>
__device__ __forceinline__ void load_refs(const Slot &slot, int (&refs)[TPW][NB], int &xref) {
    const uint4 r0 = slot.get(24), r1 = slot.get(25);
    const unsigned w[6] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y};
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        refs[k][0] = ref_lo(w[2 * k]);
        refs[k][1] = ref_hi(w[2 * k]);
        refs[k][2] = ref_lo(w[2 * k + 1]);
        refs[k][3] = ref_hi(w[2 * k + 1]);
    }
    xref = (int)r1.z;
}

// Everything a wave carries from row to row.
struct Carry {
    bf16x8 kb0[S], kb1[S];   // key tiles: positions 0 and 2 use kb0, positions 1 and 3 kb1
    uint4 qst[8];            // the next row's query fragments, staged in registers
    Merge mg;
    Fetch ft;
};

struct Lds {
    uint4 *sq, *sslot;
    float2 *spart;
    float *sfin, *sxs;
    int *sctl;
};

// One row step i: the tiles of row i (when i < R) into slot `cur`, the merge
// duty of row i-1, the publication of row i, and the finished scores of row
// i-2 from slot `fin`. Returns false when the call gave up (every wave of the
// workgroup returns false together).
template <typename SlotCur, typename SlotFin>
__device__ __forceinline__ bool row_step(const Args &a, int i, SlotCur &cur, SlotFin &fin, Carry &cy, const Lds &m,
                                         int c, int wave, int lane, int gw, int qoff) {
    const int tid = wave * 64 + lane, col = lane & 31, hf = lane >> 5;
    const int mq = gw / a.MD, mphase = gw % a.MD;
    const bool has_row = i < a.R;
    const bool has_next = i + 1 < a.R;
    RowState st;
    reset_stats(st);
#pragma unroll
    for (int k = 0; k < TPW; ++k)
#pragma unroll
        for (int b = 0; b < NB; ++b) st.refs[k][b] = REF_EMPTY;
    st.xref = REF_EMPTY;
    cy.mg.j = i - 1;
    cy.mg.due = i >= 1 && i - 1 < a.R && (i - 1) % a.MD == mphase && mq < 128 && !a.no_merge;
    cy.mg.done = false;
    cy.ft.j = i - 2;
    cy.ft.due = wave == 1 && i >= 2 && i - 2 < a.R;
    cy.ft.done = false;
    float *fin_row = m.sfin + ((i - 2) & 1) * 128;
    unsigned abort_word = 0u;

    if (has_row) {
        const RowTiles rt = row_tiles(a, i, c, gw);
        const RowTiles rn = row_tiles(a, has_next ? i + 1 : i, c, gw);
        // position 0
        load_tile(a, i, rt.base[1], lane, cy.kb1);
        if (rt.base[0] >= 0)
            base_tile<false>(a, cy.kb0, m.sq, lane, qoff, 32 * (int64_t)rt.base[0], 0, cur, st.refs[0], st.M, st.l);
        // hook A: the next row's queries, first attempts of the duties
        {
            const uint16_t *Qn = row_queries(a, has_next ? i + 1 : i);
#pragma unroll
            for (int k = 0; k < 8; ++k) cy.qst[k] = query_entry(Qn, tid + THREADS * k);
        }
        cy.mg.issue(a, mq, lane);
        cy.ft.issue(a, lane);
        // position 1
        load_tile(a, i, rt.base[2], lane, cy.kb0);
        if (rt.base[1] >= 0)
            base_tile<false>(a, cy.kb1, m.sq, lane, qoff, 32 * (int64_t)rt.base[1], 1, cur, st.refs[1], st.M, st.l);
        // hook B
        cy.mg.check(a, mq, lane);
        cy.mg.issue(a, mq, lane);
        cy.ft.check(lane, fin_row);
        cy.ft.issue(a, lane);
        // position 2
        load_tile(a, i, rt.split, lane, cy.kb1);
        if (rt.base[2] >= 0)
            base_tile<false>(a, cy.kb0, m.sq, lane, qoff, 32 * (int64_t)rt.base[2], 2, cur, st.refs[2], st.M, st.l);
        // hook C (and the abort word, looked at the row's end)
        cy.mg.check(a, mq, lane);
        cy.mg.issue(a, mq, lane);
        cy.ft.check(lane, fin_row);
        cy.ft.issue(a, lane);
        abort_word = __hip_atomic_load(a.ctl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // position 3: this wave's query block of the split tile
        load_tile(a, has_next ? i + 1 : i, has_next ? rn.base[0] : -1, lane, cy.kb0);
        if (rt.split >= 0) {
            const f32x16 acc = block_logits<true>(cy.kb1, m.sq, wave, lane, qoff, 32 * (int64_t)rt.split, a);
            uint4 lo, hi;
            int Mw = M_EMPTY;
            float lw = 0.f;
            st.xref = block_exps(acc, a.c2, lo, hi, Mw, lw);
            // fold into this wave's block (static indices: the block is the wave)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b == wave) fold_stats(st.M[b], st.l[b], Mw, lw);
            cur.put(26, lo);
            cur.put(27, hi);
        }
        store_refs(cur, st);
    }
    // the duties still open wait here, each at most wait_ticks
    bool ok = true;
    // the loads this row's last hook issued first (a step without tiles had no
    // hooks: its registers hold other words), then (rarely) bounded retries
    if (has_row) {
        cy.mg.check(a, mq, lane);
        cy.ft.check(lane, fin_row);
    }
    if (cy.mg.due && !cy.mg.done) {
        const long long t0 = (long long)__builtin_amdgcn_s_memrealtime();
        do {
            __builtin_amdgcn_s_sleep(2);
            cy.mg.issue(a, mq, lane);
            cy.mg.check(a, mq, lane);
        } while (!cy.mg.done && keep_waiting(a, t0));
        ok &= cy.mg.done;
    }
    if (cy.ft.due && !cy.ft.done) {
        const long long t0 = (long long)__builtin_amdgcn_s_memrealtime();
        do {
            __builtin_amdgcn_s_sleep(2);
            cy.ft.issue(a, lane);
            cy.ft.check(lane, fin_row);
        } while (!cy.ft.done && keep_waiting(a, t0));
        ok &= cy.ft.done;
    }
    if (!ok) {
        if (lane == 0) give_up(a, 1u);
        if (lane == 0) m.sctl[0] = 1;
    }
    // this wave's statistics per query row: lanes c and c+32 hold the same row
    if (has_row) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int Mo = __shfl_xor(st.M[b], 32);
            const float lo = __shfl_xor(st.l[b], 32);
            const int Mx = max(st.M[b], Mo);
            const float ls = __builtin_ldexpf(st.l[b], st.M[b] - Mx) + __builtin_ldexpf(lo, Mo - Mx);
            if (hf == 0) m.spart[wave * 128 + b * 32 + col] = make_float2(__int_as_float(Mx), ls);
        }
    }
    if (tid == 0 && abort_word != 0u) m.sctl[0] = 1;
    __syncthreads();
    if (m.sctl[0]) return false;
    // publish row i: one log-sum-exp per query row for this workgroup
    if (has_row && tid < 128) {
        int Mx = M_EMPTY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) Mx = max(Mx, __float_as_int(m.spart[w * 128 + tid].x));
        float ls = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float2 p = m.spart[w * 128 + tid];
            ls += __builtin_ldexpf(p.y, __float_as_int(p.x) - Mx);
        }
        const float lse = ls > 0.f ? (float)Mx + __builtin_amdgcn_logf(ls) : -INFINITY;
        ll_store(a.P1 + ((size_t)(i % RING) * a.NWG + c) * 128 + tid, ll_word(lse, (unsigned)i + 1u));
    }
    // the next row's queries replace this row's
    if (has_next) {
#pragma unroll
        for (int k = 0; k < 8; ++k) m.sq[tid + THREADS * k] = cy.qst[k];
    }
    // finish row i-2
    const int i2 = i - 2;
    RowTiles r2;
    r2.split = -1;
    if (i2 >= 0 && i2 < a.R) {
        r2 = row_tiles(a, i2, c, gw);
        int refs[TPW][NB], xref;
        load_refs(fin, refs, xref);
        float f[NB];
        int n[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float lse = fin_row[b * 32 + col];
            const float fl = floorf(lse);
            n[b] = (int)fminf(fmaxf(fl, -60000.f), 60000.f);
            f[b] = lse > -INFINITY ? __builtin_amdgcn_exp2f(fl - lse) : 0.f;
        }
        float *out = a.scores + (size_t)i2 * a.T;
#pragma unroll
        for (int k = 0; k < TPW; ++k)
            if (r2.base[k] >= 0) finish_base(a, out, 32 * (int64_t)r2.base[k], k, fin, refs[k], f, n, lane);
        if (r2.split >= 0) {
            float fw = 0.f;
            int nw = 0;
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b == wave) {
                    fw = f[b];
                    nw = n[b];
                }
            finish_split(fin, xref, fw, nw, lane, m.sxs + ((i2 & 1) * WAVES + wave) * 32);
        }
    }
    __syncthreads();
    if (r2.split >= 0 && wave == 0 && lane < 32) {
        const int64_t key = 32 * (int64_t)r2.split + lane;
        const float *xs = m.sxs + (i2 & 1) * WAVES * 32;
        if (key < a.T) a.scores[(size_t)i2 * a.T + key] = ((xs[lane] + xs[32 + lane]) + xs[64 + lane]) + xs[96 + lane];
    }
    return true;
}

__global__ void __launch_bounds__(THREADS, 1) score_once_kernel(Args a) {
    extern __shared__ uint4 lds[];
    Lds m;
    m.sq = lds;
    m.sslot = lds + LDS_Q / 16;
    m.spart = reinterpret_cast<float2 *>(m.sslot + LDS_SLOT / 16);
    m.sfin = reinterpret_cast<float *>(m.spart + WAVES * 128);
    m.sxs = m.sfin + 2 * 128;
    m.sctl = reinterpret_cast<int *>(m.sxs + 2 * WAVES * 32);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = blockIdx.x, gw = c * WAVES + wave;
    int qoff = lane;
    asm volatile("" : "+v"(qoff));   // keeps the query-fragment LDS reads inside the tile loops

    RegSlot rs0, rs1;
    SlotRef<false> s0{rs0}, s1{rs1};
    SlotRef<true> s2{m.sslot + (wave * SLOT_V) * 64 + lane};
    Carry cy;

    if (tid == 0) m.sctl[0] = 0;
    {
        const uint16_t *Qg = row_queries(a, 0);
        for (int e = tid; e < 4 * S * 64; e += THREADS) m.sq[e] = query_entry(Qg, e);
    }
    const RowTiles r0 = row_tiles(a, 0, c, gw);
    if (r0.base[0] >= 0) load_tile(a, 0, r0.base[0], lane, cy.kb0);
    __syncthreads();
    // rows i, i+1, i+2 use slots 0, 1, 2; row i-2's slot is finished at step i
    for (int i = 0; i < a.R + 2; i += 3) {
        if (!row_step(a, i, s0, s1, cy, m, c, wave, lane, gw, qoff)) return;
        if (i + 1 >= a.R + 2) break;
        if (!row_step(a, i + 1, s1, s2, cy, m, c, wave, lane, gw, qoff)) return;
        if (i + 2 >= a.R + 2) break;
        if (!row_step(a, i + 2, s2, s0, cy, m, c, wave, lane, gw, qoff)) return;
    }
}

__global__ void clear_words(unsigned long long *p, size_t n, unsigned *ctl) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (size_t k = i; k < n; k += (size_t)gridDim.x * blockDim.x) p[k] = 0ull;
    if (i < 4) ctl[i] = 0u;
}

// ---------------------------------------------------------------- host side

struct DevInfo {
    int cus = 0, coop = 0, occ = 0;
    bool ok = false;
};
static std::mutex g_info_mu;
static std::vector<DevInfo> g_info;

static DevInfo device_info() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DevInfo{};
    std::lock_guard<std::mutex> lock(g_info_mu);
    if ((size_t)dev >= g_info.size()) g_info.resize((size_t)dev + 1);
    DevInfo &d = g_info[dev];
    if (!d.ok) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DevInfo{};
        d.cus = prop.multiProcessorCount;
        if (hipDeviceGetAttribute(&d.coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess) d.coop = 0;
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(&score_once_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES) != hipSuccess)
            return DevInfo{};
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&d.occ, score_once_kernel, THREADS, LDS_BYTES) !=
            hipSuccess)
            d.occ = 0;
        d.ok = true;
    }
    return d;
}

// Workgroups the kernel runs with on this device: one per CU, a multiple of
// 32 (so NWAVE / 128 mergers per query row is whole), at most NWG_MAX.
static int plan_workgroups(const DevInfo &d) {
    if (!d.ok || !d.coop || d.occ < 1) return 0;
    int n = d.cus < NWG_MAX ? d.cus : NWG_MAX;
    return (n / 32) * 32;
}

}  // namespace once

static long long g_wait_us = 200000;   // every wait of the single-read kernel, microseconds
static bool g_no_merge = false;        // diagnostics: mergers publish nothing, so every fetch runs out

int score_once_plan(const kvc_dims *d, int W, size_t *ws_bytes) {
    const int G = d->n_q_heads / d->n_kv_heads;
    const int64_t T = d->n_tokens, rows = n_rows(d);
    if (d->head_dim != once::D || G * W != 128 || rows < 1 || rows > (1 << 24)) return 0;
    if (T < 32768) return 0;    // short rows: the per-row exchange would dominate
    const once::DevInfo info = once::device_info();
    const int nwg = once::plan_workgroups(info);
    if (nwg < 32) return 0;
    const int64_t nt = (T + 31) / 32;
    const int64_t nt0 = std::min<int64_t>((int64_t)3 * nwg * once::WAVES, (T - W + 1) / 32);
    if (nt - nt0 > nwg || nt0 < 1) return 0;
    *ws_bytes = 256 + ((size_t)once::RING * nwg * 128 + (size_t)once::RING * 128) * sizeof(unsigned long long);
    return nwg;
}

int launch_score_once(const kvc_dims *d, const uint16_t *K, const uint16_t *Q, int W, float *scores, void *ws,
                      int nwg, hipStream_t s) {
    once::Args a;
    a.K = K;
    a.Q = Q;
    a.scores = scores;
    a.T = d->n_tokens;
    a.W = W;
    a.G = d->n_q_heads / d->n_kv_heads;
    a.L = d->n_layers;
    a.Hkv = d->n_kv_heads;
    a.Hq = d->n_q_heads;
    a.R = (int)n_rows(d);
    a.NT = (int)((a.T + 31) / 32);
    a.NT0 = (int)std::min<int64_t>((int64_t)3 * nwg * once::WAVES, (a.T - W + 1) / 32);
    a.X = a.NT - a.NT0;
    a.NWG = nwg;
    a.MD = nwg * once::WAVES / 128;
    a.c2 = (float)(1.4426950408889634 / std::sqrt((double)d->head_dim));
    a.ctl = reinterpret_cast<unsigned *>(ws);
    a.P1 = reinterpret_cast<unsigned long long *>(reinterpret_cast<char *>(ws) + 256);
    a.P2 = a.P1 + (size_t)once::RING * nwg * 128;
    a.wait_ticks = g_wait_us * 100;   // s_memrealtime runs at 100 MHz
    a.no_merge = g_no_merge ? 1 : 0;
    const size_t nwords = (size_t)once::RING * nwg * 128 + (size_t)once::RING * 128;
    once::clear_words<<<dim3(256), dim3(256), 0, s>>>(a.P1, nwords, a.ctl);
    int st = check_launch("kvc_score: clear exchange words");
    if (st != KVC_OK) return st;
    void *args[] = {&a};
    const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(&once::score_once_kernel),
                                                    dim3(nwg), dim3(once::THREADS), args, once::LDS_BYTES, s);
    if (e != hipSuccess) return fail(KVC_ERR_HIP, "kvc_score: cooperative launch failed: %s", hipGetErrorString(e));
    return check_launch("kvc_score single-read kernel");
}

void set_score_wait(int64_t wait_us, bool no_merge) {
    g_wait_us = wait_us;
    g_no_merge = no_merge;
}

}  // namespace kvc
