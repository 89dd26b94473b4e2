// kvc_score: observation-window attention score.
//
// Per row (sequence, layer, KV head) the G*W window queries of the GQA group
// (query row qr = g*W + w at position qbase+w, qbase = T-W) attend causally to
// the cached keys; the score of key j is the sum over query rows of its softmax
// weight (PASK §3.1 Eq. 1 attention, window queries as in CommitKV §3.1 Eq. 5,
// causal rule of CommitKV Eq. 6).
//
// A softmax weight needs its query row's normaliser over all keys, so the keys
// are read twice: pass 1 gives every query row a reference r and its exp-sum
// sum_j exp2(logit*c - r) (log2 domain) chunk by chunk, a merge folds the
// chunks into mm[qr] = r + log2(sum), and pass 2 recomputes the logits and
// writes score[j] = sum_qr exp2(logit*c - mm[qr]).
//
// kvc_score launches pass 1 (one workgroup per row and STATS_CHUNK keys), the
// merge (one workgroup per row) and pass 2 (same grid as pass 1).
//
// Tiles. A workgroup has four waves; each wave owns whole 32-key tiles of the
// chunk (tiles w, w+4, ...), so each key is loaded once, straight into MFMA operand registers. The
// row's window queries are staged in LDS in MFMA fragment order (entry
// (b*S + s)*64 + lane is the 16-byte slice lane `lane` feeds for query block
// b, k-step s) and read back with conflict-free 16-byte loads.
//
// Logits come from v_mfma_f32_32x32x16_bf16. Lane l holds key (l & 31), dims
// 8*(l>>5)..+8 of each 16-dim slice; that layout is the A operand (rows = keys)
// in pass 1 and the B operand (columns = keys) in pass 2. Pass 1 computes
// C[key][qrow] (a lane owns one query row: its reference and sum stay in-lane);
// pass 2 computes C[qrow][key] (a lane owns one key: the sum over query rows
// stays in-lane).
#include <cmath>
#include <mutex>
#include <vector>

#include "kvc_internal.h"

namespace kvc {

static constexpr int SCORE_WAVES = 4;  // waves per workgroup
static constexpr int SCORE_THREADS = SCORE_WAVES * 64;
static constexpr int SCORE_MAX_QR = 256;  // query rows per row (8 blocks of 32)
#ifndef KVC_STATS_CHUNK
#define KVC_STATS_CHUNK 4096
#endif
static constexpr int STATS_CHUNK = KVC_STATS_CHUNK;  // keys per workgroup of both passes

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t window_chunks(int64_t kend) { return (kend + STATS_CHUNK - 1) / STATS_CHUNK; }

// kvc_score workspace: a 256-byte control block (word 0: the call's status),
// then either path's scratch: the two passes' chunk partials [rows][QRP][n_chunks]
// and merged normalisers [rows][QRP], or the single-read kernel's exchange words.
static size_t two_pass_bytes(const kvc_dims *d, int32_t W) {
    const int G = d->n_q_heads / d->n_kv_heads;
    const int QRP = ((G * W + 31) / 32) * 32;
    const int64_t rows = n_rows(d);
    const int64_t nch = window_chunks(d->n_tokens);
    return align256((size_t)rows * nch * QRP * sizeof(float2)) + align256((size_t)rows * QRP * sizeof(float));
}

static bool g_single_read = false;  // kvc_score_options (the single-read kernel measured slower)

// Covers both paths (whichever kvc_score_options selects when the call runs).
size_t score_workspace_bytes(const kvc_dims *d, int32_t W) {
    size_t once_bytes = 0;
    const size_t two = two_pass_bytes(d, W) + 256;
    if (score_once_plan(d, W, &once_bytes) > 0 && once_bytes > two) return once_bytes;
    return two;
}

// Stage the row's queries in fragment order (zero rows beyond QR).
template <int D, int NB>
__device__ __forceinline__ void stage_queries(const uint16_t *Qg, int QR, uint4 *sq) {
    constexpr int S = D / 16;
    for (int e = threadIdx.x; e < NB * S * 64; e += SCORE_THREADS) {
        const int lane = e & 63, bs = e >> 6, s = bs % S, b = bs / S;
        const int qr = b * 32 + (lane & 31);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (qr < QR) v = *reinterpret_cast<const uint4 *>(Qg + (size_t)qr * D + 16 * s + 8 * (lane >> 5));
        sq[e] = v;
    }
}

template <int S>
__device__ __forceinline__ void load_key_tile(const uint16_t *Kr, int64_t key, int64_t kend, int hf, bf16x8 *kf) {
    constexpr int D = S * 16;
#pragma unroll
    for (int s = 0; s < S; ++s) kf[s] = key < kend ? load8(Kr + (size_t)key * D + 16 * s + 8 * hf) : zero8();
}

// Loads the tile of keys [j0, j0 + 32) into registers; keys at or past kend
// read the chunk's last key instead (the tile's consumer ignores them), so
// every call issues the same loads and the next tile's loads can stay in
// flight while this one is consumed.
template <int S>
__device__ __forceinline__ void load_tile_clamped(const uint16_t *Kr, int64_t j0, int64_t kend, int lane,
                                                  bf16x8 (&kf)[S]) {
    constexpr int D = S * 16;
    int64_t key = j0 + (lane & 31);
    if (key >= kend) key = kend - 1;
    key = KVC_IDX(key, kend, KVC_CHK_SCORE);
    const uint16_t *p = Kr + (size_t)key * D + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < S; ++s) kf[s] = load8(p + 16 * s);
}

// Number of tiles of [k0, k0 + 32*ntiles) whose last key is <= qbase (visible
// to every query row).
__device__ __forceinline__ int visible_tiles(int64_t k0, int64_t qbase, int ntiles) {
    const int64_t v = qbase + 1 - k0 >= 0 ? (qbase + 1 - k0) / 32 : 0;
    return v < ntiles ? (int)v : ntiles;
}

// ---------------------------------------------------------------- pass 1

// One 32-key tile (in registers) for every query block: running (reference,
// exp-sum) per query row (this lane's query row is b*32 + col of block b).
// The reference m need not be the running max: any m with every term
// exp2(x - m) finite gives the same normaliser m + log2(l). So a tile's terms
// are summed against the current reference first, and only when that sum is
// not below 2^64 (or is not finite: the row's first tile, or a logit well
// above the reference) does the tile take its max and rescale. The per-block
// state m[], l[] rotates by one each iteration, so block b's state is always
// at index 0 and the arrays are back in order after NB iterations; up to 7
// blocks the loop is unrolled (the rotation is then free), with 8 it stays
// rolled (static register indices, one accumulator live) so that the kernel
// fits 128 VGPRs.
template <int D, int NB, bool MASKED>
__device__ __forceinline__ void p1_tile(const bf16x8 (&kf)[D / 16], int64_t j0, int lane, const uint4 *sq,
                                        int64_t qbase, int W, int QR, float c2, float (&m)[NB], float (&l)[NB]) {
    constexpr int S = D / 16;
    const int col = lane & 31, hf = lane >> 5;
    // Re-read the queries from LDS every tile (an opaque lane offset keeps the
    // loads in the loop): holding all of them in registers would cost occupancy.
    int qoff = lane;
    asm volatile("" : "+v"(qoff));
    constexpr int UNROLL = NB <= 7 ? NB : 1;
#pragma unroll UNROLL
    for (int b = 0; b < NB; ++b) {
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const bf16x8 qf = __builtin_bit_cast(bf16x8, sq[(b * S + s) * 64 + qoff]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf, acc, 0, 0, 0);
        }
        // acc[i] = logit of key j0 + acc_row(i, hf) for query row b*32 + col
        if (MASKED) {
            // key j0 + acc_row(i, hf) is visible to query row qr when its offset
            // from qbase is at most qr % W (masked tiles lie within W + 32 keys
            // of qbase); padding query rows see no key. Comparing acc_row(i, 0)
            // against one per-lane bound keeps the offsets as inline constants.
            const int qr = b * 32 + col;
            const int lim = qr < QR ? qr % W : -(1 << 30);
            const int bound = lim - (int)(j0 - qbase) - 4 * hf;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (acc_row(i, 0) > bound) acc[i] = -INFINITY;
        }
        float mc = m[0], lc = l[0];
        float sum = __builtin_amdgcn_exp2f(fmaf(acc[0], c2, -mc));
#pragma unroll
        for (int i = 1; i < 16; ++i) sum += __builtin_amdgcn_exp2f(fmaf(acc[i], c2, -mc));
        if (!(sum <= 0x1p64f)) {
            float tmax = acc[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, acc[i]);
            tmax *= c2;
            if (tmax > mc) {
                lc *= __builtin_amdgcn_exp2f(mc - tmax);
                mc = tmax;
            }
            // A row with no visible key yet keeps m = -inf; its exponents are all -inf.
            const float mb = mc == -INFINITY ? 0.f : mc;
            sum = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) sum += __builtin_amdgcn_exp2f(fmaf(acc[i], c2, -mb));
        }
        lc += sum;
#pragma unroll
        for (int k = 0; k + 1 < NB; ++k) {
            m[k] = m[k + 1];
            l[k] = l[k + 1];
        }
        m[NB - 1] = mc;
        l[NB - 1] = lc;
    }
}

// Pass 1 over keys [k0, k1): (reference, exp-sum) of every query row q -> out[q * out_stride].
// Uses s_m/s_l (SCORE_WAVES x QRP floats each) and ends with a barrier.
template <int D, int NB>
__device__ __forceinline__ void p1_chunk(const uint16_t *Kr, int64_t k0, int64_t k1, int64_t qbase, int W, int QR,
                                         float c2, const uint4 *sq, float *s_m, float *s_l, float2 *out,
                                         int64_t out_stride) {
    constexpr int QRP = NB * 32;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, hf = lane >> 5;
    float m[NB], l[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        m[b] = -INFINITY;
        l[b] = 0.f;
    }
    const int ntiles = (int)((k1 - k0 + 31) / 32);
    const int nvis = visible_tiles(k0, qbase, ntiles);
    // tiles wave, wave+4, ...; the next tile's loads are in flight while the
    // current one is computed (keys past k1 are masked out)
    int t = wave;
    if (t < ntiles) {
        constexpr int S = D / 16;
        auto tile = [&](const bf16x8(&kf)[S], int tt) {
            if (tt < nvis)
                p1_tile<D, NB, false>(kf, k0 + 32 * tt, lane, sq, qbase, W, QR, c2, m, l);
            else
                p1_tile<D, NB, true>(kf, k0 + 32 * tt, lane, sq, qbase, W, QR, c2, m, l);
        };
        const int last = ntiles - 1;
        bf16x8 ka[S], kb[S];
        load_tile_clamped<S>(Kr, k0 + 32 * t, k1, lane, ka);
        for (;;) {
            const int t1 = t + SCORE_WAVES;
            load_tile_clamped<S>(Kr, k0 + 32 * (t1 < last ? t1 : last), k1, lane, kb);
            tile(ka, t);
            if (t1 > last) break;
            const int t2 = t1 + SCORE_WAVES;
            load_tile_clamped<S>(Kr, k0 + 32 * (t2 < last ? t2 : last), k1, lane, ka);
            tile(kb, t1);
            if (t2 > last) break;
            t = t2;
        }
    }
    // Lanes l and l^32 hold the same query row over different keys; then the
    // waves of the workgroup hold it over different tiles.
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const float mo = __shfl_xor(m[b], 32);
        const float lo = __shfl_xor(l[b], 32);
        const float M = fmaxf(m[b], mo);
        float Ls = 0.f;
        if (M > -INFINITY) Ls = l[b] * __builtin_amdgcn_exp2f(m[b] - M) + lo * __builtin_amdgcn_exp2f(mo - M);
        if (hf == 0) {
            s_m[wave * QRP + b * 32 + col] = M;
            s_l[wave * QRP + b * 32 + col] = Ls;
        }
    }
    __syncthreads();
    for (int q = threadIdx.x; q < QRP; q += SCORE_THREADS) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < SCORE_WAVES; ++w) M = fmaxf(M, s_m[w * QRP + q]);
        float Ls = 0.f;
        if (M > -INFINITY) {
#pragma unroll
            for (int w = 0; w < SCORE_WAVES; ++w)
                if (s_l[w * QRP + q] > 0.f) Ls += s_l[w * QRP + q] * __builtin_amdgcn_exp2f(s_m[w * QRP + q] - M);
        }
        out[q * out_stride] = make_float2(M, Ls);
    }
    __syncthreads();
}

// mm[q] = M + log2(S), the fold of a row's chunk partials (reference, sum)
// part[q][0..nch); padding rows get +inf (their weights exp2(x - inf) are 0). All threads of the
// workgroup take part: query row q is folded by blockDim/QRP threads, each over
// a contiguous range of chunks in one online (max, sum) pass; the ranges are
// then combined in a fixed order, so the result does not depend on timing.
__device__ __forceinline__ void fold(float &M, float &S, float m, float l) {
    if (!(l > 0.f)) return;
    if (m > M) {
        S = S * __builtin_amdgcn_exp2f(M - m) + l;
        M = m;
    } else {
        S += l * __builtin_amdgcn_exp2f(m - M);
    }
}

__device__ void merge_row(const float2 *part, int64_t nch, int QR, int QRP, float *mm, float2 *s_tmp) {
    const int groups = (int)blockDim.x / QRP;  // >= 1 (QRP <= 256 = blockDim)
    const int q = threadIdx.x % QRP, g = threadIdx.x / QRP;
    if (g < groups) {
        const int64_t per = (nch + groups - 1) / groups;
        const int64_t c0 = g * per, c1 = c0 + per < nch ? c0 + per : nch;
        const float2 *pq = part + (size_t)q * nch;
        float M = -INFINITY, S = 0.f;
        int64_t c = c0;
        for (; c + 8 <= c1; c += 8) {
            float2 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = pq[c + u];
#pragma unroll
            for (int u = 0; u < 8; ++u) fold(M, S, v[u].x, v[u].y);
        }
        for (; c < c1; ++c) fold(M, S, pq[c].x, pq[c].y);
        s_tmp[g * QRP + q] = make_float2(M, S);
    }
    __syncthreads();
    if (threadIdx.x < QRP) {
        float M = -INFINITY, S = 0.f;
        for (int gg = 0; gg < groups; ++gg) fold(M, S, s_tmp[gg * QRP + q].x, s_tmp[gg * QRP + q].y);
        mm[q] = q < QR ? M + log2f(S) : INFINITY;
    }
    __syncthreads();
}

// ---------------------------------------------------------------- pass 2

// One 32-key tile already in registers: softmax weights of every query row
// for this lane's key, summed; one query block at a time (interleaving blocks
// would hold several accumulators and fragment sets live and cost occupancy).
template <int D, int NB, bool MASKED>
__device__ __forceinline__ void p2_tile(const bf16x8 (&kf)[D / 16], int64_t j0, int64_t kend, int lane,
                                        const uint4 *sq, const float4 *s_mm, float c2, int64_t qbase, int W,
                                        float *out) {
    constexpr int S = D / 16;
    const int col = lane & 31, hf = lane >> 5;
    const int64_t key = j0 + col;
    int qoff = lane, moff = hf;  // opaque offsets keep the LDS reads inside the loop
    asm volatile("" : "+v"(qoff), "+v"(moff));
    float p = 0.f;
#pragma unroll 1
    for (int b = 0; b < NB; ++b) {
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const bf16x8 qf = __builtin_bit_cast(bf16x8, sq[(b * S + s) * 64 + qoff]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kf[s], acc, 0, 0, 0);
        }
        // acc[i] = logit of query row b*32 + acc_row(i, hf) for key `key`; rows
        // acc_row(4k..4k+3, hf) are 8k + 4hf .. +3: one float4 of normalisers each.
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            const float4 mv = s_mm[b * 8 + 2 * k4 + moff];
            const float mvs[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * k4 + e;
                float x = fmaf(acc[i], c2, -mvs[e]);
                if (MASKED) {
                    const int qr = b * 32 + acc_row(i, hf);
                    if ((int)(key - qbase) > qr % W) x = -INFINITY;
                }
                p += __builtin_amdgcn_exp2f(x);
            }
        }
    }
    p = xor32_sum(p);  // + the other half-wave's query rows (all lanes active here)
    if (hf == 0 && key < kend) out[KVC_IDX(key, kend, KVC_CHK_SCORE)] = p;
}

// Pass 2 over keys [k0, k1): each wave walks its tiles (wave, wave+4, ...)
// with the next tile's loads issued before the current tile is computed.
template <int D, int NB>
__device__ __forceinline__ void p2_chunk(const uint16_t *Kr, int64_t k0, int64_t k1, int64_t qbase, int W,
                                         float c2, const uint4 *sq, const float4 *s_mm, float *out) {
    constexpr int S = D / 16;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ntiles = (int)((k1 - k0 + 31) / 32);
    const int nvis = visible_tiles(k0, qbase, ntiles);
    int t = wave;
    if (t >= ntiles) return;
    auto tile = [&](const bf16x8(&kf)[S], int tt) {
        if (tt < nvis)
            p2_tile<D, NB, false>(kf, k0 + 32 * tt, k1, lane, sq, s_mm, c2, qbase, W, out);
        else
            p2_tile<D, NB, true>(kf, k0 + 32 * tt, k1, lane, sq, s_mm, c2, qbase, W, out);
    };
    const int last = ntiles - 1;
    bf16x8 ka[S], kb[S];
    load_tile_clamped<S>(Kr, k0 + 32 * t, k1, lane, ka);
    for (;;) {
        const int t1 = t + SCORE_WAVES;
        load_tile_clamped<S>(Kr, k0 + 32 * (t1 < last ? t1 : last), k1, lane, kb);
        tile(ka, t);
        if (t1 > last) break;
        const int t2 = t1 + SCORE_WAVES;
        load_tile_clamped<S>(Kr, k0 + 32 * (t2 < last ? t2 : last), k1, lane, ka);
        tile(kb, t1);
        if (t2 > last) break;
        t = t2;
    }
}

// ---------------------------------------------------------------- kernels

// Pass 1: one workgroup per (local row, STATS_CHUNK keys); also used for
// windows inside the cache (page effects).
template <int D, int NB>
__global__ void __launch_bounds__(SCORE_THREADS) __attribute__((amdgpu_waves_per_eu(4))) score_pass1(const uint16_t *__restrict__ K,
                                                             const uint16_t *__restrict__ Q, int64_t T, int W,
                                                             int G, int L, int Hkv, int Hq, int64_t n_chunks,
                                                             float c2, WindowGeom wg, float2 *__restrict__ part) {
    constexpr int QRP = NB * 32;
    extern __shared__ uint4 sq[];
    __shared__ float s_m[SCORE_WAVES * QRP], s_l[SCORE_WAVES * QRP];
    const int64_t r = blockIdx.x / n_chunks;
    const int64_t chunk = blockIdx.x % n_chunks;
    const int64_t gr = wg.global_row(r, L, Hkv);
    const RowIdx ri = split_row(gr, L, Hkv);
    const uint16_t *Kr = K + (size_t)gr * T * D;
    const uint16_t *Qg = Q + ((size_t)(ri.n * L + ri.l) * Hq + (size_t)ri.h * G) * W * D;
    stage_queries<D, NB>(Qg, G * W, sq);
    __syncthreads();
    const int64_t k0 = chunk * STATS_CHUNK;
    const int64_t k1 = k0 + STATS_CHUNK < wg.kend ? k0 + STATS_CHUNK : wg.kend;
    p1_chunk<D, NB>(Kr, k0, k1, wg.qbase, W, G * W, c2, sq, s_m, s_l, part + ((size_t)r * QRP) * n_chunks + chunk,
                    n_chunks);
}

__global__ void __launch_bounds__(SCORE_THREADS) score_merge(const float2 *__restrict__ part, int64_t n_chunks,
                                                              int QR, int QRP, float *__restrict__ mm) {
    __shared__ float2 s_tmp[SCORE_THREADS];
    const int64_t r = blockIdx.x;
    merge_row(part + (size_t)r * n_chunks * QRP, n_chunks, QR, QRP, mm + r * QRP, s_tmp);
}

// Pass 2: one workgroup per (row, STATS_CHUNK keys), with the row's merged
// normalisers mm[row][QRP].
template <int D, int NB>
__global__ void __launch_bounds__(SCORE_THREADS) score_pass2(const uint16_t *__restrict__ K,
                                                             const uint16_t *__restrict__ Q, int64_t T, int W,
                                                             int G, int L, int Hkv, int Hq, int64_t n_chunks,
                                                             float c2, const float *__restrict__ mm,
                                                             float *__restrict__ scores, unsigned *__restrict__ ctl) {
    constexpr int QRP = NB * 32;
    if (blockIdx.x == 0 && threadIdx.x == 0) ctl[0] = 0u;   // the two passes never give up
    extern __shared__ uint4 sq[];
    __shared__ float4 s_mm[QRP / 4];
    const int64_t r = blockIdx.x / n_chunks;
    const int64_t chunk = blockIdx.x % n_chunks;
    const RowIdx ri = split_row(r, L, Hkv);
    const uint16_t *Kr = K + (size_t)r * T * D;
    const uint16_t *Qg = Q + ((size_t)(ri.n * L + ri.l) * Hq + (size_t)ri.h * G) * W * D;
    stage_queries<D, NB>(Qg, G * W, sq);
    for (int q = threadIdx.x; q < QRP / 4; q += SCORE_THREADS)
        s_mm[q] = *reinterpret_cast<const float4 *>(mm + r * QRP + 4 * q);
    __syncthreads();
    const int64_t k0 = chunk * STATS_CHUNK;
    const int64_t k1 = k0 + STATS_CHUNK < T ? k0 + STATS_CHUNK : T;
    p2_chunk<D, NB>(Kr, k0, k1, T - W, W, c2, sq, s_mm, scores + (size_t)r * T);
}

// ---------------------------------------------------------------- launches

template <int D, int NB>
static int launch_pass1(int64_t blocks, hipStream_t s, const uint16_t *K, const uint16_t *Q, int64_t T, int W,
                        int G, int L, int Hkv, int Hq, int64_t n_chunks, float c2, WindowGeom wg, float2 *part) {
    const size_t lds = (size_t)NB * (D / 16) * 64 * sizeof(uint4);
    score_pass1<D, NB><<<dim3((unsigned)blocks), dim3(SCORE_THREADS), lds, s>>>(K, Q, T, W, G, L, Hkv, Hq,
                                                                               n_chunks, c2, wg, part);
    return check_launch("score pass 1");
}

template <int D, int NB>
static int launch_pass2(int64_t blocks, hipStream_t s, const uint16_t *K, const uint16_t *Q, int64_t T, int W,
                        int G, int L, int Hkv, int Hq, int64_t n_chunks, float c2, const float *mm,
                        float *scores, unsigned *ctl) {
    const size_t lds = (size_t)NB * (D / 16) * 64 * sizeof(uint4);
    score_pass2<D, NB><<<dim3((unsigned)blocks), dim3(SCORE_THREADS), lds, s>>>(K, Q, T, W, G, L, Hkv, Hq,
                                                                               n_chunks, c2, mm, scores, ctl);
    return check_launch("kvc_score pass 2");
}

#define KVC_NB_SWITCH(nb, D, CALL) \
    switch (nb) {                  \
    case 1: return CALL(D, 1);     \
    case 2: return CALL(D, 2);     \
    case 3: return CALL(D, 3);     \
    case 4: return CALL(D, 4);     \
    case 5: return CALL(D, 5);     \
    case 6: return CALL(D, 6);     \
    case 7: return CALL(D, 7);     \
    default: return CALL(D, 8);    \
    }

int launch_window_stats(const kvc_dims *d, const uint16_t *K, const uint16_t *Q, int W, WindowGeom wg,
                        int64_t rows_local, float2 *part, float *mm, hipStream_t s) {
    const int G = d->n_q_heads / d->n_kv_heads;
    const int QR = G * W, nb = (QR + 31) / 32, QRP = nb * 32;
    const int64_t n_chunks = window_chunks(wg.kend);
    const int64_t blocks = rows_local * n_chunks;
    if (blocks > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "window stats: grid too large");
    const float c2 = (float)(1.4426950408889634 / std::sqrt((double)d->head_dim));
    const int64_t T = d->n_tokens;
    const int L = d->n_layers, Hkv = d->n_kv_heads, Hq = d->n_q_heads;
    auto p1 = [&]() -> int {
#define P1(DD, NN) launch_pass1<DD, NN>(blocks, s, K, Q, T, W, G, L, Hkv, Hq, n_chunks, c2, wg, part)
        if (d->head_dim == 128) {
            KVC_NB_SWITCH(nb, 128, P1)
        } else {
            KVC_NB_SWITCH(nb, 64, P1)
        }
#undef P1
    };
    int st = p1();
    if (st != KVC_OK) return st;
    score_merge<<<dim3((unsigned)rows_local), dim3(SCORE_THREADS), 0, s>>>(part, n_chunks, QR, QRP, mm);
    return check_launch("window stats merge");
}

}  // namespace kvc

namespace kvc {

KVC_CHECK_READER(check_read_score)

// Argument checks shared by both score entry points; on success `need` holds
// the workspace bytes the call uses.
static int score_check(const kvc_dims *dims, const uint16_t *K, const uint16_t *Q_obs, int32_t W,
                       const float *scores, const char *who, size_t *need) {
    int st = check_dims(dims, who);
    if (st != KVC_OK) return st;
    if (!K || !Q_obs || !scores) return fail(KVC_ERR_ARG, "%s: NULL tensor pointer", who);
    if (W <= 0 || W > dims->n_tokens)
        return fail(KVC_ERR_ARG, "%s: W=%d must be in [1, T=%lld]", who, W, (long long)dims->n_tokens);
    const int G = dims->n_q_heads / dims->n_kv_heads;
    if ((int64_t)G * W > SCORE_MAX_QR)
        return fail(KVC_ERR_UNSUPPORTED, "%s: W*G=%d exceeds %d query rows", who, G * W, SCORE_MAX_QR);
    *need = score_workspace_bytes(dims, W);
    return KVC_OK;
}

// The score kernels over a checked call, with `ws` (>= the bytes score_check
// reported) as their scratch.
static int score_enqueue(const kvc_dims *dims, const uint16_t *K, const uint16_t *Q_obs, int32_t W,
                         float *scores, void *ws, hipStream_t s);

// ---------------------------------------------------------------- the no-allocation variant
//
// Scratch of kvc_score_noalloc: a file-scope device array (each GPU the
// library runs on holds its own copy until the process ends). Host code
// never uses the array's name as an address: it takes each device's address
// once, through hipGetSymbolAddress with that device current, and passes
// that pointer to the kernels.
static constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static std::vector<void *> g_scratch_ptr;   // per device ordinal; NULL until first looked up

static int scratch_pointer(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return fail(KVC_ERR_HIP, "kvc_score_noalloc: no current device");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(KVC_ERR_HIP, "kvc_score_noalloc: hipGetSymbolAddress of the scratch array failed: %s",
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KVC_OK;
}

}  // namespace kvc

using namespace kvc;

extern "C" size_t kvc_score_noalloc_max_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

extern "C" int kvc_score_options(int32_t single_read, int64_t wait_us, int32_t diag_no_merge) {
    if (single_read != 0 && single_read != 1) return fail(KVC_ERR_ARG, "kvc_score_options: single_read must be 0 or 1");
    if (wait_us < 0) return fail(KVC_ERR_ARG, "kvc_score_options: wait_us must be >= 0");
    g_single_read = single_read != 0;
    set_score_wait(wait_us, diag_no_merge != 0);
    return KVC_OK;
}

extern "C" int kvc_score_status(const void *ws, void *stream) {
    void *p = const_cast<void *>(ws);
    if (!p) {
        const int st = scratch_pointer(&p);
        if (st != KVC_OK) return st;
    }
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return fail(KVC_ERR_HIP, "kvc_score_status: stream");
    unsigned w = 0;
    if (hipMemcpy(&w, p, sizeof(w), hipMemcpyDeviceToHost) != hipSuccess)
        return fail(KVC_ERR_HIP, "kvc_score_status: copy of the status word failed");
    if (w != 0u) return fail(KVC_ERR_HIP, "kvc_score: the single-read kernel gave up waiting (status %u)", w);
    return KVC_OK;
}

extern "C" int kvc_score_noalloc(const kvc_dims *dims, const uint16_t *K, const uint16_t *Q_obs, int32_t W,
                                 float *scores, void *stream) {
    size_t need = 0;
    int st = score_check(dims, K, Q_obs, W, scores, "kvc_score_noalloc", &need);
    if (st != KVC_OK) return st;
    if (need > NOALLOC_SCRATCH_BYTES)
        return fail(KVC_ERR_WORKSPACE,
                    "kvc_score_noalloc: the call needs %zu bytes of scratch, above the library's static %zu "
                    "(fewer rows or shorter rows per call, or kvc_score with a workspace)",
                    need, NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if ((st = scratch_pointer(&ws)) != KVC_OK) return st;
    return score_enqueue(dims, K, Q_obs, W, scores, ws, as_stream(stream));
}

extern "C" int kvc_score(const kvc_dims *dims, const uint16_t *K, const uint16_t *Q_obs, int32_t W,
                         float *scores, void *ws, size_t ws_bytes, void *stream) {
    size_t need = 0;
    int st = score_check(dims, K, Q_obs, W, scores, "kvc_score", &need);
    if (st != KVC_OK) return st;
    if (!ws || ws_bytes < need)
        return fail(KVC_ERR_WORKSPACE, "kvc_score: workspace %zu < %zu bytes", ws_bytes, need);
    return score_enqueue(dims, K, Q_obs, W, scores, ws, as_stream(stream));
}

namespace kvc {

static int score_enqueue(const kvc_dims *dims, const uint16_t *K, const uint16_t *Q_obs, int32_t W,
                         float *scores, void *ws, hipStream_t s) {
    int st;
    size_t once_bytes = 0;
    const int nwg = g_single_read ? score_once_plan(dims, W, &once_bytes) : 0;
    if (nwg > 0) return launch_score_once(dims, K, Q_obs, W, scores, ws, nwg, s);
    unsigned *ctl = reinterpret_cast<unsigned *>(ws);
    ws = reinterpret_cast<char *>(ws) + 256;
    const int G = dims->n_q_heads / dims->n_kv_heads;
    float2 *part = reinterpret_cast<float2 *>(ws);
    const int64_t rows = n_rows(dims), T = dims->n_tokens;
    const int64_t n_chunks = window_chunks(T);
    const int nb = (G * W + 31) / 32, QRP = nb * 32;
    float *mm = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) +
                                          align256((size_t)rows * n_chunks * QRP * sizeof(float2)));
    st = launch_window_stats(dims, K, Q_obs, W, WindowGeom{T - W, T, -1}, rows, part, mm, s);
    if (st != KVC_OK) return st;
    const int64_t blocks = rows * n_chunks;
    if (blocks > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "kvc_score: grid too large");
    const float c2 = (float)(1.4426950408889634 / std::sqrt((double)dims->head_dim));
    const int L = dims->n_layers, Hkv = dims->n_kv_heads, Hq = dims->n_q_heads;
#define P2(DD, NN) launch_pass2<DD, NN>(blocks, s, K, Q_obs, T, W, G, L, Hkv, Hq, n_chunks, c2, mm, scores, ctl)
    if (dims->head_dim == 128) {
        KVC_NB_SWITCH(nb, 128, P2)
    } else {
        KVC_NB_SWITCH(nb, 64, P2)
    }
#undef P2
}

}  // namespace kvc
