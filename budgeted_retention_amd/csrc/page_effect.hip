// kvc_page_effect / kvc_page_retire: CommitKV page deletion effects.
//
// CommitKV §3.2: for one attention layer, query p of a window pays weight a_pi
// to token i and outputs o_p. Deleting a page E and renormalising gives, by
// Eq. 6, o_p^{\E} = (o_p - S_E) / (1 - alpha_E) with alpha_E = sum_{i in E} a_pi
// and S_E = sum_{i in E} a_pi v_i, so
//   o_p - o_p^{\E} = (S_E - alpha_E o_p) / (1 - alpha_E)
//                  = sum_{i in E} a_pi (v_i - o_p) / (1 - alpha_E).
// Eq. 7 takes ||.|| / ||o_p||, the max over the window's queries and over the
// layer's query heads. The deletion vector is formed directly as
// sum a_pi (v_i - o_p), never as a difference of two large norms.
//
// Stages, all for the chosen layer:
//   1. window statistics (the score kernels' pass 1 + merge): per query row
//      the log2-domain max and normaliser, so a_pi = exp2(logit*c - mm);
//   2. pe_out: o_p for every query row (MFMA logits, a_pi staged in LDS,
//      thread <-> (dimension pair, query stripe) accumulation over V in LDS);
//   3. pe_effect: for every page, alpha and ||sum a (v - o)|| per query row,
//      reduced to the max over rows and heads with an atomic max on the
//      non-negative float bit pattern (order-independent, so deterministic);
//   4. pe_retire (kvc_page_retire): CommitKV §3.3 Eq. 11 greedy joint test in
//      the caller's candidate order, one workgroup per sequence; a candidate is
//      accepted iff the effect of deleting it together with the pages already
//      accepted stays within tau_joint.
//
// kvc_page_scores serves the compression checkpoint that follows (CommitKV
// §3.3, Eq. 13 with Eq. 4): one page score per sequence, the window score of
// every token summed over the page's tokens and over all layers and KV heads,
// so that one page set can be kept for the whole sequence; pages accepted for
// retirement are scored -inf.
#include <cmath>

#include "kvc_internal.h"

namespace kvc {

static constexpr int PE_TILE = 64;      // keys per tile
static constexpr int PE_THREADS = 128;  // two waves: 32 query rows x 64 keys of logits
static constexpr int PE_PAGE_CHUNK = 4096;  // keys per pe_effect workgroup
static constexpr int PR_THREADS = 256;
static constexpr int PR_PMAX = 16;      // largest page the retire kernel takes
static constexpr int PR_BATCH = 8;      // candidates whose deletion terms are formed per launch
static constexpr int PG_THREADS = 1024; // greedy walk: one workgroup per sequence
static constexpr int PG_RPT = 4;        // query rows per walk thread: Hkv * G * W <= 4096
static constexpr int GR = 80;           // Gram record per query row (see pr_gram)
static constexpr int PO_CHUNK = 4096;   // keys per pe_out_mfma / pe_effect_mfma workgroup
static constexpr int PM_THREADS = 256;  // four waves, each on its own 32-key tiles

struct PageGeom {
    int64_t rows_local, n_chunks;
    int G, QR, nb, QRP;
};

static PageGeom page_geom(const kvc_dims *d, int W, int64_t kend) {
    PageGeom g;
    g.G = d->n_q_heads / d->n_kv_heads;
    g.rows_local = (int64_t)d->n_seq * d->n_kv_heads;
    g.n_chunks = window_chunks(kend);
    g.QR = g.G * W;
    g.nb = (g.QR + 31) / 32;
    g.QRP = g.nb * 32;
    return g;
}

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct PageWs {
    float2 *part;
    float *mm, *o, *accD, *alphaD;
    float *tD, *tA;   // [PR_BATCH][rows][QRP][D] and [PR_BATCH][rows][QRP]: one batch's deletion terms
    float *opart;     // [chunks][rows][QRP][D]: per-chunk partial window outputs
    float *gram;      // [rows][QRP][GR]: inner products of one batch (pr_gram)
};

static size_t page_ws_layout(const kvc_dims *d, int W, int64_t kend, void *base, PageWs *w) {
    const PageGeom g = page_geom(d, W, kend);
    const size_t s_part = al256((size_t)g.rows_local * g.n_chunks * g.QRP * sizeof(float2));
    const size_t s_mm = al256((size_t)g.rows_local * g.QRP * sizeof(float));
    const size_t s_o = al256((size_t)g.rows_local * g.QRP * d->head_dim * sizeof(float));
    const size_t s_a = al256((size_t)g.rows_local * g.QRP * sizeof(float));
    const size_t s_tD = al256((size_t)PR_BATCH * g.rows_local * g.QRP * d->head_dim * sizeof(float));
    const size_t s_tA = al256((size_t)PR_BATCH * g.rows_local * g.QRP * sizeof(float));
    const int64_t och = (kend + PO_CHUNK - 1) / PO_CHUNK;
    const size_t s_op = al256((size_t)och * g.rows_local * g.QRP * d->head_dim * sizeof(float));
    const size_t s_gr = al256((size_t)g.rows_local * g.QRP * GR * sizeof(float));
    if (w) {
        char *p = reinterpret_cast<char *>(base);
        w->part = reinterpret_cast<float2 *>(p);
        w->mm = reinterpret_cast<float *>(p + s_part);
        w->o = reinterpret_cast<float *>(p + s_part + s_mm);
        w->accD = reinterpret_cast<float *>(p + s_part + s_mm + s_o);
        w->alphaD = reinterpret_cast<float *>(p + s_part + s_mm + 2 * s_o);
        w->tD = reinterpret_cast<float *>(p + s_part + s_mm + 2 * s_o + s_a);
        w->tA = reinterpret_cast<float *>(p + s_part + s_mm + 2 * s_o + s_a + s_tD);
        w->opart = reinterpret_cast<float *>(p + s_part + s_mm + 2 * s_o + s_a + s_tD + s_tA);
        w->gram = reinterpret_cast<float *>(p + s_part + s_mm + 2 * s_o + s_a + s_tD + s_tA + s_op);
    }
    return s_part + s_mm + 2 * s_o + s_a + s_tD + s_tA + s_op + s_gr;
}

struct PeArgs {
    const uint16_t *K, *V, *Q;
    int64_t T;
    int W, G, L, Hkv, Hq, lsel;
    int64_t qbase, kend;
    float c2;
    const float *mm;
    float *o;
    int page_size, n_pages;
    const int32_t *pfirst, *plen;   // event pages [N][n_pages], or NULL for uniform pages
    float *eff_rel, *eff_abs;
    float *opart;
};

// Token span of page e of sequence n: [first, first + len). Event pages are
// clamped to the cache and to page_size (the longest page).
__device__ __forceinline__ void page_span(const PeArgs &a, int n, int e, int64_t &first, int &len) {
    if (a.pfirst) {
        int64_t f = a.pfirst[(size_t)n * a.n_pages + e];
        int64_t l = a.plen[(size_t)n * a.n_pages + e];
        KVC_NOTE(f < 0 || l < 0 || l > a.page_size || f + l > a.T, KVC_CHK_SPAN);
        f = f < 0 ? 0 : (f > a.T ? a.T : f);
        l = l < 0 ? 0 : (l > a.page_size ? a.page_size : l);
        if (l > a.T - f) l = a.T - f;
        first = f;
        len = (int)l;
    } else {
        first = (int64_t)e * a.page_size;
        len = a.page_size;
    }
}

// Stages one 64-key tile: a_pi for the block's 32 query rows into sp[32][64]
// (0 for invisible keys and padding rows) and V into sv[64][D] as fp32.
template <int D>
__device__ void pe_stage_tile(const PeArgs &a, const uint16_t *Kr, const uint16_t *Vr, const bf16x8 *qf,
                              const float *mmq, const int64_t *qposq, int64_t j0, float (*sp)[PE_TILE + 1],
                              float (*sv)[D]) {
    constexpr int S = D / 16;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hf = lane >> 5;
    const int64_t jb = j0 + 32 * wave;
    const int64_t key = jb + col;
    bf16x8 kf[S];
#pragma unroll
    for (int s = 0; s < S; ++s) kf[s] = key < a.kend ? load8(Kr + (size_t)key * D + 16 * s + 8 * hf) : zero8();
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < S; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], acc, 0, 0, 0);
    // acc[i]: key jb + acc_row(i, hf), query row `col` of the block
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t k = jb + acc_row(i, hf);
        const float p = (k <= qposq[0]) ? __builtin_amdgcn_exp2f(fmaf(acc[i], a.c2, -mmq[0])) : 0.f;
        sp[col][32 * wave + acc_row(i, hf)] = p;
    }
    for (int e = tid; e < PE_TILE * D / 2; e += PE_THREADS) {
        const int k = e / (D / 2), c = 2 * (e % (D / 2));
        float v0 = 0.f, v1 = 0.f;
        if (j0 + k < a.kend) {
            const uint32_t u = *reinterpret_cast<const uint32_t *>(Vr + (size_t)(j0 + k) * D + c);
            v0 = bf16_to_f32((uint16_t)(u & 0xFFFF));
            v1 = bf16_to_f32((uint16_t)(u >> 16));
        }
        sv[k][c] = v0;
        sv[k][c + 1] = v1;
    }
}

// Per-lane window data of query row `col` of block `b`: Q fragments, mm, position.
template <int D>
__device__ void pe_load_queries(const PeArgs &a, int64_t rr, int b, bf16x8 *qf, float *mmq, int64_t *qposq,
                                const uint16_t **Kr, const uint16_t **Vr) {
    constexpr int S = D / 16;
    const int lane = threadIdx.x & 63, col = lane & 31, hf = lane >> 5;
    const int64_t gr = ((rr / a.Hkv) * a.L + a.lsel) * a.Hkv + rr % a.Hkv;
    const RowIdx ri = split_row(gr, a.L, a.Hkv);
    *Kr = a.K + (size_t)gr * a.T * D;
    *Vr = a.V + (size_t)gr * a.T * D;
    const uint16_t *Qg = a.Q + ((size_t)(ri.n * a.L + ri.l) * a.Hq + (size_t)ri.h * a.G) * a.W * D;
    const int qrow = b * 32 + col;
    const int QR = a.G * a.W;
#pragma unroll
    for (int s = 0; s < S; ++s) qf[s] = qrow < QR ? load8(Qg + (size_t)qrow * D + 16 * s + 8 * hf) : zero8();
    const int QRP = ((QR + 31) / 32) * 32;
    mmq[0] = a.mm[rr * QRP + qrow];
    qposq[0] = qrow < QR ? a.qbase + qrow % a.W : -1;
}

__device__ __forceinline__ void atomic_max_nonneg(float *addr, float v) {
    atomicMax(reinterpret_cast<unsigned int *>(addr), __float_as_uint(v));
}

template <int D>
__global__ void __launch_bounds__(PE_THREADS) pe_effect(PeArgs a, int chunks_per_row) {
    constexpr int DP = D / 2, STRIPES = PE_THREADS / DP, QPS = 32 / STRIPES;
    __shared__ float sp[32][PE_TILE + 1];
    __shared__ float sv[PE_TILE][D];
    __shared__ float s_alpha[32][PE_TILE];   // per query row and page of the tile (<= 64 pages)
    __shared__ float s_best[2][STRIPES][PE_TILE];
    const int nb = (a.G * a.W + 31) / 32;
    const int64_t rr = blockIdx.x / (nb * chunks_per_row);
    const int b = (int)((blockIdx.x / chunks_per_row) % nb);
    const int pc = (int)(blockIdx.x % chunks_per_row);
    bf16x8 qf[D / 16];
    float mmq[1];
    int64_t qposq[1];
    const uint16_t *Kr, *Vr;
    pe_load_queries<D>(a, rr, b, qf, mmq, qposq, &Kr, &Vr);
    const int tid = threadIdx.x, dp = tid % DP, stripe = tid / DP;
    const int QR = a.G * a.W, QRP = nb * 32;
    const int ps = a.page_size, ppt = PE_TILE / ps;  // pages per tile
    const int64_t n_tok = (int64_t)a.n_pages * ps;
    const int n_seq_idx = (int)(rr / a.Hkv);

    // o and ||o|| for this thread's query rows
    float o0[QPS], o1[QPS], onorm[QPS];
#pragma unroll
    for (int q = 0; q < QPS; ++q) {
        const float *o = a.o + ((size_t)rr * QRP + b * 32 + stripe * QPS + q) * D;
        o0[q] = o[2 * dp];
        o1[q] = o[2 * dp + 1];
        float n2 = o0[q] * o0[q] + o1[q] * o1[q];
        for (int m = DP / 2; m >= 1; m >>= 1) n2 += __shfl_xor(n2, m);
        onorm[q] = sqrtf(n2);
    }
    const int64_t t_begin = (int64_t)pc * PE_PAGE_CHUNK;
    const int64_t t_end = t_begin + PE_PAGE_CHUNK < n_tok ? t_begin + PE_PAGE_CHUNK : n_tok;
    for (int64_t j0 = t_begin; j0 < t_end; j0 += PE_TILE) {
        pe_stage_tile<D>(a, Kr, Vr, qf, mmq, qposq, j0, sp, sv);
        __syncthreads();
        for (int e = tid; e < 32 * ppt; e += PE_THREADS) {
            const int q = e / ppt, pg = e % ppt;
            float al = 0.f;
            for (int k = 0; k < ps; ++k) al += sp[q][pg * ps + k];
            s_alpha[q][pg] = al;
        }
        __syncthreads();
        for (int pg = 0; pg < ppt; ++pg) {
            float best_rel = 0.f, best_abs = 0.f;
#pragma unroll
            for (int q = 0; q < QPS; ++q) {
                const int ql = stripe * QPS + q;
                float t0 = 0.f, t1 = 0.f;
                for (int k = 0; k < ps; ++k) {
                    const float p = sp[ql][pg * ps + k];
                    t0 = fmaf(p, sv[pg * ps + k][2 * dp] - o0[q], t0);
                    t1 = fmaf(p, sv[pg * ps + k][2 * dp + 1] - o1[q], t1);
                }
                float n2 = t0 * t0 + t1 * t1;
                for (int m = DP / 2; m >= 1; m >>= 1) n2 += __shfl_xor(n2, m);
                if (b * 32 + ql < QR) {
                    const float al = s_alpha[ql][pg];
                    const float num = sqrtf(n2);
                    const float den = 1.f - al;
                    float ab = den > 0.f ? num / den : INFINITY;
                    float rel = onorm[q] > 0.f ? ab / onorm[q] : (num > 0.f ? INFINITY : 0.f);
                    if (!(num > 0.f)) ab = rel = 0.f;
                    best_rel = fmaxf(best_rel, rel);
                    best_abs = fmaxf(best_abs, ab);
                }
            }
            if (dp == 0) {
                s_best[0][stripe][pg] = best_rel;
                s_best[1][stripe][pg] = best_abs;
            }
        }
        __syncthreads();
        for (int pg = tid; pg < ppt; pg += PE_THREADS) {
            const int64_t page = (j0 / ps) + pg;
            if (page >= a.n_pages) continue;
            float br = 0.f, ba = 0.f;
            for (int s = 0; s < STRIPES; ++s) {
                br = fmaxf(br, s_best[0][s][pg]);
                ba = fmaxf(ba, s_best[1][s][pg]);
            }
            atomic_max_nonneg(a.eff_rel + (size_t)n_seq_idx * a.n_pages + page, br);
            if (a.eff_abs) atomic_max_nonneg(a.eff_abs + (size_t)n_seq_idx * a.n_pages + page, ba);
        }
        __syncthreads();
    }
}

// Event pages of at most PE_TILE tokens (page_first / page_len). A workgroup
// walks its run of PE_SPAN_CHUNK pages: it stages the 64 keys from the first
// page's first token, takes every following page lying wholly inside them, and
// goes on from the first page that does not (pages in token order cover each
// staged tile with at least 64 - page_size + 1 tokens of whole pages).
static constexpr int PE_SPAN_CHUNK = 256;

template <int D>
__global__ void __launch_bounds__(PE_THREADS) pe_effect_spans(PeArgs a, int chunks_per_row) {
    constexpr int DP = D / 2, STRIPES = PE_THREADS / DP, QPS = 32 / STRIPES;
    __shared__ float sp[32][PE_TILE + 1];
    __shared__ float sv[PE_TILE][D];
    __shared__ float s_alpha[32][PE_TILE];
    __shared__ float s_best[2][STRIPES][PE_TILE];
    __shared__ int64_t s_first[PE_SPAN_CHUNK];
    __shared__ int s_len[PE_SPAN_CHUNK];
    const int nb = (a.G * a.W + 31) / 32;
    const int64_t rr = blockIdx.x / (nb * chunks_per_row);
    const int b = (int)((blockIdx.x / chunks_per_row) % nb);
    const int pc = (int)(blockIdx.x % chunks_per_row);
    bf16x8 qf[D / 16];
    float mmq[1];
    int64_t qposq[1];
    const uint16_t *Kr, *Vr;
    pe_load_queries<D>(a, rr, b, qf, mmq, qposq, &Kr, &Vr);
    const int tid = threadIdx.x, dp = tid % DP, stripe = tid / DP;
    const int QR = a.G * a.W, QRP = nb * 32;
    const int n_seq_idx = (int)(rr / a.Hkv);
    const int e_begin = pc * PE_SPAN_CHUNK;
    const int e_end = e_begin + PE_SPAN_CHUNK < a.n_pages ? e_begin + PE_SPAN_CHUNK : a.n_pages;
    for (int e = e_begin + tid; e < e_end; e += PE_THREADS) {
        int64_t f;
        int l;
        page_span(a, n_seq_idx, e, f, l);
        s_first[e - e_begin] = f;
        s_len[e - e_begin] = l;
    }
    float o0[QPS], o1[QPS], onorm[QPS];
#pragma unroll
    for (int q = 0; q < QPS; ++q) {
        const float *o = a.o + ((size_t)rr * QRP + b * 32 + stripe * QPS + q) * D;
        o0[q] = o[2 * dp];
        o1[q] = o[2 * dp + 1];
        float n2 = o0[q] * o0[q] + o1[q] * o1[q];
        for (int m = DP / 2; m >= 1; m >>= 1) n2 += __shfl_xor(n2, m);
        onorm[q] = sqrtf(n2);
    }
    __syncthreads();
    int e = e_begin;
    while (e < e_end) {   // the same sequence of pages for every thread
        const int64_t j0 = s_first[e - e_begin];
        int e1 = e + 1;
        while (e1 < e_end && e1 - e < PE_TILE && s_first[e1 - e_begin] >= j0 &&
               s_first[e1 - e_begin] + s_len[e1 - e_begin] <= j0 + PE_TILE)
            ++e1;
        const int np = e1 - e;
        pe_stage_tile<D>(a, Kr, Vr, qf, mmq, qposq, j0, sp, sv);
        __syncthreads();
        for (int t = tid; t < 32 * np; t += PE_THREADS) {
            const int q = t / np, pg = t % np;
            const int off = (int)(s_first[e - e_begin + pg] - j0), len = s_len[e - e_begin + pg];
            float al = 0.f;
            for (int k = 0; k < len; ++k) al += sp[q][off + k];
            s_alpha[q][pg] = al;
        }
        __syncthreads();
        for (int pg = 0; pg < np; ++pg) {
            const int off = (int)(s_first[e - e_begin + pg] - j0), len = s_len[e - e_begin + pg];
            float best_rel = 0.f, best_abs = 0.f;
#pragma unroll
            for (int q = 0; q < QPS; ++q) {
                const int ql = stripe * QPS + q;
                float t0 = 0.f, t1 = 0.f;
                for (int k = 0; k < len; ++k) {
                    const float p = sp[ql][off + k];
                    t0 = fmaf(p, sv[off + k][2 * dp] - o0[q], t0);
                    t1 = fmaf(p, sv[off + k][2 * dp + 1] - o1[q], t1);
                }
                float n2 = t0 * t0 + t1 * t1;
                for (int m = DP / 2; m >= 1; m >>= 1) n2 += __shfl_xor(n2, m);
                if (b * 32 + ql < QR) {
                    const float al = s_alpha[ql][pg];
                    const float num = sqrtf(n2);
                    const float den = 1.f - al;
                    float ab = den > 0.f ? num / den : INFINITY;
                    float rel = onorm[q] > 0.f ? ab / onorm[q] : (num > 0.f ? INFINITY : 0.f);
                    if (!(num > 0.f)) ab = rel = 0.f;
                    best_rel = fmaxf(best_rel, rel);
                    best_abs = fmaxf(best_abs, ab);
                }
            }
            if (dp == 0) {
                s_best[0][stripe][pg] = best_rel;
                s_best[1][stripe][pg] = best_abs;
            }
        }
        __syncthreads();
        for (int pg = tid; pg < np; pg += PE_THREADS) {
            float br = 0.f, ba = 0.f;
            for (int st = 0; st < STRIPES; ++st) {
                br = fmaxf(br, s_best[0][st][pg]);
                ba = fmaxf(ba, s_best[1][st][pg]);
            }
            atomic_max_nonneg(a.eff_rel + (size_t)n_seq_idx * a.n_pages + e + pg, br);
            if (a.eff_abs) atomic_max_nonneg(a.eff_abs + (size_t)n_seq_idx * a.n_pages + e + pg, ba);
        }
        __syncthreads();
        e = e1;
    }
}

__global__ void fill_f32(float *p, int64_t n, float v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}


// ---------------------------------------------------------------- P·V on the matrix cores
//
// A wave owns one block of 32 query rows of one row and walks 32-key tiles.
// Logits come from v_mfma_f32_32x32x16_bf16 as C[key][q] (lane (col, hf) holds
// query row col and keys acc_row(i, hf)); the weights a = exp2(logit*c - mm)
// stay in those registers. P·V is then C[d][q] = sum_k V[k][d] P[q][k], again
// on v_mfma_f32_32x32x16_bf16 over 16 keys at a time: lane (col, g) supplies
// A[col][8g .. 8g+7] and B[8g .. 8g+7][col]. The instruction's k index is
// mapped to keys so that B is the lane's own weights: in key block beta (keys
// 16*beta .. 16*beta + 15 of the tile) k = 8g + t stands for key
// acc_row(8*beta + t, g), which is where the logits left that key's weight
// for query row col; A is then V of those keys at dimension col of the
// dimension block, gathered from the wave's V tile in LDS. Each fp32 weight
// is split into hi = bf16(w) and lo = bf16(w - hi) (w - hi is exact in fp32),
// so hi + lo carries about 16 significant bits; V is bf16 already. Every
// lane then holds query row col over 16 dimensions of each block, so a row's
// squared norm is an in-lane sum plus one shuffle.

template <int D>
__device__ __forceinline__ void pm_setup(const PeArgs &a, int64_t rr, int b, bf16x8 (&qf)[D / 16], float &mmq,
                                         int64_t &qpos, bool &qvalid, const uint16_t **Kr, const uint16_t **Vr) {
    float mm1[1];
    int64_t qp1[1];
    pe_load_queries<D>(a, rr, b, qf, mm1, qp1, Kr, Vr);
    mmq = mm1[0];
    qpos = qp1[0];
    qvalid = b * 32 + (int)(threadIdx.x & 31) < a.G * a.W;
}

// One 32-key tile: the wave's V tile into its LDS slice (bf16 [32][D]), the
// logits and the weights a[i] of keys j0 + acc_row(i, hf) (0 past kend or qpos).
template <int D>
__device__ __forceinline__ void pm_tile(const PeArgs &a, const uint16_t *Kr, const uint16_t *Vr, int64_t j0,
                                        const bf16x8 (&qf)[D / 16], float mmq, int64_t qpos, uint16_t *sv,
                                        float (&w)[16]) {
    constexpr int S = D / 16;
    constexpr int CPK = D / 8;  // 16-byte pieces per key
    const int lane = threadIdx.x & 63, col = lane & 31, hf = lane >> 5;
    bf16x8 kf[S];
    const int64_t key = j0 + col;
#pragma unroll
    for (int s = 0; s < S; ++s) kf[s] = key < a.kend ? load8(Kr + (size_t)key * D + 16 * s + 8 * hf) : zero8();
    // the previous tile's reads of the wave's V slice come before this tile's writes
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int u = 0; u < 32 * CPK / 64; ++u) {
        const int c = lane + 64 * u, k = c / CPK, part = c % CPK;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (j0 + k < a.kend) v = *reinterpret_cast<const uint4 *>(Vr + (size_t)(j0 + k) * D + 8 * part);
        *reinterpret_cast<uint4 *>(sv + k * D + 8 * part) = v;
    }
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < S; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t k = j0 + acc_row(i, hf);
        w[i] = (k < a.kend && k <= qpos) ? __builtin_amdgcn_exp2f(fmaf(acc[i], a.c2, -mmq)) : 0.f;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // the V tile is written before it is read
}

// The split weights of one tile: hi[beta], lo[beta] are the B operands of key block beta.
struct PvWeights {
    bf16x8 hi[2], lo[2];
};

__device__ __forceinline__ PvWeights pv_split(const float (&w)[16]) {
    PvWeights p;
#pragma unroll
    for (int beta = 0; beta < 2; ++beta)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float x = w[8 * beta + t];
            const __bf16 h = (__bf16)x;
            p.hi[beta][t] = h;
            p.lo[beta][t] = (__bf16)(x - (float)h);
        }
    return p;
}

// The A operand of key block beta and dimension block db: V[acc_row(8*beta + t, g)][db*32 + col].
template <int D>
__device__ __forceinline__ bf16x8 pv_v(const uint16_t *sv, int db, int beta) {
    const int lane = threadIdx.x & 63, col = lane & 31, g = lane >> 5;
    uint16_t e[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) e[t] = sv[acc_row(8 * beta + t, g) * D + db * 32 + col];
    const uint4 u = make_uint4(e[0] | (uint32_t)e[1] << 16, e[2] | (uint32_t)e[3] << 16,
                               e[4] | (uint32_t)e[5] << 16, e[6] | (uint32_t)e[7] << 16);
    return __builtin_bit_cast(bf16x8, u);
}

// c += V^T P over key block beta with split weights (hi, then lo).
__device__ __forceinline__ void pv_block(const bf16x8 &va, const bf16x8 &hi, const bf16x8 &lo, f32x16 &c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, hi, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, lo, c, 0, 0, 0);
}

// The weights of one key block with those of keys outside [lo, hi) of the tile set to 0.
__device__ __forceinline__ bf16x8 pv_mask(const bf16x8 &x, int beta, int lo, int hi) {
    const int g = (threadIdx.x & 63) >> 5;
    uint4 u = __builtin_bit_cast(uint4, x);
    uint32_t m[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int k0 = acc_row(8 * beta + 2 * q, g), k1 = acc_row(8 * beta + 2 * q + 1, g);
        m[q] = (k0 >= lo && k0 < hi ? 0xFFFFu : 0u) | (k1 >= lo && k1 < hi ? 0xFFFF0000u : 0u);
    }
    u.x &= m[0];
    u.y &= m[1];
    u.z &= m[2];
    u.w &= m[3];
    return __builtin_bit_cast(bf16x8, u);
}

// Window outputs o_q = sum_k a_qk v_k: each workgroup covers PO_CHUNK keys for one
// query block, its four waves summed in LDS, one partial per chunk.
template <int D>
__global__ void __launch_bounds__(PM_THREADS) pe_out_mfma(PeArgs a, int chunks) {
    constexpr int NDB = D / 32;
    __shared__ uint16_t s_v[PM_THREADS / 64][32 * D];
    __shared__ float s_o[32][D];
    const int nb = (a.G * a.W + 31) / 32;
    const int64_t rr = blockIdx.x / (nb * chunks);
    const int b = (int)((blockIdx.x / chunks) % nb);
    const int ch = (int)(blockIdx.x % chunks);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 31, hf = lane >> 5;
    bf16x8 qf[D / 16];
    float mmq;
    int64_t qpos;
    bool qvalid;
    const uint16_t *Kr, *Vr;
    pm_setup<D>(a, rr, b, qf, mmq, qpos, qvalid, &Kr, &Vr);
    f32x16 co[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) co[db] = f32x16{};
    const int64_t c0 = (int64_t)ch * PO_CHUNK;
    const int64_t c1 = c0 + PO_CHUNK < a.kend ? c0 + PO_CHUNK : a.kend;
    for (int64_t j0 = c0 + 32 * wave; j0 < c1; j0 += 32 * (PM_THREADS / 64)) {
        float w[16];
        pm_tile<D>(a, Kr, Vr, j0, qf, mmq, qpos, s_v[wave], w);
        const PvWeights pw = pv_split(w);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int beta = 0; beta < 2; ++beta)
                pv_block(pv_v<D>(s_v[wave], db, beta), pw.hi[beta], pw.lo[beta], co[db]);
    }
    // waves in turn add their partial into s_o
    for (int wv = 0; wv < PM_THREADS / 64; ++wv) {
        if (wave == wv) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float &dst = s_o[col][db * 32 + acc_row(i, hf)];
                    dst = (wv == 0 ? 0.f : dst) + co[db][i];
                }
        }
        __syncthreads();
    }
    const int QRP = nb * 32;
    float *out = a.opart + (((size_t)ch * (gridDim.x / (nb * chunks)) + rr) * QRP + b * 32) * D;
    for (int e = threadIdx.x; e < 32 * D; e += PM_THREADS) out[e] = s_o[e / D][e % D];
}

// o[rr][q][:] = sum over chunks of the partials, in chunk order.
__global__ void pe_out_reduce(const float *opart, float *o, int64_t n, int chunks) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        float acc = 0.f;
        for (int c = 0; c < chunks; ++c) acc += opart[(size_t)c * n + i];
        o[i] = acc;
    }
}

// Page effects for pages of PS = 8, 16 or 32 tokens: per page and query row,
// t = S - alpha o with S = sum_{k in page} a_qk v_k from the matrix cores, the
// relative norm reduced to the max over the wave's query rows and then over
// workgroups with an atomic max on the non-negative float bits.
template <int D, int PS>
__global__ void __launch_bounds__(PM_THREADS) pe_effect_mfma(PeArgs a, int chunks) {
    constexpr int NDB = D / 32;
    constexpr int JP = PS / 2;  // a page's weights among a lane's 16
    __shared__ uint16_t s_v[PM_THREADS / 64][32 * D];
    const int nb = (a.G * a.W + 31) / 32;
    const int64_t rr = blockIdx.x / (nb * chunks);
    const int b = (int)((blockIdx.x / chunks) % nb);
    const int ch = (int)(blockIdx.x % chunks);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 31, hf = lane >> 5;
    bf16x8 qf[D / 16];
    float mmq;
    int64_t qpos;
    bool qvalid;
    const uint16_t *Kr, *Vr;
    pm_setup<D>(a, rr, b, qf, mmq, qpos, qvalid, &Kr, &Vr);
    const int QRP = nb * 32;
    // this lane's part of o_q in the C[d][q] layout, and ||o_q||
    float ov[NDB][16];
    float o2 = 0.f;
    {
        const float *o = a.o + ((size_t)rr * QRP + b * 32 + col) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                ov[db][i] = o[db * 32 + acc_row(i, hf)];
                o2 = fmaf(ov[db][i], ov[db][i], o2);
            }
    }
    o2 += __shfl_xor(o2, 32);
    const float onorm = sqrtf(o2);
    const int n_seq_idx = (int)(rr / a.Hkv);
    const int64_t n_tok = (int64_t)a.n_pages * PS;
    const int64_t c0 = (int64_t)ch * PO_CHUNK;
    const int64_t c1 = c0 + PO_CHUNK < n_tok ? c0 + PO_CHUNK : n_tok;
    for (int64_t j0 = c0 + 32 * wave; j0 < c1; j0 += 32 * (PM_THREADS / 64)) {
        float w[16];
        pm_tile<D>(a, Kr, Vr, j0, qf, mmq, qpos, s_v[wave], w);
        const PvWeights pw = pv_split(w);
#pragma unroll
        for (int pg = 0; pg < 32 / PS; ++pg) {
            float al = 0.f;
#pragma unroll
            for (int j = pg * JP; j < (pg + 1) * JP; ++j) al += w[j];
            al += __shfl_xor(al, 32);
            // key blocks of the page: both (32 tokens), block pg (16), or half of block pg / 2 (8)
            const int beta = PS == 16 ? pg : pg / 2;
            bf16x8 mh = pw.hi[beta], ml = pw.lo[beta];
            if (PS == 8) {
                mh = pv_mask(mh, beta, 8 * pg, 8 * pg + 8);
                ml = pv_mask(ml, beta, 8 * pg, 8 * pg + 8);
            }
            float n2 = 0.f;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                f32x16 c = {};
                if (PS == 32) {
                    pv_block(pv_v<D>(s_v[wave], db, 0), pw.hi[0], pw.lo[0], c);
                    pv_block(pv_v<D>(s_v[wave], db, 1), pw.hi[1], pw.lo[1], c);
                } else {
                    pv_block(pv_v<D>(s_v[wave], db, beta), mh, ml, c);
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float t = fmaf(-al, ov[db][i], c[i]);
                    n2 = fmaf(t, t, n2);
                }
            }
            n2 += __shfl_xor(n2, 32);
            float rel = 0.f, ab = 0.f;
            if (qvalid) {
                const float num = sqrtf(n2);
                const float den = 1.f - al;
                ab = den > 0.f ? num / den : INFINITY;
                rel = onorm > 0.f ? ab / onorm : (num > 0.f ? INFINITY : 0.f);
                if (!(num > 0.f)) ab = rel = 0.f;
            }
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) {
                rel = fmaxf(rel, __shfl_xor(rel, off));
                ab = fmaxf(ab, __shfl_xor(ab, off));
            }
            const int64_t page = j0 / PS + pg;
            if (lane == 0 && page < a.n_pages) {
                atomic_max_nonneg(a.eff_rel + (size_t)n_seq_idx * a.n_pages + page, rel);
                if (a.eff_abs) atomic_max_nonneg(a.eff_abs + (size_t)n_seq_idx * a.n_pages + page, ab);
            }
        }
    }
}

// Event pages of at most 32 tokens on the matrix cores. Each wave walks its
// own run of PSM_PAGES pages: it forms the logits, weights and V tile of the
// 32 keys from a page's first token (pm_tile), takes every following page
// lying wholly inside them, and for each page masks the weights of the other
// keys and forms S = sum_{k in page} a_qk v_k over the key groups the page
// touches; the norm and the reduction to the page's maximum are as in
// pe_effect_mfma. Pages in token order share tiles; any order is correct.
static constexpr int PSM_PAGES = 64;   // pages per wave: lane i holds page i's span

template <int D>
__global__ void __launch_bounds__(PM_THREADS) pe_effect_spans_mfma(PeArgs a, int chunks) {
    constexpr int NDB = D / 32;
    __shared__ uint16_t s_v[PM_THREADS / 64][32 * D];
    __shared__ float s_o[32][D + 4];
    const int nb = (a.G * a.W + 31) / 32;
    const int64_t rr = blockIdx.x / (nb * chunks);
    const int b = (int)((blockIdx.x / chunks) % nb);
    const int ch = (int)(blockIdx.x % chunks);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 31, hf = lane >> 5;
    bf16x8 qf[D / 16];
    float mmq;
    int64_t qpos;
    bool qvalid;
    const uint16_t *Kr, *Vr;
    pm_setup<D>(a, rr, b, qf, mmq, qpos, qvalid, &Kr, &Vr);
    const int QRP = nb * 32;
    // the block's window outputs o_q, shared by the four waves (rows padded against bank conflicts)
    const float *ob = a.o + ((size_t)rr * QRP + b * 32) * D;
    for (int e = threadIdx.x; e < 32 * D; e += PM_THREADS) s_o[e / D][e % D] = ob[e];
    __syncthreads();
    float o2 = 0.f;
    for (int e = hf * 4; e < D; e += 8) {   // the lane's elements in pe_effect_mfma's order
        const float4 ov = *reinterpret_cast<const float4 *>(&s_o[col][e]);
        o2 = fmaf(ov.x, ov.x, o2);
        o2 = fmaf(ov.y, ov.y, o2);
        o2 = fmaf(ov.z, ov.z, o2);
        o2 = fmaf(ov.w, ov.w, o2);
    }
    o2 += __shfl_xor(o2, 32);
    const float onorm = sqrtf(o2);
    const int n_seq_idx = (int)(rr / a.Hkv);
    const int e_begin = (ch * (PM_THREADS / 64) + wave) * PSM_PAGES;
    const int n_here = a.n_pages - e_begin < PSM_PAGES ? a.n_pages - e_begin : PSM_PAGES;
    int my_first = 0, my_len = 0;
    if (lane < n_here) {
        int64_t f;
        int l;
        page_span(a, n_seq_idx, e_begin + lane, f, l);
        my_first = (int)f;
        my_len = l;
    }
    int i = 0;
    while (i < n_here) {   // i, i1 and p are the same for every lane
        const int j0 = __builtin_amdgcn_readlane(my_first, i);
        int i1 = i + 1;
        while (i1 < n_here) {
            const int f = __builtin_amdgcn_readlane(my_first, i1), l = __builtin_amdgcn_readlane(my_len, i1);
            if (f < j0 || f + l > j0 + 32) break;
            ++i1;
        }
        float w[16];
        pm_tile<D>(a, Kr, Vr, j0, qf, mmq, qpos, s_v[wave], w);
        const PvWeights pw = pv_split(w);
        for (int p = i; p < i1; ++p) {
            const int lo = __builtin_amdgcn_readlane(my_first, p) - j0;
            const int hi = lo + __builtin_amdgcn_readlane(my_len, p);
            float al = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int k = acc_row(j, hf);
                al += (k >= lo && k < hi) ? w[j] : 0.f;
            }
            al += __shfl_xor(al, 32);
            // the key blocks (tile keys 0..15, 16..31) the page touches, other keys' weights masked
            const bool in0 = hi > lo && lo < 16, in1 = hi > lo && hi > 16;
            const bf16x8 mh0 = pv_mask(pw.hi[0], 0, lo, hi), ml0 = pv_mask(pw.lo[0], 0, lo, hi);
            const bf16x8 mh1 = pv_mask(pw.hi[1], 1, lo, hi), ml1 = pv_mask(pw.lo[1], 1, lo, hi);
            float n2 = 0.f;
#pragma unroll 1
            for (int db = 0; db < NDB; ++db) {   // one accumulator live at a time
                f32x16 c = {};
                if (in0) pv_block(pv_v<D>(s_v[wave], db, 0), mh0, ml0, c);
                if (in1) pv_block(pv_v<D>(s_v[wave], db, 1), mh1, ml1, c);
#pragma unroll
                for (int r = 0; r < 16; r += 4) {
                    const float4 ov = *reinterpret_cast<const float4 *>(&s_o[col][db * 32 + acc_row(r, hf)]);
                    const float ovs[4] = {ov.x, ov.y, ov.z, ov.w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float t = fmaf(-al, ovs[u], c[r + u]);
                        n2 = fmaf(t, t, n2);
                    }
                }
            }
            n2 += __shfl_xor(n2, 32);
            float rel = 0.f, ab = 0.f;
            if (qvalid) {
                const float num = sqrtf(n2);
                const float den = 1.f - al;
                ab = den > 0.f ? num / den : INFINITY;
                rel = onorm > 0.f ? ab / onorm : (num > 0.f ? INFINITY : 0.f);
                if (!(num > 0.f)) ab = rel = 0.f;
            }
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) {
                rel = fmaxf(rel, __shfl_xor(rel, off));
                ab = fmaxf(ab, __shfl_xor(ab, off));
            }
            if (lane == 0) {
                atomic_max_nonneg(a.eff_rel + (size_t)n_seq_idx * a.n_pages + e_begin + p, rel);
                if (a.eff_abs) atomic_max_nonneg(a.eff_abs + (size_t)n_seq_idx * a.n_pages + e_begin + p, ab);
            }
        }
        i = i1;
    }
}

// Greedy joint retirement (CommitKV §3.3 Eq. 11), in two kernels per batch of
// PR_BATCH candidates.
//
// pr_terms, one workgroup per (sequence, KV head, candidate): for every query
// row q of the window, the page's weights a_qi, their sum alpha_q and the
// deletion term t_q = sum_{i in page} a_qi (v_i - o_q), written to the
// workspace. The terms do not depend on the decisions, so all candidates of a
// batch are formed in parallel.
//
// The walk works on inner products. With a_q the running deletion vector of
// the accepted set and t_q(j) the batch's terms, the joint vector of the set
// plus candidate j has squared norm |a_q|^2 + 2<a_q, t_q(j)> + |t_q(j)|^2, and
// accepting j adds t_q(j) to a_q. pr_gram forms, for every query row, |a_q|^2,
// <a_q, t_q(k)>, <t_q(j), t_q(k)> and |o_q| in parallel; pr_walk, one
// workgroup per sequence, then walks the batch on those scalars: the joint
// relative effect is maximised over the rows of every KV head and compared
// with tau_joint, and an accepted candidate updates each row's |a|^2, <a, t>
// and alpha. pr_accum adds the accepted terms to a_q and alpha_q for the next
// batch.
template <int D>
__global__ void __launch_bounds__(PR_THREADS) pr_terms(PeArgs a, const int32_t *order, int n_cand, int c0, int nc,
                                                       float *tD, float *tA) {
    __shared__ float s_k[PR_PMAX][D];
    __shared__ float s_v[PR_PMAX][D];
    const int j = blockIdx.x % nc;
    const int64_t nh = blockIdx.x / nc;
    const int n = (int)(nh / a.Hkv), h = (int)(nh % a.Hkv);
    const int page = order[(size_t)n * n_cand + c0 + j];
    if (page < 0 || page >= a.n_pages) return;  // skipped by the walk
    const int tid = threadIdx.x;
    const int QR = a.G * a.W, QRP = ((QR + 31) / 32) * 32;
    int64_t pf;
    int ps;   // this page's tokens pf .. pf + ps - 1 (ps <= PR_PMAX)
    page_span(a, n, page, pf, ps);
    const int64_t rows_local = (int64_t)gridDim.x / nc;
    const int64_t rr = (int64_t)n * a.Hkv + h;
    const int64_t gr = ((int64_t)n * a.L + a.lsel) * a.Hkv + h;
    const uint16_t *Kr = a.K + (size_t)gr * a.T * D;
    const uint16_t *Vr = a.V + (size_t)gr * a.T * D;
    for (int e = tid; e < ps * D; e += PR_THREADS) {
        const int k = e / D, cc = e % D;
        const int64_t t = pf + k;
        s_k[k][cc] = bf16_to_f32(Kr[(size_t)t * D + cc]);
        s_v[k][cc] = bf16_to_f32(Vr[(size_t)t * D + cc]);
    }
    __syncthreads();
    const RowIdx ri = split_row(gr, a.L, a.Hkv);
    const uint16_t *Qg = a.Q + ((size_t)(ri.n * a.L + ri.l) * a.Hq + (size_t)ri.h * a.G) * a.W * D;
    float *t_out = tD + ((size_t)j * rows_local + rr) * QRP * D;
    float *a_out = tA + ((size_t)j * rows_local + rr) * QRP;
    for (int q = tid; q < QR; q += PR_THREADS) {
        const int64_t qpos = a.qbase + q % a.W;
        const float mq = a.mm[rr * QRP + q];
        float p[PR_PMAX];
#pragma unroll
        for (int k = 0; k < PR_PMAX; ++k) p[k] = 0.f;
        for (int cc = 0; cc < D; cc += 8) {
            const uint4 u = *reinterpret_cast<const uint4 *>(Qg + (size_t)q * D + cc);
            const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float q0 = bf16_to_f32((uint16_t)(w4[e] & 0xFFFF)), q1 = bf16_to_f32((uint16_t)(w4[e] >> 16));
#pragma unroll
                for (int k = 0; k < PR_PMAX; ++k)
                    if (k < ps) p[k] = fmaf(q1, s_k[k][cc + 2 * e + 1], fmaf(q0, s_k[k][cc + 2 * e], p[k]));
            }
        }
        float al = 0.f;
#pragma unroll
        for (int k = 0; k < PR_PMAX; ++k) {
            const int64_t t = pf + k;
            p[k] = (k < ps && t <= qpos) ? __builtin_amdgcn_exp2f(fmaf(p[k], a.c2, -mq)) : 0.f;
            al += p[k];
        }
        const float *o = a.o + ((size_t)rr * QRP + q) * D;
        for (int cc = 0; cc < D; cc += 4) {
            const float4 o4 = *reinterpret_cast<const float4 *>(o + cc);
            float4 t4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int k = 0; k < PR_PMAX; ++k) {
                if (k < ps) {
                    t4.x = fmaf(p[k], s_v[k][cc] - o4.x, t4.x);
                    t4.y = fmaf(p[k], s_v[k][cc + 1] - o4.y, t4.y);
                    t4.z = fmaf(p[k], s_v[k][cc + 2] - o4.z, t4.z);
                    t4.w = fmaf(p[k], s_v[k][cc + 3] - o4.w, t4.w);
                }
            }
            *reinterpret_cast<float4 *>(t_out + (size_t)q * D + cc) = t4;
        }
        a_out[q] = al;
    }
}

// Gram record of query row q (GR floats): [0] |a|^2, [1 + k] <a, t(k)>,
// [9 + 8j + k] <t(j), t(k)>, [73] |o|. D/8 threads per query row.
template <int D>
__global__ void __launch_bounds__(PR_THREADS) pr_gram(PeArgs a, const int32_t *order, int n_cand, int c0, int nc,
                                                      int first, const float *tD, const float *accD, float *gram,
                                                      int64_t rows_local) {
    constexpr int TPP = D / 8;
    const int QR = a.G * a.W, QRP = ((QR + 31) / 32) * 32;
    const int64_t nrows = rows_local * QR;
    const int64_t p = (int64_t)blockIdx.x * (PR_THREADS / TPP) + threadIdx.x / TPP;
    const int sub = threadIdx.x % TPP;
    const bool valid = p < nrows;  // every lane takes part in the lane exchanges below
    const int64_t rr = valid ? p / QR : 0;
    const int q = valid ? (int)(p % QR) : 0;
    const int n = (int)(rr / a.Hkv);
    const size_t row = (size_t)rr * QRP + q;
    auto load8 = [&](const float *src, float (&x)[8]) {
        const float4 u = *reinterpret_cast<const float4 *>(src), v = *reinterpret_cast<const float4 *>(src + 4);
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
        x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
    };
    float acc[8], o[8], t[PR_BATCH][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = o[e] = 0.f;
    if (valid && !first) load8(accD + row * D + 8 * sub, acc);
    if (valid) load8(a.o + row * D + 8 * sub, o);
#pragma unroll
    for (int j = 0; j < PR_BATCH; ++j) {
#pragma unroll
        for (int e = 0; e < 8; ++e) t[j][e] = 0.f;
        if (valid && j < nc) {
            const int page = order[(size_t)n * n_cand + c0 + j];
            if (page >= 0 && page < a.n_pages) load8(tD + (((size_t)j * rows_local + rr) * QRP + q) * D + 8 * sub, t[j]);
        }
    }
    auto dot = [&](const float (&x)[8], const float (&y)[8]) {
        float s2 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s2 = fmaf(x[e], y[e], s2);
        return group_sum<TPP>(s2);
    };
    float *g = gram + row * GR;
    const float aa = dot(acc, acc), oo = dot(o, o);
    if (valid && sub == 0) {
        g[0] = aa;
        g[73] = sqrtf(oo);
    }
#pragma unroll
    for (int k = 0; k < PR_BATCH; ++k) {
        const float at = dot(acc, t[k]);
        if (valid && sub == 0) g[1 + k] = at;
#pragma unroll
        for (int j = 0; j <= k; ++j) {
            const float tt = dot(t[j], t[k]);
            if (valid && sub == 0) {
                g[9 + 8 * j + k] = tt;
                g[9 + 8 * k + j] = tt;
            }
        }
    }
}

// One workgroup per sequence; PG_RPT query rows per thread, kept in registers.
__global__ void __launch_bounds__(PG_THREADS) pr_walk(PeArgs a, const int32_t *order, int n_cand, int c0, int nc,
                                                      int first, float tau_joint, const float *tA,
                                                      const float *alphaD, const float *gram, uint8_t *accepted,
                                                      float *joint_rel, int64_t rows_local) {
    __shared__ float s_red[PG_THREADS / 64];
    __shared__ int s_accept;
    const int n = blockIdx.x;
    const int tid = threadIdx.x;
    const int QR = a.G * a.W, QRP = ((QR + 31) / 32) * 32;
    const int P = a.Hkv * QR;
    float base[PG_RPT], cross[PG_RPT][PR_BATCH], alpha[PG_RPT], onorm[PG_RPT];
    size_t rowi[PG_RPT];
    int64_t rri[PG_RPT];
    int qi[PG_RPT];
#pragma unroll
    for (int i = 0; i < PG_RPT; ++i) {
        const int pq = tid + i * PG_THREADS;
        const bool ok = pq < P;
        rri[i] = (int64_t)n * a.Hkv + (ok ? pq / QR : 0);
        qi[i] = ok ? pq % QR : 0;
        rowi[i] = (size_t)rri[i] * QRP + qi[i];
        const float *g = gram + rowi[i] * GR;
        base[i] = ok ? g[0] : 0.f;
        onorm[i] = ok ? g[73] : 0.f;
        alpha[i] = (ok && !first) ? alphaD[rowi[i]] : 0.f;
#pragma unroll
        for (int k = 0; k < PR_BATCH; ++k) cross[i][k] = (ok && k < nc) ? g[1 + k] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < PR_BATCH; ++j) {
        if (j >= nc) break;
        const int c = c0 + j;
        const int page = order[(size_t)n * n_cand + c];
        if (page < 0 || page >= a.n_pages) {
            if (tid == 0) {
                accepted[(size_t)n * n_cand + c] = 0;
                if (joint_rel) joint_rel[(size_t)n * n_cand + c] = -1.f;
            }
            continue;
        }
        float worst = 0.f, tj[PG_RPT];
#pragma unroll
        for (int i = 0; i < PG_RPT; ++i) {
            tj[i] = 0.f;
            if (tid + i * PG_THREADS >= P) continue;
            tj[i] = tA[((size_t)j * rows_local + rri[i]) * QRP + qi[i]];
            const float num2 = base[i] + 2.f * cross[i][j] + gram[rowi[i] * GR + 9 + 9 * j];
            const float num = sqrtf(fmaxf(num2, 0.f)), alj = alpha[i] + tj[i];
            float rel = 0.f;
            if (num > 0.f) rel = (1.f - alj > 0.f && onorm[i] > 0.f) ? num / ((1.f - alj) * onorm[i]) : INFINITY;
            worst = fmaxf(worst, rel);
        }
        float v = xor32_max(xor16_max(group_max<16>(worst)));
        if ((tid & 63) == 0) s_red[tid >> 6] = v;
        __syncthreads();
        if (tid == 0) {
            float m = s_red[0];
            for (int w = 1; w < PG_THREADS / 64; ++w) m = fmaxf(m, s_red[w]);
            s_accept = m <= tau_joint;
            accepted[(size_t)n * n_cand + c] = (uint8_t)s_accept;
            if (joint_rel) joint_rel[(size_t)n * n_cand + c] = m;
        }
        __syncthreads();
        if (s_accept) {
#pragma unroll
            for (int i = 0; i < PG_RPT; ++i) {
                if (tid + i * PG_THREADS >= P) continue;
                const float *gj = gram + rowi[i] * GR + 9 + 8 * j;
                base[i] += 2.f * cross[i][j] + gj[j];
                alpha[i] += tj[i];
#pragma unroll
                for (int k = 0; k < PR_BATCH; ++k) cross[i][k] += gj[k];
            }
        }
    }
}

// a_q += sum of the accepted candidates' t_q, alpha_q likewise (a_q = 0 first).
template <int D>
__global__ void __launch_bounds__(PR_THREADS) pr_accum(PeArgs a, const int32_t *order, int n_cand, int c0, int nc,
                                                       int first, const uint8_t *accepted, const float *tD,
                                                       const float *tA, float *accD, float *alphaD,
                                                       int64_t rows_local) {
    constexpr int TPP = D / 8;
    const int QR = a.G * a.W, QRP = ((QR + 31) / 32) * 32;
    const int64_t p = (int64_t)blockIdx.x * (PR_THREADS / TPP) + threadIdx.x / TPP;
    if (p >= rows_local * QR) return;
    const int sub = threadIdx.x % TPP;
    const int64_t rr = p / QR;
    const int q = (int)(p % QR);
    const int n = (int)(rr / a.Hkv);
    const size_t row = (size_t)rr * QRP + q;
    float x[8], al = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = first ? 0.f : accD[row * D + 8 * sub + e];
    if (!first) al = alphaD[row];
    for (int j = 0; j < nc; ++j) {
        if (!accepted[(size_t)n * n_cand + c0 + j]) continue;
        const float *t = tD + (((size_t)j * rows_local + rr) * QRP + q) * D + 8 * sub;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] += t[e];
        al += tA[((size_t)j * rows_local + rr) * QRP + q];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) accD[row * D + 8 * sub + e] = x[e];
    if (sub == 0) alphaD[row] = al;
}

static int pe_common_checks(const kvc_dims *dims, int32_t layer, const uint16_t *K, const uint16_t *V,
                            const uint16_t *Q, int32_t W, int64_t q_first, int32_t page_size,
                            const int32_t *page_first, const int32_t *page_len, int32_t n_pages,
                            const char *who) {
    int st = check_dims(dims, who);
    if (st != KVC_OK) return st;
    if (!K || !V || !Q) return fail(KVC_ERR_ARG, "%s: NULL tensor pointer", who);
    if (layer < 0 || layer >= dims->n_layers)
        return fail(KVC_ERR_ARG, "%s: layer %d outside [0, %d)", who, layer, dims->n_layers);
    if (W <= 0 || q_first < 0 || q_first + W > dims->n_tokens)
        return fail(KVC_ERR_ARG, "%s: window [%lld, %lld) outside the %lld cached tokens", who,
                    (long long)q_first, (long long)(q_first + W), (long long)dims->n_tokens);
    const int G = dims->n_q_heads / dims->n_kv_heads;
    if (G * W > 256) return fail(KVC_ERR_UNSUPPORTED, "%s: W*G = %d exceeds 256", who, G * W);
    if ((page_first == nullptr) != (page_len == nullptr))
        return fail(KVC_ERR_ARG, "%s: page_first and page_len go together", who);
    if (page_first) {   // event pages: page_size bounds their length
        if (page_size <= 0 || page_size > PE_TILE)
            return fail(KVC_ERR_UNSUPPORTED, "%s: event pages of up to %d tokens, not %d", who, PE_TILE, page_size);
        if (n_pages <= 0) return fail(KVC_ERR_ARG, "%s: n_pages %d must be positive", who, n_pages);
        return KVC_OK;
    }
    if (page_size <= 0 || PE_TILE % page_size)
        return fail(KVC_ERR_UNSUPPORTED, "%s: page_size %d must divide %d", who, page_size, PE_TILE);
    if (n_pages <= 0 || (int64_t)n_pages * page_size > dims->n_tokens)
        return fail(KVC_ERR_ARG, "%s: %d pages of %d tokens exceed the cache", who, n_pages, page_size);
    return KVC_OK;
}

static PeArgs pe_args(const kvc_dims *dims, int32_t layer, const uint16_t *K, const uint16_t *V,
                      const uint16_t *Q, int32_t W, int64_t q_first, int32_t page_size,
                      const int32_t *page_first, const int32_t *page_len, int32_t n_pages, const PageWs &w) {
    PeArgs a;
    a.K = K;
    a.V = V;
    a.Q = Q;
    a.T = dims->n_tokens;
    a.W = W;
    a.G = dims->n_q_heads / dims->n_kv_heads;
    a.L = dims->n_layers;
    a.Hkv = dims->n_kv_heads;
    a.Hq = dims->n_q_heads;
    a.lsel = layer;
    a.qbase = q_first;
    a.kend = q_first + W;
    a.c2 = (float)(1.4426950408889634 / std::sqrt((double)dims->head_dim));
    a.mm = w.mm;
    a.o = w.o;
    a.page_size = page_size;
    a.n_pages = n_pages;
    a.pfirst = page_first;
    a.plen = page_len;
    a.eff_rel = a.eff_abs = nullptr;
    a.opart = w.opart;
    return a;
}

// Stages 1 and 2 (statistics and outputs), shared by both entry points.
static int pe_prepare(const kvc_dims *dims, const PeArgs &a, const PageWs &w, hipStream_t s) {
    const PageGeom g = page_geom(dims, a.W, a.kend);
    WindowGeom wg{a.qbase, a.kend, a.lsel};
    int st = launch_window_stats(dims, a.K, a.Q, a.W, wg, g.rows_local, w.part, w.mm, s);
    if (st != KVC_OK) return st;
    const int chunks = (int)((a.kend + PO_CHUNK - 1) / PO_CHUNK);
    const int64_t blocks = g.rows_local * g.nb * chunks;
    if (blocks > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "page effect outputs: grid too large");
    if (dims->head_dim == 128)
        pe_out_mfma<128><<<dim3((unsigned)blocks), dim3(PM_THREADS), 0, s>>>(a, chunks);
    else
        pe_out_mfma<64><<<dim3((unsigned)blocks), dim3(PM_THREADS), 0, s>>>(a, chunks);
    if ((st = check_launch("page effect outputs")) != KVC_OK) return st;
    const int64_t n_o = g.rows_local * g.QRP * dims->head_dim;
    pe_out_reduce<<<dim3(1024), dim3(256), 0, s>>>(a.opart, w.o, n_o, chunks);
    return check_launch("page effect outputs (sum)");
}

KVC_CHECK_READER(check_read_page)

}  // namespace kvc

using namespace kvc;

// One workgroup per (sequence, run of whole pages of at most PS_TOK tokens):
// every thread sums its tokens over the sequence's L*Hkv score rows (rows in
// order, coalesced across the workgroup), then one thread per page sums the
// page's tokens in order. Fixed summation order: the result is deterministic.
static constexpr int PS_THREADS = 256;
static constexpr int PS_TOK = 1024;

__global__ void __launch_bounds__(PS_THREADS)
page_score_kernel(const float *scores, int64_t T, int64_t rows_per_seq, int page_size, int n_pages,
                  int pages_per_block, int blocks_per_seq, const int32_t *order,
                  const uint8_t *accepted, int n_cand, float *page_score) {
    __shared__ float s_tok[PS_TOK];
    __shared__ uint8_t s_ret[PS_TOK];
    const int n = blockIdx.x / blocks_per_seq;
    const int p0 = (blockIdx.x % blocks_per_seq) * pages_per_block;
    const int np = min(pages_per_block, n_pages - p0);
    const int64_t t0 = (int64_t)p0 * page_size;
    const int ntok = np * page_size;
    const int tid = threadIdx.x;
    const float *base = scores + (int64_t)n * rows_per_seq * T + t0;
    constexpr int PER = PS_TOK / PS_THREADS;
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.f;
#pragma unroll 4
    for (int64_t r = 0; r < rows_per_seq; ++r) {
        const float *row = base + r * T;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int t = tid + k * PS_THREADS;
            if (t < ntok) acc[k] += row[t];
        }
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) s_tok[tid + k * PS_THREADS] = acc[k];
    for (int e = tid; e < PS_TOK; e += PS_THREADS) s_ret[e] = 0;
    __syncthreads();
    if (order && accepted) {
        for (int c = tid; c < n_cand; c += PS_THREADS) {
            const int e = order[(int64_t)n * n_cand + c];
            if (accepted[(int64_t)n * n_cand + c] && e >= p0 && e < p0 + np) s_ret[e - p0] = 1;
        }
    }
    __syncthreads();
    for (int e = tid; e < np; e += PS_THREADS) {
        float sum = 0.f;
        for (int i = 0; i < page_size; ++i) sum += s_tok[e * page_size + i];
        page_score[(int64_t)n * n_pages + p0 + e] = s_ret[e] ? -INFINITY : sum;
    }
}

// Event pages (page_first / page_len): one workgroup per (sequence, run of
// PS_RUN pages). When the run's pages lie within PS_TOK tokens, the token sums
// are staged as in the uniform kernel; otherwise each thread sums its own page
// token by token. Both add every token over the rows in order, then the page's
// tokens in order, so the two give the same bits.
static constexpr int PS_RUN = 64;

__global__ void __launch_bounds__(PS_THREADS)
page_score_spans(const float *scores, int64_t T, int64_t rows_per_seq, int page_size, int n_pages,
                 int runs_per_seq, const int32_t *pfirst, const int32_t *plen, const int32_t *order,
                 const uint8_t *accepted, int n_cand, float *page_score) {
    __shared__ float s_tok[PS_TOK];
    __shared__ int64_t s_f[PS_RUN];
    __shared__ int s_l[PS_RUN];
    __shared__ uint8_t s_ret[PS_RUN];
    __shared__ int64_t s_span[2];
    const int n = blockIdx.x / runs_per_seq;
    const int p0 = (blockIdx.x % runs_per_seq) * PS_RUN;
    const int np = min(PS_RUN, n_pages - p0);
    const int tid = threadIdx.x;
    if (tid < 64) {   // wave 0: the run's spans and their extent
        int64_t f = 0, l = 0;
        if (tid < np) {
            f = pfirst[(int64_t)n * n_pages + p0 + tid];
            l = plen[(int64_t)n * n_pages + p0 + tid];
            KVC_NOTE(f < 0 || l < 0 || l > page_size || f + l > T, KVC_CHK_SPAN);
            f = f < 0 ? 0 : (f > T ? T : f);
            l = l < 0 ? 0 : (l > page_size ? page_size : l);
            if (l > T - f) l = T - f;
            s_f[tid] = f;
            s_l[tid] = (int)l;
            s_ret[tid] = 0;
        }
        int64_t lo = l > 0 ? f : T, hi = l > 0 ? f + l : 0;
        for (int m = 1; m < 64; m <<= 1) {
            lo = min(lo, (int64_t)__shfl_xor(lo, m));
            hi = max(hi, (int64_t)__shfl_xor(hi, m));
        }
        if (tid == 0) {
            s_span[0] = lo;
            s_span[1] = hi;
        }
    }
    __syncthreads();
    const int64_t lo = s_span[0], hi = s_span[1];
    const bool staged = hi - lo <= PS_TOK;
    if (staged && hi > lo) {
        const float *base = scores + (int64_t)n * rows_per_seq * T + lo;
        const int ntok = (int)(hi - lo);
        constexpr int PER = PS_TOK / PS_THREADS;
        float acc[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] = 0.f;
#pragma unroll 4
        for (int64_t r = 0; r < rows_per_seq; ++r) {
            const float *row = base + r * T;
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int t = tid + k * PS_THREADS;
                if (t < ntok) acc[k] += row[t];
            }
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) s_tok[tid + k * PS_THREADS] = acc[k];
    }
    if (order && accepted) {
        for (int c = tid; c < n_cand; c += PS_THREADS) {
            const int e = order[(int64_t)n * n_cand + c];
            if (accepted[(int64_t)n * n_cand + c] && e >= p0 && e < p0 + np) s_ret[e - p0] = 1;
        }
    }
    __syncthreads();
    for (int e = tid; e < np; e += PS_THREADS) {
        float sum = 0.f;
        if (staged) {
            for (int i = 0; i < s_l[e]; ++i) sum += s_tok[s_f[e] - lo + i];
        } else {
            const float *base = scores + (int64_t)n * rows_per_seq * T + s_f[e];
            for (int i = 0; i < s_l[e]; ++i) {
                float tok = 0.f;
                for (int64_t r = 0; r < rows_per_seq; ++r) tok += base[r * T + i];
                sum += tok;
            }
        }
        page_score[(int64_t)n * n_pages + p0 + e] = s_ret[e] ? -INFINITY : sum;
    }
}

// Page list -> token list, one workgroup per sequence: runs of PT_THREADS
// listed pages, each thread placing its page's tokens after an exclusive scan
// of the page lengths.
static constexpr int PT_THREADS = 256;

__global__ void __launch_bounds__(PT_THREADS)
page_tokens_kernel(int64_t T, int page_size, int n_pages, const int32_t *pfirst, const int32_t *plen,
                   const int32_t *pages, const int32_t *n_listed, int list_stride, int32_t *tokens,
                   int32_t *n_tokens, int out_stride) {
    __shared__ int s_wave[PT_THREADS / 64];
    const int n = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int listed = n_listed[n];
    KVC_NOTE(listed > list_stride, KVC_CHK_COUNT);
    listed = listed < 0 ? 0 : (listed > list_stride ? list_stride : listed);
    int64_t total = 0;
    int32_t *out = tokens + (int64_t)n * out_stride;
    for (int c0 = 0; c0 < listed; c0 += PT_THREADS) {
        const int c = c0 + tid;
        int64_t f = 0;
        int len = 0;
        if (c < listed) {
            const int e = pages[(int64_t)n * list_stride + c];
            if (e >= 0 && e < n_pages) {
                if (pfirst) {
                    int64_t ff = pfirst[(int64_t)n * n_pages + e], ll = plen[(int64_t)n * n_pages + e];
                    KVC_NOTE(ff < 0 || ll < 0 || ll > page_size || ff + ll > T, KVC_CHK_SPAN);
                    ff = ff < 0 ? 0 : (ff > T ? T : ff);
                    ll = ll < 0 ? 0 : (ll > page_size ? page_size : ll);
                    if (ll > T - ff) ll = T - ff;
                    f = ff;
                    len = (int)ll;
                } else {
                    f = (int64_t)e * page_size;
                    len = f + page_size <= T ? page_size : (int)(T - f > 0 ? T - f : 0);
                }
            }
        }
        int incl = len;
        for (int m = 1; m < 64; m <<= 1) {
            const int v = __shfl_up(incl, m);
            if (lane >= m) incl += v;
        }
        if (lane == 63) s_wave[wave] = incl;
        __syncthreads();
        int before = 0, run = 0;
        for (int w = 0; w < PT_THREADS / 64; ++w) {
            if (w < wave) before += s_wave[w];
            run += s_wave[w];
        }
        __syncthreads();
        const int64_t pos0 = total + before + incl - len;
        for (int k = 0; k < len; ++k)
            if (pos0 + k < out_stride) out[KVC_IDX(pos0 + k, out_stride, KVC_CHK_PAGE)] = (int32_t)(f + k);
        total += run;
    }
    if (tid == 0) n_tokens[n] = (int32_t)(total < INT32_MAX ? total : INT32_MAX);
}

// Pages kept under a token budget, one workgroup per sequence. The ranking
// is (score descending, index ascending), a NaN below every other score; the
// kept pages are the longest prefix of it whose lengths fit the budget. A
// three-digit radix select on the score's order key, whose histograms add
// page lengths instead of counts, finds the key k* of the first page that
// does not fit and the budget left for the pages of key k*; an ordered pass
// keeps every page of a larger key and the pages of key k* while their
// running length (in index order) stays within what is left.
static constexpr int PK_THREADS = 1024;
static constexpr int PK_BINS = 2048;

__device__ __forceinline__ uint32_t pk_order_key(float x) {
    if (x != x) return 0u;
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan over the workgroup; `total` gets the sum. Ends with a barrier.
__device__ __forceinline__ uint32_t pk_excl_scan(uint32_t v, uint32_t *s_w, uint32_t &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = v;
    for (int m = 1; m < 64; m <<= 1) {
        const uint32_t u = __shfl_up(incl, m);
        if (lane >= m) incl += u;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
    total = 0;
    for (int w = 0; w < PK_THREADS / 64; ++w) {
        const uint32_t x = s_w[w];
        if (w < wave) before += x;
        total += x;
    }
    __syncthreads();
    return before + incl - v;
}

__global__ void __launch_bounds__(PK_THREADS)
page_select_kernel(const float *page_score, int64_t T, int page_size, int n_pages, const int32_t *pfirst,
                   const int32_t *plen, uint32_t budget, int32_t *kept, int kept_stride, int32_t *n_kept,
                   int32_t *n_tokens) {
    __shared__ uint32_t hist[PK_BINS];
    __shared__ uint32_t s_w[PK_THREADS / 64];
    __shared__ uint32_t s_sel[2];
    __shared__ uint32_t s_tie_max;
    const int n = blockIdx.x, tid = threadIdx.x;
    const float *sc = page_score + (int64_t)n * n_pages;
    // page length as the other page calls clamp it (at most 4096 tokens)
    auto length = [&](int e) -> uint32_t {
        if (!pfirst) return (uint32_t)page_size;
        int64_t f = pfirst[(int64_t)n * n_pages + e], l = plen[(int64_t)n * n_pages + e];
        f = f < 0 ? 0 : (f > T ? T : f);
        l = l < 0 ? 0 : (l > page_size ? page_size : l);
        if (l > T - f) l = T - f;
        return (uint32_t)l;
    };
    uint32_t mine = 0;
    for (int e = tid; e < n_pages; e += PK_THREADS) mine += length(e);
    uint32_t total;
    pk_excl_scan(mine, s_w, total);
    const bool keep_all = total <= budget;
    uint32_t prefix = 0, mask = 0, rem = budget;
    if (!keep_all) {
        // the scope (pages whose key matches the prefix) always outweighs rem
        const int shifts[3] = {21, 10, 0}, widths[3] = {11, 11, 10};
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = shifts[pass];
            const uint32_t bmask = (1u << widths[pass]) - 1u;
            for (int i = tid; i < PK_BINS; i += PK_THREADS) hist[i] = 0;
            __syncthreads();
            for (int e = tid; e < n_pages; e += PK_THREADS) {
                const uint32_t k = pk_order_key(sc[e]);
                if ((k & mask) != prefix) continue;
                const uint32_t w = length(e);
                if (w) atomicAdd(&hist[(k >> shift) & bmask], w);
            }
            __syncthreads();
            // bins in descending order, two per thread: thread t has 2047 - 2t, 2046 - 2t
            const int b0 = PK_BINS - 1 - 2 * tid;
            const uint32_t h0 = hist[b0], h1 = hist[b0 - 1];
            uint32_t dummy;
            const uint32_t before = pk_excl_scan(h0 + h1, s_w, dummy);
            if (before <= rem && rem - before < h0) {
                s_sel[0] = (uint32_t)b0;
                s_sel[1] = rem - before;
            } else if (before + h0 <= rem && rem - before - h0 < h1) {
                s_sel[0] = (uint32_t)(b0 - 1);
                s_sel[1] = rem - before - h0;
            }
            __syncthreads();
            prefix |= s_sel[0] << shift;
            mask |= bmask << shift;
            rem = s_sel[1];
            __syncthreads();
        }
    }
    // prefix = k*, rem = the budget left for the pages of key k*
    if (tid == 0) s_tie_max = 0;
    __syncthreads();
    int32_t *out = kept + (int64_t)n * kept_stride;
    uint32_t tie_run = 0, count = 0;
    for (int e0 = 0; e0 < n_pages; e0 += PK_THREADS) {
        const int e = e0 + tid;
        uint32_t key = 0, w = 0;
        if (e < n_pages) {
            key = pk_order_key(sc[e]);
            w = length(e);
        }
        const bool tie = !keep_all && e < n_pages && key == prefix;
        uint32_t tie_sum;
        const uint32_t tie_incl = tie_run + pk_excl_scan(tie ? w : 0u, s_w, tie_sum) + (tie ? w : 0u);
        const bool keep = e < n_pages && (keep_all || key > prefix || (tie && tie_incl <= rem));
        if (keep && tie) atomicMax(&s_tie_max, tie_incl);
        uint32_t n_chunk;
        const uint32_t slot = count + pk_excl_scan(keep ? 1u : 0u, s_w, n_chunk);
        if (keep && slot < (uint32_t)kept_stride) out[slot] = e;
        tie_run += tie_sum;
        count += n_chunk;
    }
    __syncthreads();
    if (tid == 0) {
        n_kept[n] = (int32_t)count;
        if (n_tokens) n_tokens[n] = (int32_t)(keep_all ? total : budget - rem + s_tie_max);
    }
}

extern "C" size_t kvc_page_workspace_bytes(const kvc_dims *dims, int32_t W, int64_t q_first) {
    if (check_dims(dims, "kvc_page_workspace_bytes") != KVC_OK) return 0;
    if (W <= 0 || q_first < 0) {
        fail(KVC_ERR_ARG, "kvc_page_workspace_bytes: bad window");
        return 0;
    }
    return page_ws_layout(dims, W, q_first + W, nullptr, nullptr);
}

extern "C" int kvc_page_effect(const kvc_dims *dims, int32_t layer, const uint16_t *K, const uint16_t *V,
                               const uint16_t *Q_win, int32_t W, int64_t q_first, int32_t page_size,
                               const int32_t *page_first, const int32_t *page_len, int32_t n_pages,
                               float *effect_rel, float *effect_abs, void *ws, size_t ws_bytes, void *stream) {
    int st = pe_common_checks(dims, layer, K, V, Q_win, W, q_first, page_size, page_first, page_len, n_pages,
                              "kvc_page_effect");
    if (st != KVC_OK) return st;
    if (!effect_rel) return fail(KVC_ERR_ARG, "kvc_page_effect: effect_rel is NULL");
    const size_t need = page_ws_layout(dims, W, q_first + W, nullptr, nullptr);
    if (!ws || ws_bytes < need)
        return fail(KVC_ERR_WORKSPACE, "kvc_page_effect: workspace %zu < %zu bytes", ws_bytes, need);
    PageWs w;
    page_ws_layout(dims, W, q_first + W, ws, &w);
    PeArgs a = pe_args(dims, layer, K, V, Q_win, W, q_first, page_size, page_first, page_len, n_pages, w);
    a.eff_rel = effect_rel;
    a.eff_abs = effect_abs;
    hipStream_t s = as_stream(stream);
    const int64_t n_out = (int64_t)dims->n_seq * n_pages;
    fill_f32<<<dim3(256), dim3(256), 0, s>>>(effect_rel, n_out, 0.f);
    if (effect_abs) fill_f32<<<dim3(256), dim3(256), 0, s>>>(effect_abs, n_out, 0.f);
    if ((st = check_launch("kvc_page_effect clear")) != KVC_OK) return st;
    if ((st = pe_prepare(dims, a, w, s)) != KVC_OK) return st;
    const PageGeom g = page_geom(dims, W, q_first + W);
    if (page_first && page_size <= 32) {
        const int per_wg = PSM_PAGES * (PM_THREADS / 64);
        const int chunks = (n_pages + per_wg - 1) / per_wg;
        const int64_t blocks = g.rows_local * g.nb * chunks;
        if (blocks > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "kvc_page_effect: grid too large");
        if (dims->head_dim == 128)
            pe_effect_spans_mfma<128><<<dim3((unsigned)blocks), dim3(PM_THREADS), 0, s>>>(a, chunks);
        else
            pe_effect_spans_mfma<64><<<dim3((unsigned)blocks), dim3(PM_THREADS), 0, s>>>(a, chunks);
        return check_launch("kvc_page_effect");
    }
    if (page_first) {   // event pages of 33 .. 64 tokens
        const int cpr = (n_pages + PE_SPAN_CHUNK - 1) / PE_SPAN_CHUNK;
        const int64_t blocks = g.rows_local * g.nb * cpr;
        if (blocks > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "kvc_page_effect: grid too large");
        if (dims->head_dim == 128)
            pe_effect_spans<128><<<dim3((unsigned)blocks), dim3(PE_THREADS), 0, s>>>(a, cpr);
        else
            pe_effect_spans<64><<<dim3((unsigned)blocks), dim3(PE_THREADS), 0, s>>>(a, cpr);
        return check_launch("kvc_page_effect");
    }
    const int64_t n_tok = (int64_t)n_pages * page_size;
    if (page_size == 8 || page_size == 16 || page_size == 32) {
        const int chunks = (int)((n_tok + PO_CHUNK - 1) / PO_CHUNK);
        const int64_t blocks = g.rows_local * g.nb * chunks;
        if (blocks > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "kvc_page_effect: grid too large");
        const dim3 grid((unsigned)blocks), block(PM_THREADS);
#define PEM(DD, PP) pe_effect_mfma<DD, PP><<<grid, block, 0, s>>>(a, chunks)
        if (dims->head_dim == 128) {
            if (page_size == 8) PEM(128, 8);
            else if (page_size == 16) PEM(128, 16);
            else PEM(128, 32);
        } else {
            if (page_size == 8) PEM(64, 8);
            else if (page_size == 16) PEM(64, 16);
            else PEM(64, 32);
        }
#undef PEM
        return check_launch("kvc_page_effect");
    }
    const int cpr = (int)((n_tok + PE_PAGE_CHUNK - 1) / PE_PAGE_CHUNK);
    const int64_t blocks = g.rows_local * g.nb * cpr;
    if (blocks > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "kvc_page_effect: grid too large");
    if (dims->head_dim == 128)
        pe_effect<128><<<dim3((unsigned)blocks), dim3(PE_THREADS), 0, s>>>(a, cpr);
    else
        pe_effect<64><<<dim3((unsigned)blocks), dim3(PE_THREADS), 0, s>>>(a, cpr);
    return check_launch("kvc_page_effect");
}

extern "C" int kvc_page_retire(const kvc_dims *dims, int32_t layer, const uint16_t *K, const uint16_t *V,
                               const uint16_t *Q_win, int32_t W, int64_t q_first, int32_t page_size,
                               const int32_t *page_first, const int32_t *page_len, int32_t n_pages,
                               const int32_t *order, int32_t n_cand, float tau_joint, uint8_t *accepted,
                               float *joint_rel, void *ws, size_t ws_bytes, void *stream) {
    int st = pe_common_checks(dims, layer, K, V, Q_win, W, q_first, page_size, page_first, page_len, n_pages,
                              "kvc_page_retire");
    if (st != KVC_OK) return st;
    if (!order || !accepted || n_cand <= 0)
        return fail(KVC_ERR_ARG, "kvc_page_retire: order/accepted missing or n_cand <= 0");
    if (page_size > PR_PMAX)
        return fail(KVC_ERR_UNSUPPORTED, "kvc_page_retire: page_size %d above %d", page_size, PR_PMAX);
    const size_t need = page_ws_layout(dims, W, q_first + W, nullptr, nullptr);
    if (!ws || ws_bytes < need)
        return fail(KVC_ERR_WORKSPACE, "kvc_page_retire: workspace %zu < %zu bytes", ws_bytes, need);
    PageWs w;
    page_ws_layout(dims, W, q_first + W, ws, &w);
    PeArgs a = pe_args(dims, layer, K, V, Q_win, W, q_first, page_size, page_first, page_len, n_pages, w);
    hipStream_t s = as_stream(stream);
    if ((st = pe_prepare(dims, a, w, s)) != KVC_OK) return st;
    const PageGeom g = page_geom(dims, W, q_first + W);
    if ((int64_t)dims->n_kv_heads * g.QR > (int64_t)PG_THREADS * PG_RPT)
        return fail(KVC_ERR_UNSUPPORTED, "kvc_page_retire: %d KV heads x %d rows too many", dims->n_kv_heads, g.QR);
    const int64_t rows_q = g.rows_local * g.QR;
    const int64_t qblocks = (rows_q + PR_THREADS / (dims->head_dim / 8) - 1) / (PR_THREADS / (dims->head_dim / 8));
    if (qblocks > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "kvc_page_retire: grid too large");
    for (int c0 = 0; c0 < n_cand; c0 += PR_BATCH) {
        const int nc = n_cand - c0 < PR_BATCH ? n_cand - c0 : PR_BATCH;
        const int first = c0 == 0, last = c0 + PR_BATCH >= n_cand;
        const dim3 tgrid((unsigned)(g.rows_local * nc)), qgrid((unsigned)qblocks);
        if (dims->head_dim == 128) {
            pr_terms<128><<<tgrid, dim3(PR_THREADS), 0, s>>>(a, order, n_cand, c0, nc, w.tD, w.tA);
            pr_gram<128><<<qgrid, dim3(PR_THREADS), 0, s>>>(a, order, n_cand, c0, nc, first, w.tD, w.accD, w.gram,
                                                             g.rows_local);
        } else {
            pr_terms<64><<<tgrid, dim3(PR_THREADS), 0, s>>>(a, order, n_cand, c0, nc, w.tD, w.tA);
            pr_gram<64><<<qgrid, dim3(PR_THREADS), 0, s>>>(a, order, n_cand, c0, nc, first, w.tD, w.accD, w.gram,
                                                            g.rows_local);
        }
        pr_walk<<<dim3(dims->n_seq), dim3(PG_THREADS), 0, s>>>(a, order, n_cand, c0, nc, first, tau_joint, w.tA,
                                                                w.alphaD, w.gram, accepted, joint_rel, g.rows_local);
        if (!last) {  // the next batch starts from the accepted set
            if (dims->head_dim == 128)
                pr_accum<128><<<qgrid, dim3(PR_THREADS), 0, s>>>(a, order, n_cand, c0, nc, first, accepted, w.tD,
                                                                  w.tA, w.accD, w.alphaD, g.rows_local);
            else
                pr_accum<64><<<qgrid, dim3(PR_THREADS), 0, s>>>(a, order, n_cand, c0, nc, first, accepted, w.tD,
                                                                 w.tA, w.accD, w.alphaD, g.rows_local);
        }
        if ((st = check_launch("kvc_page_retire")) != KVC_OK) return st;
    }
    return KVC_OK;
}

extern "C" int kvc_page_scores(const kvc_dims *dims, const float *scores, int32_t page_size,
                               const int32_t *page_first, const int32_t *page_len, int32_t n_pages,
                               const int32_t *order, const uint8_t *accepted, int32_t n_cand,
                               float *page_score, void *stream) {
    int st = check_dims(dims, "kvc_page_scores");
    if (st != KVC_OK) return st;
    if (!scores || !page_score) return fail(KVC_ERR_ARG, "kvc_page_scores: NULL tensor pointer");
    if (page_size <= 0 || page_size > PS_TOK)
        return fail(KVC_ERR_UNSUPPORTED, "kvc_page_scores: page_size %d outside [1, %d]", page_size, PS_TOK);
    if ((page_first == nullptr) != (page_len == nullptr))
        return fail(KVC_ERR_ARG, "kvc_page_scores: page_first and page_len go together");
    if (n_pages <= 0 || (!page_first && (int64_t)n_pages * page_size > dims->n_tokens))
        return fail(KVC_ERR_ARG, "kvc_page_scores: %d pages of %d tokens exceed the cache", n_pages, page_size);
    if ((order == nullptr) != (accepted == nullptr) || (order && n_cand <= 0))
        return fail(KVC_ERR_ARG, "kvc_page_scores: order and accepted go together, with n_cand > 0");
    const int64_t rows_per_seq_s = (int64_t)dims->n_layers * dims->n_kv_heads;
    if (page_first) {
        const int runs = (n_pages + PS_RUN - 1) / PS_RUN;
        const int64_t blocks = (int64_t)dims->n_seq * runs;
        if (blocks > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "kvc_page_scores: grid too large");
        page_score_spans<<<dim3((unsigned)blocks), dim3(PS_THREADS), 0, as_stream(stream)>>>(
            scores, dims->n_tokens, rows_per_seq_s, page_size, n_pages, runs, page_first, page_len, order,
            accepted, order ? n_cand : 0, page_score);
        return check_launch("kvc_page_scores");
    }
    const int ppb = PS_TOK / page_size;
    const int bps = (n_pages + ppb - 1) / ppb;
    const int64_t blocks = (int64_t)dims->n_seq * bps;
    if (blocks > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "kvc_page_scores: grid too large");
    const int64_t rows_per_seq = (int64_t)dims->n_layers * dims->n_kv_heads;
    page_score_kernel<<<dim3((unsigned)blocks), dim3(PS_THREADS), 0, as_stream(stream)>>>(
        scores, dims->n_tokens, rows_per_seq, page_size, n_pages, ppb, bps, order, accepted,
        order ? n_cand : 0, page_score);
    return check_launch("kvc_page_scores");
}

extern "C" int kvc_page_select(const kvc_dims *dims, const float *page_score, int32_t page_size,
                               const int32_t *page_first, const int32_t *page_len, int32_t n_pages, int32_t budget,
                               int32_t *kept, int32_t kept_stride, int32_t *n_kept, int32_t *n_tokens,
                               void *stream) {
    int st = check_dims(dims, "kvc_page_select");
    if (st != KVC_OK) return st;
    if (!page_score || !kept || !n_kept) return fail(KVC_ERR_ARG, "kvc_page_select: NULL pointer");
    if ((page_first == nullptr) != (page_len == nullptr))
        return fail(KVC_ERR_ARG, "kvc_page_select: page_first and page_len go together");
    if (page_size <= 0 || page_size > 4096)
        return fail(KVC_ERR_UNSUPPORTED, "kvc_page_select: page_size %d outside [1, 4096]", page_size);
    if (n_pages <= 0 || n_pages >= (1 << 20))
        return fail(KVC_ERR_UNSUPPORTED, "kvc_page_select: n_pages %d outside [1, 2^20)", n_pages);
    if (!page_first && (int64_t)n_pages * page_size > dims->n_tokens)
        return fail(KVC_ERR_ARG, "kvc_page_select: %d pages of %d tokens exceed the cache", n_pages, page_size);
    if (budget < 0 || kept_stride <= 0)
        return fail(KVC_ERR_ARG, "kvc_page_select: budget %d and kept_stride %d", budget, kept_stride);
    page_select_kernel<<<dim3((unsigned)dims->n_seq), dim3(PK_THREADS), 0, as_stream(stream)>>>(
        page_score, dims->n_tokens, page_size, n_pages, page_first, page_len, (uint32_t)budget, kept, kept_stride,
        n_kept, n_tokens);
    return check_launch("kvc_page_select");
}

extern "C" int kvc_page_tokens(const kvc_dims *dims, int32_t page_size, const int32_t *page_first,
                               const int32_t *page_len, int32_t n_pages, const int32_t *pages,
                               const int32_t *n_listed, int32_t list_stride, int32_t *tokens, int32_t *n_tokens,
                               int32_t out_stride, void *stream) {
    int st = check_dims(dims, "kvc_page_tokens");
    if (st != KVC_OK) return st;
    if (!pages || !n_listed || !tokens || !n_tokens) return fail(KVC_ERR_ARG, "kvc_page_tokens: NULL pointer");
    if ((page_first == nullptr) != (page_len == nullptr))
        return fail(KVC_ERR_ARG, "kvc_page_tokens: page_first and page_len go together");
    if (page_size <= 0 || page_size > (1 << 20) || n_pages <= 0 || list_stride <= 0 || out_stride <= 0)
        return fail(KVC_ERR_ARG, "kvc_page_tokens: page_size %d (at most 2^20), n_pages %d, list_stride %d, "
                    "out_stride %d must be positive", page_size, n_pages, list_stride, out_stride);
    page_tokens_kernel<<<dim3((unsigned)dims->n_seq), dim3(PT_THREADS), 0, as_stream(stream)>>>(
        dims->n_tokens, page_size, n_pages, page_first, page_len, pages, n_listed, list_stride, tokens, n_tokens,
        out_stride);
    return check_launch("kvc_page_tokens");
}
