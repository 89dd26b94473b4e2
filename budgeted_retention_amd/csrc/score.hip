// kvc_score: observation-window attention score.
//
// Per row (sequence, layer, KV head) the G*W window queries of the GQA group
// (query row qr = g*W + w at position T-W+w) attend causally to the T cached
// keys; the score of key j is the sum over query rows of its softmax weight
// (PASK §3.1 Eq. 1 attention, window queries as in CommitKV §3.1 Eq. 5,
// causal rule of CommitKV Eq. 6).
//
// A softmax weight needs its query row's normaliser over all T keys, so the
// keys are streamed twice:
//   pass 1  each workgroup takes CHUNK keys of one row and produces, per
//           query row, the running max and exp-sum of its logits (log2 domain);
//   merge   one workgroup per row folds the chunk partials into
//           mm[qr] = max + log2(sum) for every query row;
//   pass 2  each workgroup recomputes its chunk's logits and writes
//           score[j] = sum_qr exp2(logit*c - mm[qr]).
//
// Logits come from MFMA v_mfma_f32_32x32x16_bf16 tiles. A 32-key x 16-dim slice of
// K is loaded so that lane l holds key (l & 31), dims 8*(l>>5)..+8 of the
// slice; that register layout serves as the A operand (rows = keys) in pass 1
// and as the B operand (columns = keys) in pass 2, so one load feeds both
// orientations. Pass 1 computes C[key][qrow] (a lane owns one query row, so the
// max/sum over keys stay in-lane); pass 2 computes C[qrow][key] (a lane owns
// one key, so the sum over query rows stays in-lane). Each wave owns 32 query
// rows; a workgroup has ceil(G*W/32) waves.
#include <cmath>

#include "kvc_internal.h"

namespace kvc {

static constexpr int SCORE_CHUNK = 1024;  // keys per workgroup
static constexpr int SCORE_MAX_QR = 256;  // query rows per row (8 waves)

struct ScoreGeom {
    int64_t rows, n_chunks;
    int QR, QRP, nb;
};

static ScoreGeom score_geom(const kvc_dims *d, int32_t W) {
    ScoreGeom g;
    int G = d->n_q_heads / d->n_kv_heads;
    g.rows = n_rows(d);
    g.n_chunks = (d->n_tokens + SCORE_CHUNK - 1) / SCORE_CHUNK;
    g.QR = G * W;
    g.nb = (g.QR + 31) / 32;
    g.QRP = g.nb * 32;
    return g;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t score_workspace_bytes(const kvc_dims *d, int32_t W) {
    ScoreGeom g = score_geom(d, W);
    size_t part = (size_t)g.rows * g.n_chunks * g.QRP * sizeof(float2);
    size_t mm = (size_t)g.rows * g.QRP * sizeof(float);
    return align256(part) + align256(mm);
}

template <int D>
__global__ void __launch_bounds__(512) score_pass1(const uint16_t *__restrict__ K,
                                                   const uint16_t *__restrict__ Q, int64_t T, int W,
                                                   int G, int L, int Hkv, int Hq, int64_t n_chunks,
                                                   float c2, WindowGeom wg, float2 *__restrict__ part) {
    constexpr int S = D / 16;
    const int QR = G * W;
    const int QRP = (blockDim.x >> 6) * 32;
    const int64_t r = blockIdx.x / n_chunks;  // local row
    const int64_t chunk = blockIdx.x % n_chunks;
    const int64_t gr = wg.global_row(r, L, Hkv);
    const RowIdx ri = split_row(gr, L, Hkv);
    const uint16_t *Kr = K + (size_t)gr * T * D;
    const uint16_t *Qg = Q + ((size_t)(ri.n * L + ri.l) * Hq + (size_t)ri.h * G) * W * D;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, hf = lane >> 5;
    const int64_t qbase = wg.qbase;

    const int qrow = wave * 32 + col;
    bf16x8 qf[S];
#pragma unroll
    for (int s = 0; s < S; ++s) qf[s] = qrow < QR ? load8(Qg + (size_t)qrow * D + 16 * s + 8 * hf) : zero8();
    const int64_t qpos = qrow < QR ? qbase + qrow % W : -1;

    float m = -INFINITY, l = 0.f;
    const int64_t k0 = chunk * SCORE_CHUNK;
    const int64_t k1 = k0 + SCORE_CHUNK < wg.kend ? k0 + SCORE_CHUNK : wg.kend;
    for (int64_t j0 = k0; j0 < k1; j0 += 32) {
        const int64_t key = j0 + col;
        bf16x8 kf[S];
#pragma unroll
        for (int s = 0; s < S; ++s) kf[s] = key < T ? load8(Kr + (size_t)key * D + 16 * s + 8 * hf) : zero8();
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < S; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], acc, 0, 0, 0);
        // acc[i] = logit of key j0 + acc_row(i, hf) for query row `qrow`
        const bool all_vis = j0 + 31 <= qbase;  // every key of the tile is visible to every query
        float tmax = -INFINITY;
        if (all_vis) {
#pragma unroll
            for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, acc[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (j0 + acc_row(i, hf) <= qpos) tmax = fmaxf(tmax, acc[i]);
        }
        tmax *= c2;
        if (tmax > m) {
            l *= __builtin_amdgcn_exp2f(m - tmax);
            m = tmax;
        }
        float sum = 0.f;
        if (all_vis) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sum += __builtin_amdgcn_exp2f(fmaf(acc[i], c2, -m));
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (j0 + acc_row(i, hf) <= qpos) sum += __builtin_amdgcn_exp2f(fmaf(acc[i], c2, -m));
        }
        l += sum;
    }
    // Lanes l and l^32 hold the same query row over different keys.
    const float mo = __shfl_xor(m, 32);
    const float lo = __shfl_xor(l, 32);
    const float M = fmaxf(m, mo);
    float Ls = 0.f;
    if (M > -INFINITY) Ls = l * __builtin_amdgcn_exp2f(m - M) + lo * __builtin_amdgcn_exp2f(mo - M);
    if (hf == 0) part[((size_t)r * n_chunks + chunk) * QRP + qrow] = make_float2(M, Ls);
}

__global__ void score_merge(const float2 *__restrict__ part, int64_t n_chunks, int QR, int QRP,
                            float *__restrict__ mm) {
    const int64_t r = blockIdx.x;
    const int q = threadIdx.x;
    if (q >= QRP) return;
    if (q >= QR) {
        mm[r * QRP + q] = INFINITY;  // padding rows contribute exp2(-inf) = 0
        return;
    }
    const float2 *p = part + (size_t)r * n_chunks * QRP + q;
    float M = -INFINITY;
    for (int64_t c = 0; c < n_chunks; ++c) M = fmaxf(M, p[c * QRP].x);
    float S = 0.f;
    for (int64_t c = 0; c < n_chunks; ++c) {
        float2 v = p[c * QRP];
        if (v.y > 0.f) S += v.y * exp2f(v.x - M);
    }
    mm[r * QRP + q] = M + log2f(S);
}

template <int D>
__global__ void __launch_bounds__(512) score_pass2(const uint16_t *__restrict__ K,
                                                   const uint16_t *__restrict__ Q, int64_t T, int W,
                                                   int G, int L, int Hkv, int Hq, int64_t n_chunks,
                                                   float c2, const float *__restrict__ mm,
                                                   float *__restrict__ scores) {
    const WindowGeom wg{T - W, T, -1};
    constexpr int S = D / 16;
    extern __shared__ float red[];  // [nb][SCORE_CHUNK]
    const int QR = G * W;
    const int nb = blockDim.x >> 6;
    const int QRP = nb * 32;
    const int64_t r = blockIdx.x / n_chunks;
    const int64_t chunk = blockIdx.x % n_chunks;
    const RowIdx ri = split_row(wg.global_row(r, L, Hkv), L, Hkv);
    const uint16_t *Kr = K + (size_t)r * T * D;
    const uint16_t *Qg = Q + ((size_t)(ri.n * L + ri.l) * Hq + (size_t)ri.h * G) * W * D;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, hf = lane >> 5;

    bf16x8 qf[S];
    {
        const int qrow = wave * 32 + col;
#pragma unroll
        for (int s = 0; s < S; ++s)
            qf[s] = qrow < QR ? load8(Qg + (size_t)qrow * D + 16 * s + 8 * hf) : zero8();
    }
    // This lane's 16 accumulator rows.
    float mmi[16];
    int64_t qpos[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int qr = wave * 32 + acc_row(i, hf);
        mmi[i] = mm[r * QRP + qr];
        qpos[i] = qr < QR ? wg.qbase + qr % W : -1;
    }

    const int64_t k0 = chunk * SCORE_CHUNK;
    const int64_t k1 = k0 + SCORE_CHUNK < T ? k0 + SCORE_CHUNK : T;
    for (int64_t j0 = k0; j0 < k1; j0 += 32) {
        const int64_t key = j0 + col;
        bf16x8 kf[S];
#pragma unroll
        for (int s = 0; s < S; ++s) kf[s] = key < T ? load8(Kr + (size_t)key * D + 16 * s + 8 * hf) : zero8();
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < S; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[s], kf[s], acc, 0, 0, 0);
        // acc[i] = logit of query row wave*32 + acc_row(i, hf) for key `key`
        float p = 0.f;
        if (j0 + 31 <= wg.qbase) {
#pragma unroll
            for (int i = 0; i < 16; ++i) p += __builtin_amdgcn_exp2f(fmaf(acc[i], c2, -mmi[i]));
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (key <= qpos[i]) p += __builtin_amdgcn_exp2f(fmaf(acc[i], c2, -mmi[i]));
        }
        p += __shfl_xor(p, 32);
        if (hf == 0) red[wave * SCORE_CHUNK + (j0 - k0) + col] = p;
    }
    __syncthreads();
    for (int64_t t = threadIdx.x; t < k1 - k0; t += blockDim.x) {
        float s = 0.f;
        for (int b = 0; b < nb; ++b) s += red[b * SCORE_CHUNK + t];
        scores[(size_t)r * T + k0 + t] = s;
    }
}

int launch_window_stats(const kvc_dims *d, const uint16_t *K, const uint16_t *Q, int W, WindowGeom wg,
                        int64_t rows_local, float2 *part, float *mm, hipStream_t s) {
    const int G = d->n_q_heads / d->n_kv_heads;
    const int QR = G * W, nb = (QR + 31) / 32, QRP = nb * 32;
    const int64_t n_chunks = window_chunks(wg.kend);
    const int64_t blocks = rows_local * n_chunks;
    if (blocks > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "window stats: grid too large");
    const float c2 = (float)(1.4426950408889634 / std::sqrt((double)d->head_dim));
    const int L = d->n_layers, Hkv = d->n_kv_heads, Hq = d->n_q_heads;
    const int64_t T = d->n_tokens;
    if (d->head_dim == 128)
        score_pass1<128><<<dim3((unsigned)blocks), dim3(nb * 64), 0, s>>>(K, Q, T, W, G, L, Hkv, Hq, n_chunks,
                                                                        c2, wg, part);
    else
        score_pass1<64><<<dim3((unsigned)blocks), dim3(nb * 64), 0, s>>>(K, Q, T, W, G, L, Hkv, Hq, n_chunks,
                                                                       c2, wg, part);
    int st = check_launch("window stats pass 1");
    if (st != KVC_OK) return st;
    score_merge<<<dim3((unsigned)rows_local), dim3(QRP), 0, s>>>(part, n_chunks, QR, QRP, mm);
    return check_launch("window stats merge");
}

int64_t window_chunks(int64_t kend) { return (kend + SCORE_CHUNK - 1) / SCORE_CHUNK; }

}  // namespace kvc

using namespace kvc;

extern "C" int kvc_score(const kvc_dims *dims, const uint16_t *K, const uint16_t *Q_obs, int32_t W,
                         float *scores, void *ws, size_t ws_bytes, void *stream) {
    int st = check_dims(dims, "kvc_score");
    if (st != KVC_OK) return st;
    if (!K || !Q_obs || !scores) return fail(KVC_ERR_ARG, "kvc_score: NULL tensor pointer");
    if (W <= 0 || W > dims->n_tokens)
        return fail(KVC_ERR_ARG, "kvc_score: W=%d must be in [1, T=%lld]", W, (long long)dims->n_tokens);
    const int G = dims->n_q_heads / dims->n_kv_heads;
    if ((int64_t)G * W > SCORE_MAX_QR)
        return fail(KVC_ERR_UNSUPPORTED, "kvc_score: W*G=%d exceeds %d query rows", G * W, SCORE_MAX_QR);
    const size_t need = score_workspace_bytes(dims, W);
    if (!ws || ws_bytes < need)
        return fail(KVC_ERR_WORKSPACE, "kvc_score: workspace %zu < %zu bytes", ws_bytes, need);

    const ScoreGeom g = score_geom(dims, W);
    const int64_t blocks = g.rows * g.n_chunks;
    if (blocks > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "kvc_score: grid too large");
    float2 *part = reinterpret_cast<float2 *>(ws);
    float *mm = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) +
                                          align256((size_t)g.rows * g.n_chunks * g.QRP * sizeof(float2)));
    const float c2 = (float)(1.4426950408889634 / std::sqrt((double)dims->head_dim));
    hipStream_t s = as_stream(stream);
    const int threads = g.nb * 64;
    const size_t red_bytes = (size_t)g.nb * SCORE_CHUNK * sizeof(float);
    const int L = dims->n_layers, Hkv = dims->n_kv_heads, Hq = dims->n_q_heads;
    const int64_t T = dims->n_tokens;
    const WindowGeom wgeo{T - W, T, -1};
    if (dims->head_dim == 128) {
        score_pass1<128><<<dim3((unsigned)blocks), dim3(threads), 0, s>>>(K, Q_obs, T, W, G, L, Hkv, Hq,
                                                                          g.n_chunks, c2, wgeo, part);
    } else {
        score_pass1<64><<<dim3((unsigned)blocks), dim3(threads), 0, s>>>(K, Q_obs, T, W, G, L, Hkv, Hq,
                                                                         g.n_chunks, c2, wgeo, part);
    }
    if ((st = check_launch("kvc_score pass 1")) != KVC_OK) return st;
    score_merge<<<dim3((unsigned)g.rows), dim3(g.QRP), 0, s>>>(part, g.n_chunks, g.QR, g.QRP, mm);
    if ((st = check_launch("kvc_score merge")) != KVC_OK) return st;
    if (dims->head_dim == 128) {
        score_pass2<128><<<dim3((unsigned)blocks), dim3(threads), red_bytes, s>>>(
            K, Q_obs, T, W, G, L, Hkv, Hq, g.n_chunks, c2, mm, scores);
    } else {
        score_pass2<64><<<dim3((unsigned)blocks), dim3(threads), red_bytes, s>>>(
            K, Q_obs, T, W, G, L, Hkv, Hq, g.n_chunks, c2, mm, scores);
    }
    return check_launch("kvc_score pass 2");
}
