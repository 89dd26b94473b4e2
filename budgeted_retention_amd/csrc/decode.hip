// kvc_decode_attn: one decode query per query head over a compacted cache.
//
// PASK §3.1 Eq. 1 attention; PASK Appendix B.5 runs it over disjoint
// partitions (a bf16 pool, an int8 pool dequantised as code*scale) with fp32
// scores, statistics and accumulation and a bf16 output, merging partitions by
// Eq. 15: with per-partition score maximum v_j, exp-sum l_j and unnormalised
// value sum u_j, o = sum_j e^{v_j - v} u_j / sum_j e^{v_j - v} l_j, v = max_j v_j;
// empty partitions contribute nothing. Query head g of a row's group reads the
// row's KV head (grouped-query attention).
//
// Split-KV: every workgroup takes one chunk of DEC_CHUNK keys of one row (from
// either partition) for all G query heads of the row and writes its (v, l, u)
// partial to the workspace; a merge kernel applies Eq. 15 across the chunks of
// both partitions.
// The bf16 partition may be paged: token t of a row then lives in slot
// block_table[n][t / page_size] * page_size + t % page_size of the row's storage.
//
// kvc_decode_attn_h2o adds H2O's cumulative attention (PACE §2 background,
// §3.1 "cumulative attention score"): the partial kernel also writes every
// key's scaled logit per head, the merge writes each head's log2 normaliser,
// and a third kernel adds sum_g 2^(logit - lse2_g) to the key's running score.
#include <cmath>

#include "kvc_internal.h"

namespace kvc {

static constexpr int DEC_CHUNK = 256;
static constexpr int DEC_THREADS = 256;
static constexpr int DEC_MAX_G = 16;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct DecodeArgs {
    const uint16_t *q;
    const uint16_t *K, *V;
    const int32_t *n_h;
    int64_t stride_h;
    const int32_t *block_table;
    int32_t page_size, blocks_per_seq;
    const int8_t *Kq, *Vq;    // int8 codes, or INT4 nibble pairs (low_bits 4)
    const uint16_t *Ks, *Vs;
    const int32_t *n_l;
    int64_t stride_l;
    int low_bits;             // 8 or 4
    int L, Hkv, Hq, G;
    int chunks_h, chunks_l;  // chunk slots per row for each partition
    float c2;                // log2(e) / sqrt(d)
    float *part;             // [rows][chunks_h + chunks_l][G][D + 2]
    uint16_t *o;
    float *lse;
    float *logit;            // H2O: [rows][G][chunks_h * DEC_CHUNK] log2-scaled logits, or NULL
    float *lse2;             // H2O: [rows][G] log2 normalisers
};

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
    const int ex = (h >> 10) & 31, mt = h & 1023;
    const float v = ex == 0 ? ldexpf((float)mt, -24) : ldexpf((float)(1024 + mt), ex - 25);
    return (h & 0x8000) ? -v : v;
}

__device__ __forceinline__ float block_reduce(float v, bool is_max, float *s_red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float o = __shfl_xor(v, off);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    if (lane == 0) s_red[wave] = v;
    __syncthreads();
    float r = s_red[0];
    for (int w = 1; w < DEC_THREADS / 64; ++w) r = is_max ? fmaxf(r, s_red[w]) : r + s_red[w];
    __syncthreads();
    return r;
}

// Storage slot of token t of row r in the bf16 partition, or -1 when a paged
// block id points outside the row's storage.
__device__ __forceinline__ int64_t bf16_slot(const DecodeArgs &a, int n, int t) {
    if (!a.block_table) return t;
    const int blk = a.block_table[(size_t)n * a.blocks_per_seq + t / a.page_size];
    const int64_t s = (int64_t)blk * a.page_size + t % a.page_size;
    KVC_NOTE(blk < 0 || s >= a.stride_h, KVC_CHK_BLOCK);
    return (blk < 0 || s >= a.stride_h) ? -1 : s;
}

// One chunk of DEC_CHUNK keys of one row (either partition) for the GM >= G
// query heads of the row's group. A key is owned by TPK = D/8 threads, each
// holding 8 consecutive dimensions: every thread issues the loads of all its
// keys (16 bytes each) before using any, partial dot products are summed
// across the key's threads with shuffles, and the softmax statistics need
// three barriers for all heads together.
static_assert(DEC_CHUNK == DEC_THREADS, "the statistics map one thread to one key");

// LOWB: 0 = the bf16 partition, 8 = int8 codes, 4 = INT4 codes (two signed
// nibbles per byte, dimension 2i in the low nibble of byte i).
template <int D, int GM, int LOWB>
__global__ void __launch_bounds__(DEC_THREADS) decode_partial(DecodeArgs a) {
    constexpr bool LOW = LOWB != 0;
    constexpr int CB = LOWB == 4 ? D / 2 : D;   // code bytes per low-precision row
    constexpr int TPK = D / 8;                  // threads per key
    constexpr int KPI = DEC_THREADS / TPK;      // keys per pass over the block
    constexpr int ITER = DEC_CHUNK / KPI;       // passes per chunk
    constexpr int NW = DEC_THREADS / 64;
    __shared__ float s_q[GM][D];
    __shared__ float s_p[GM][DEC_CHUNK];        // logits, then weights
    __shared__ float s_w[NW][GM];
    __shared__ float s_acc[NW][GM][D];

    // the bf16 partition's chunks come first in a row's partial slots
    const int slots = a.chunks_h + a.chunks_l;
    const int own = LOW ? a.chunks_l : a.chunks_h;
    const int64_t r = blockIdx.x / own;
    const int chunk = blockIdx.x % own;
    const int slot = LOW ? a.chunks_h + chunk : chunk;
    constexpr bool low = LOW;
    const RowIdx ri = split_row(r, a.L, a.Hkv);
    const int G = a.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = tid % TPK, kin = tid / TPK;  // dimension group, key within a pass
    float *out = a.part + ((size_t)r * slots + slot) * G * (D + 2);

    const int64_t k0 = (int64_t)chunk * DEC_CHUNK;
    const uint16_t *qrow = a.q + ((size_t)(ri.n * a.L + ri.l) * a.Hq + (size_t)ri.h * G) * D;
    // bf16 keys: the query's bf16 pairs as stored (dot2 on packed bf16, fp32
    // accumulation), loaded before the row's count arrives. Heads past G
    // repeat head G-1; nothing of theirs is written.
    uint32_t qp[LOW ? 1 : GM][4];
    if (!LOW) {
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            const uint4 w = *reinterpret_cast<const uint4 *>(qrow + (size_t)(g < G ? g : G - 1) * D + 8 * sub);
            qp[LOW ? 0 : g][0] = w.x;
            qp[LOW ? 0 : g][1] = w.y;
            qp[LOW ? 0 : g][2] = w.z;
            qp[LOW ? 0 : g][3] = w.w;
        }
    }
    int64_t n = low ? (a.n_l ? a.n_l[r] : 0) : a.n_h[r];
    const int64_t cap = low ? a.stride_l
                            : (a.block_table ? (int64_t)a.blocks_per_seq * a.page_size : a.stride_h);
    KVC_NOTE(n > cap, KVC_CHK_COUNT);
    if (n > cap) n = cap;
    const int cnt = n - k0 < DEC_CHUNK ? (int)(n - k0) : DEC_CHUNK;
    if (cnt <= 0) {  // empty chunk: contributes nothing
        for (int i = tid; i < G * (D + 2); i += DEC_THREADS) out[i] = (i % (D + 2)) == 0 ? -INFINITY : 0.f;
        return;
    }
    if (LOW)
        for (int i = tid; i < GM * D; i += DEC_THREADS) s_q[i / D][i % D] = i / D < G ? bf16_to_f32(qrow[i]) : 0.f;

    // Storage row of every key this thread touches (-1: none), then all loads.
    int32_t srow[ITER];   // storage slots fit int32: the caller checks the strides
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int e = it * KPI + kin;
        int64_t sl = -1;
        if (e < cnt) sl = low ? k0 + e : bf16_slot(a, ri.n, (int)(k0 + e));
        if (sl >= 0) sl = KVC_IDX(sl, low ? a.stride_l : a.stride_h, KVC_CHK_DECODE);
        srow[it] = (int32_t)sl;
    }
    uint4 kv[ITER];   // bf16: 8 values; int8: codes in .x/.y
    float ks[LOW ? ITER : 1];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        kv[it] = make_uint4(0, 0, 0, 0);
        if (LOW) ks[LOW ? it : 0] = 0.f;
        if (srow[it] < 0) continue;
        if (!low) {
            kv[it] = *reinterpret_cast<const uint4 *>(a.K + ((size_t)r * a.stride_h + srow[it]) * D + 8 * sub);
        } else if (LOWB == 4) {
            const uint32_t c = *reinterpret_cast<const uint32_t *>(a.Kq + ((size_t)r * a.stride_l + srow[it]) * CB + 4 * sub);
            kv[it] = make_uint4(c, 0, 0, 0);
            ks[LOW ? it : 0] = half_bits_to_f32(a.Ks[(size_t)r * a.stride_l + srow[it]]);
        } else {
            const uint2 c = *reinterpret_cast<const uint2 *>(a.Kq + ((size_t)r * a.stride_l + srow[it]) * CB + 8 * sub);
            kv[it] = make_uint4(c.x, c.y, 0, 0);
            ks[LOW ? it : 0] = half_bits_to_f32(a.Ks[(size_t)r * a.stride_l + srow[it]]);
        }
    }
    if (LOW) __syncthreads();  // s_q ready
    // dequantised keys: the query in fp32
    float q[LOW ? GM : 1][8];
    if (LOW) {
#pragma unroll
        for (int g = 0; g < GM; ++g)
#pragma unroll
            for (int c = 0; c < 8; ++c) q[LOW ? g : 0][c] = s_q[g][8 * sub + c];
    }

    // Logits: partial dot products over this thread's 8 dimensions, summed
    // over the key's TPK threads (lanes kin*TPK .. kin*TPK + TPK-1 of the wave).
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        float dot[GM];
        if (!low) {
            const uint32_t w[4] = {kv[it].x, kv[it].y, kv[it].z, kv[it].w};
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                float acc = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]),
                                                          __builtin_bit_cast(bf16x2, qp[LOW ? 0 : g][e]), acc, false);
                dot[g] = acc;
            }
        } else {
            float x[8];
            if (LOWB == 4) {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = (float)((int32_t)(kv[it].x << (28 - 4 * e)) >> 28) * ks[LOW ? it : 0];
            } else {
                const uint32_t w[2] = {kv[it].x, kv[it].y};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    x[e] = (float)(int8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xFF) * ks[LOW ? it : 0];
            }
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < 8; ++c) acc = fmaf(x[c], q[LOW ? g : 0][c], acc);
                dot[g] = acc;
            }
        }
#pragma unroll
        for (int g = 0; g < GM; ++g) dot[g] = group_sum<TPK>(dot[g]);
        const int e = it * KPI + kin;
        if (sub == 0) {
#pragma unroll
            for (int g = 0; g < GM; ++g) s_p[g][e] = srow[it] >= 0 ? dot[g] * a.c2 : -INFINITY;
        }
    }
    // Value loads now, so they are in flight during the statistics.
    uint4 vv[ITER];
    float vs[LOW ? ITER : 1];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        vv[it] = make_uint4(0, 0, 0, 0);
        if (LOW) vs[LOW ? it : 0] = 0.f;
        if (srow[it] < 0) continue;
        if (!low) {
            vv[it] = *reinterpret_cast<const uint4 *>(a.V + ((size_t)r * a.stride_h + srow[it]) * D + 8 * sub);
        } else if (LOWB == 4) {
            const uint32_t c = *reinterpret_cast<const uint32_t *>(a.Vq + ((size_t)r * a.stride_l + srow[it]) * CB + 4 * sub);
            vv[it] = make_uint4(c, 0, 0, 0);
            vs[LOW ? it : 0] = half_bits_to_f32(a.Vs[(size_t)r * a.stride_l + srow[it]]);
        } else {
            const uint2 c = *reinterpret_cast<const uint2 *>(a.Vq + ((size_t)r * a.stride_l + srow[it]) * CB + 8 * sub);
            vv[it] = make_uint4(c.x, c.y, 0, 0);
            vs[LOW ? it : 0] = half_bits_to_f32(a.Vs[(size_t)r * a.stride_l + srow[it]]);
        }
    }
    __syncthreads();  // logits ready
    // Per-head chunk max and exp-sum (log2 domain): thread <-> key (DEC_CHUNK == DEC_THREADS).
    float v[GM], m[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        v[g] = tid < cnt ? s_p[g][tid] : -INFINITY;
        if (!LOW && a.logit && g < G && tid < cnt)
            a.logit[((size_t)r * G + g) * ((size_t)a.chunks_h * DEC_CHUNK) + k0 + tid] = v[g];
        float x = v[g];
        x = xor32_max(xor16_max(group_max<16>(x)));
        if (lane == 0) s_w[wave][g] = x;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        float x = s_w[0][g];
#pragma unroll
        for (int w = 1; w < NW; ++w) x = fmaxf(x, s_w[w][g]);
        m[g] = x;
    }
    __syncthreads();  // every thread has read the maxima
    float l[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        const float pv = (v[g] > -INFINITY) ? __builtin_amdgcn_exp2f(v[g] - m[g]) : 0.f;
        s_p[g][tid] = pv;
        float x = pv;
        x = xor32_sum(xor16_sum(group_sum<16>(x)));
        if (lane == 0) s_w[wave][g] = x;
    }
    __syncthreads();  // weights and partial sums ready
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) x += s_w[w][g];
        l[g] = x;
    }
    // Weighted values: this thread's 8 dimensions over its keys.
    float acc[GM][8];
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[g][c] = 0.f;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        if (srow[it] < 0) continue;
        const int e = it * KPI + kin;
        float x[8];
        if (!low) {
            const uint32_t w[4] = {vv[it].x, vv[it].y, vv[it].z, vv[it].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                x[2 * c] = bf16_to_f32((uint16_t)(w[c] & 0xFFFF));
                x[2 * c + 1] = bf16_to_f32((uint16_t)(w[c] >> 16));
            }
        } else if (LOWB == 4) {
#pragma unroll
            for (int c = 0; c < 8; ++c) x[c] = (float)((int32_t)(vv[it].x << (28 - 4 * c)) >> 28) * vs[LOW ? it : 0];
        } else {
            const uint32_t w[2] = {vv[it].x, vv[it].y};
#pragma unroll
            for (int c = 0; c < 8; ++c) x[c] = (float)(int8_t)((w[c >> 2] >> (8 * (c & 3))) & 0xFF) * vs[LOW ? it : 0];
        }
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            const float pw = s_p[g][e];
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[g][c] = fmaf(pw, x[c], acc[g][c]);
        }
    }
    // Sum over the wave's keys (lanes differing in the key bits), then over waves.
    static_assert(TPK == 8 || TPK == 16, "key groups of 8 or 16 lanes");
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float x = acc[g][c];
            if (TPK == 8) x += dpp_f<0x128>(x);   // row_ror:8 pairs lane i with i ^ 8
            acc[g][c] = xor32_sum(xor16_sum(x));
        }
    if (lane < TPK) {
#pragma unroll
        for (int g = 0; g < GM; ++g)
#pragma unroll
            for (int c = 0; c < 8; ++c) s_acc[wave][g][8 * sub + c] = acc[g][c];
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += DEC_THREADS) {
        const int g = i / D, c = i % D;
        float u = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) u += s_acc[w][g][c];
        out[g * (D + 2) + 2 + c] = u;
    }
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        if (g < G && tid == 0) {
            out[g * (D + 2) + 0] = m[g];
            out[g * (D + 2) + 1] = l[g];
        }
    }
}

template <int D>
__global__ void __launch_bounds__(D) decode_merge(DecodeArgs a) {
    const int slots = a.chunks_h + a.chunks_l;
    const int64_t rg = blockIdx.x;  // (row, g)
    const int64_t r = rg / a.G;
    const int g = (int)(rg % a.G);
    const int c = threadIdx.x;
    const float *base = a.part + (size_t)r * slots * a.G * (D + 2) + (size_t)g * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < slots; ++s) M = fmaxf(M, base[(size_t)s * a.G * (D + 2)]);
    float Lsum = 0.f, U = 0.f;
    if (M > -INFINITY) {
        for (int s = 0; s < slots; ++s) {
            const float *p = base + (size_t)s * a.G * (D + 2);
            if (p[0] == -INFINITY) continue;
            const float f = __builtin_amdgcn_exp2f(p[0] - M);
            Lsum = fmaf(f, p[1], Lsum);
            U = fmaf(f, p[2 + c], U);
        }
    }
    const RowIdx ri = split_row(r, a.L, a.Hkv);
    const size_t head = (size_t)(ri.n * a.L + ri.l) * a.Hq + (size_t)ri.h * a.G + g;
    a.o[head * D + c] = f32_to_bf16(Lsum > 0.f ? U / Lsum : 0.f);
    if (c == 0 && a.lse) a.lse[head] = Lsum > 0.f ? (M + log2f(Lsum)) * 0.69314718055994531f : -INFINITY;
    if (c == 0 && a.lse2) a.lse2[rg] = Lsum > 0.f ? M + log2f(Lsum) : INFINITY;
}

// H2O: acc[r][t] += sum over the group's heads of softmax weight 2^(logit - lse2)
// for the row's n_h cached keys; one thread per key.
__global__ void __launch_bounds__(DEC_THREADS) decode_mass(DecodeArgs a, float *acc) {
    const int64_t r = blockIdx.x / a.chunks_h;
    const int chunk = blockIdx.x % a.chunks_h;
    int64_t n = a.n_h[r];
    if (n > a.stride_h) n = a.stride_h;
    const int64_t t = (int64_t)chunk * DEC_CHUNK + threadIdx.x;
    if (t >= n) return;
    const size_t lstride = (size_t)a.chunks_h * DEC_CHUNK;
    float m = 0.f;
    for (int g = 0; g < a.G; ++g)
        m += __builtin_amdgcn_exp2f(a.logit[((size_t)r * a.G + g) * lstride + t] - a.lse2[(size_t)r * a.G + g]);
    acc[(size_t)r * a.stride_h + t] += m;
}

KVC_CHECK_READER(check_read_decode)

size_t decode_workspace_bytes(const kvc_dims *d, int64_t stride_h, int64_t stride_l) {
    const int G = d->n_q_heads / d->n_kv_heads;
    const int64_t ch = (stride_h + DEC_CHUNK - 1) / DEC_CHUNK;
    const int64_t cl = (stride_l + DEC_CHUNK - 1) / DEC_CHUNK;
    return (size_t)n_rows(d) * (ch + cl) * G * (d->head_dim + 2) * sizeof(float);
}

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// H2O workspace: the partials, then the logits, then the normalisers.
size_t decode_h2o_workspace_bytes(const kvc_dims *d, int64_t stride_h) {
    const int G = d->n_q_heads / d->n_kv_heads;
    const int64_t ch = (stride_h + DEC_CHUNK - 1) / DEC_CHUNK;
    return align256(decode_workspace_bytes(d, stride_h, 0)) +
           align256((size_t)n_rows(d) * G * ch * DEC_CHUNK * sizeof(float)) + (size_t)n_rows(d) * G * sizeof(float);
}

// Partials over both partitions, the Eq. 15 merge, and (acc != NULL) the H2O update.
static int decode_launch(const kvc_dims *dims, DecodeArgs &a, float *acc, hipStream_t s, const char *who) {
    int st;
    const int G = a.G;
    const int64_t rows = n_rows(dims);
    const int64_t blocks = rows * (a.chunks_h + a.chunks_l);
    if (blocks > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "%s: grid too large", who);
    const dim3 grid_h((unsigned)(rows * a.chunks_h)), grid_l((unsigned)(rows * a.chunks_l)), block(DEC_THREADS);
#define DEC_PARTIAL_G(DD, GG)                                                              \
    do {                                                                                   \
        decode_partial<DD, GG, 0><<<grid_h, block, 0, s>>>(a);                             \
        if (a.chunks_l && a.low_bits == 4)                                                 \
            decode_partial<DD, GG, 4><<<grid_l, block, 0, s>>>(a);                         \
        else if (a.chunks_l)                                                               \
            decode_partial<DD, GG, 8><<<grid_l, block, 0, s>>>(a);                         \
    } while (0)
#define DEC_PARTIAL(DD)                                                                    \
    do {                                                                                   \
        if (G <= 4)                                                                        \
            DEC_PARTIAL_G(DD, 4);                                                          \
        else if (G <= 8)                                                                   \
            DEC_PARTIAL_G(DD, 8);                                                          \
        else                                                                               \
            DEC_PARTIAL_G(DD, 16);                                                         \
    } while (0)
    if (dims->head_dim == 128) {
        DEC_PARTIAL(128);
        if ((st = check_launch(who)) != KVC_OK) return st;
        decode_merge<128><<<dim3((unsigned)(rows * G)), dim3(128), 0, s>>>(a);
    } else {
        DEC_PARTIAL(64);
        if ((st = check_launch(who)) != KVC_OK) return st;
        decode_merge<64><<<dim3((unsigned)(rows * G)), dim3(64), 0, s>>>(a);
    }
#undef DEC_PARTIAL
#undef DEC_PARTIAL_G
    if ((st = check_launch(who)) != KVC_OK) return st;
    if (acc) {
        decode_mass<<<grid_h, block, 0, s>>>(a, acc);
        return check_launch(who);
    }
    return KVC_OK;
}


}  // namespace kvc

using namespace kvc;

extern "C" int kvc_decode_attn(const kvc_dims *dims, const uint16_t *q, const uint16_t *K,
                               const uint16_t *V, const int32_t *n_h, int64_t stride_h,
                               const int32_t *block_table, int32_t page_size, int32_t blocks_per_seq,
                               const int8_t *Kq, const int8_t *Vq, const uint16_t *Ks,
                               const uint16_t *Vs, const int32_t *n_l, int64_t stride_l, int32_t low_bits,
                               uint16_t *o, float *lse, void *ws, size_t ws_bytes, void *stream) {
    int st = check_dims(dims, "kvc_decode_attn");
    if (st != KVC_OK) return st;
    if (!q || !K || !V || !n_h || !o) return fail(KVC_ERR_ARG, "kvc_decode_attn: NULL pointer");
    if (stride_h <= 0) return fail(KVC_ERR_ARG, "kvc_decode_attn: stride_h must be positive");
    if (stride_h > (int64_t)INT32_MAX || stride_l > (int64_t)INT32_MAX)
        return fail(KVC_ERR_UNSUPPORTED, "kvc_decode_attn: pool strides must fit int32");
    const int G = dims->n_q_heads / dims->n_kv_heads;
    if (G > DEC_MAX_G)
        return fail(KVC_ERR_UNSUPPORTED, "kvc_decode_attn: GQA group %d exceeds %d", G, DEC_MAX_G);
    if (block_table && (page_size <= 0 || blocks_per_seq <= 0))
        return fail(KVC_ERR_ARG, "kvc_decode_attn: paged layout needs page_size and blocks_per_seq");
    const bool has_low = n_l != nullptr;
    if (has_low && (!Kq || !Vq || !Ks || !Vs || stride_l <= 0))
        return fail(KVC_ERR_ARG, "kvc_decode_attn: low-precision partition needs Kq, Vq, Ks, Vs and stride_l");
    if (has_low && low_bits != 8 && low_bits != 4)
        return fail(KVC_ERR_UNSUPPORTED, "kvc_decode_attn: low_bits %d (8 or 4)", low_bits);
    // The bf16 partition's token count is bounded by what the layout can address.
    const int64_t max_h = block_table ? (int64_t)blocks_per_seq * page_size : stride_h;
    const size_t need = decode_workspace_bytes(dims, max_h, has_low ? stride_l : 0);
    if (!ws || ws_bytes < need)
        return fail(KVC_ERR_WORKSPACE, "kvc_decode_attn: workspace %zu < %zu bytes", ws_bytes, need);
    DecodeArgs a;
    a.q = q;
    a.K = K;
    a.V = V;
    a.n_h = n_h;
    a.stride_h = stride_h;
    a.block_table = block_table;
    a.page_size = page_size;
    a.blocks_per_seq = blocks_per_seq;
    a.Kq = Kq;
    a.Vq = Vq;
    a.Ks = Ks;
    a.Vs = Vs;
    a.n_l = n_l;
    a.stride_l = has_low ? stride_l : 0;
    a.low_bits = low_bits;
    a.L = dims->n_layers;
    a.Hkv = dims->n_kv_heads;
    a.Hq = dims->n_q_heads;
    a.G = G;
    a.chunks_h = (int)((max_h + DEC_CHUNK - 1) / DEC_CHUNK);
    a.chunks_l = has_low ? (int)((stride_l + DEC_CHUNK - 1) / DEC_CHUNK) : 0;
    a.c2 = (float)(1.4426950408889634 / std::sqrt((double)dims->head_dim));
    a.part = reinterpret_cast<float *>(ws);
    a.o = o;
    a.lse = lse;
    a.logit = nullptr;
    a.lse2 = nullptr;
    return decode_launch(dims, a, nullptr, as_stream(stream), "kvc_decode_attn");
}

extern "C" size_t kvc_decode_h2o_workspace_bytes(const kvc_dims *dims, int64_t stride_h) {
    if (check_dims(dims, "kvc_decode_h2o_workspace_bytes") != KVC_OK) return 0;
    if (stride_h < 0) {
        fail(KVC_ERR_ARG, "kvc_decode_h2o_workspace_bytes: negative capacity");
        return 0;
    }
    return decode_h2o_workspace_bytes(dims, stride_h);
}

extern "C" int kvc_decode_attn_h2o(const kvc_dims *dims, const uint16_t *q, const uint16_t *K,
                                   const uint16_t *V, const int32_t *n_h, int64_t stride_h, float *acc,
                                   uint16_t *o, float *lse, void *ws, size_t ws_bytes, void *stream) {
    int st = check_dims(dims, "kvc_decode_attn_h2o");
    if (st != KVC_OK) return st;
    if (!q || !K || !V || !n_h || !acc || !o) return fail(KVC_ERR_ARG, "kvc_decode_attn_h2o: NULL pointer");
    if (stride_h <= 0) return fail(KVC_ERR_ARG, "kvc_decode_attn_h2o: stride_h must be positive");
    if (stride_h > (int64_t)INT32_MAX)
        return fail(KVC_ERR_UNSUPPORTED, "kvc_decode_attn_h2o: pool stride must fit int32");
    const int G = dims->n_q_heads / dims->n_kv_heads;
    if (G > DEC_MAX_G)
        return fail(KVC_ERR_UNSUPPORTED, "kvc_decode_attn_h2o: GQA group %d exceeds %d", G, DEC_MAX_G);
    const size_t need = decode_h2o_workspace_bytes(dims, stride_h);
    if (!ws || ws_bytes < need)
        return fail(KVC_ERR_WORKSPACE, "kvc_decode_attn_h2o: workspace %zu < %zu bytes", ws_bytes, need);
    DecodeArgs a;
    a.q = q;
    a.K = K;
    a.V = V;
    a.n_h = n_h;
    a.stride_h = stride_h;
    a.block_table = nullptr;
    a.page_size = 0;
    a.blocks_per_seq = 0;
    a.Kq = a.Vq = nullptr;
    a.Ks = a.Vs = nullptr;
    a.n_l = nullptr;
    a.stride_l = 0;
    a.low_bits = 8;
    a.L = dims->n_layers;
    a.Hkv = dims->n_kv_heads;
    a.Hq = dims->n_q_heads;
    a.G = G;
    a.chunks_h = (int)((stride_h + DEC_CHUNK - 1) / DEC_CHUNK);
    a.chunks_l = 0;
    a.c2 = (float)(1.4426950408889634 / std::sqrt((double)dims->head_dim));
    char *w = reinterpret_cast<char *>(ws);
    a.part = reinterpret_cast<float *>(w);
    w += align256(decode_workspace_bytes(dims, stride_h, 0));
    a.logit = reinterpret_cast<float *>(w);
    w += align256((size_t)n_rows(dims) * G * a.chunks_h * DEC_CHUNK * sizeof(float));
    a.lse2 = reinterpret_cast<float *>(w);
    a.o = o;
    a.lse = lse;
    return decode_launch(dims, a, acc, as_stream(stream), "kvc_decode_attn_h2o");
}



extern "C" size_t kvc_decode_workspace_bytes(const kvc_dims *dims, int64_t max_h, int64_t stride_l) {
    if (check_dims(dims, "kvc_decode_workspace_bytes") != KVC_OK) return 0;
    if (max_h < 0 || stride_l < 0) {
        fail(KVC_ERR_ARG, "kvc_decode_workspace_bytes: negative capacity");
        return 0;
    }
    return decode_workspace_bytes(dims, max_h, stride_l);
}
