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
// both partitions. Phase A: thread <-> key, dot products against the G queries
// (staged in LDS as fp32). Phase B: per-head chunk max and exp-sum. Phase C:
// thread <-> (dimension pair, key stripe) accumulation of sum_j p_j v_j.
// The bf16 partition may be paged: token t of a row then lives in slot
// block_table[n][t / page_size] * page_size + t % page_size of the row's storage.
#include <cmath>

#include "kvc_internal.h"

namespace kvc {

static constexpr int DEC_CHUNK = 256;
static constexpr int DEC_THREADS = 256;
static constexpr int DEC_MAX_G = 16;

struct DecodeArgs {
    const uint16_t *q;
    const uint16_t *K, *V;
    const int32_t *n_h;
    int64_t stride_h;
    const int32_t *block_table;
    int32_t page_size, blocks_per_seq;
    const int8_t *Kq, *Vq;
    const uint16_t *Ks, *Vs;
    const int32_t *n_l;
    int64_t stride_l;
    int L, Hkv, Hq, G;
    int chunks_h, chunks_l;  // chunk slots per row for each partition
    float c2;                // log2(e) / sqrt(d)
    float *part;             // [rows][chunks_h + chunks_l][G][D + 2]
    uint16_t *o;
    float *lse;
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
    return (blk < 0 || s >= a.stride_h) ? -1 : s;
}

template <int D>
__global__ void __launch_bounds__(DEC_THREADS) decode_partial(DecodeArgs a) {
    constexpr int DP = D / 2;
    constexpr int STRIPES = DEC_THREADS / DP;
    __shared__ float s_q[DEC_MAX_G][D];
    __shared__ float s_p[DEC_MAX_G][DEC_CHUNK];
    __shared__ float s_red[DEC_THREADS / 64];
    __shared__ float s_acc[STRIPES][DEC_MAX_G][D];
    __shared__ int64_t s_slot[DEC_CHUNK];

    const int slots = a.chunks_h + a.chunks_l;
    const int64_t r = blockIdx.x / slots;
    const int slot = blockIdx.x % slots;
    const bool low = slot >= a.chunks_h;
    const int chunk = low ? slot - a.chunks_h : slot;
    const RowIdx ri = split_row(r, a.L, a.Hkv);
    const int G = a.G;
    const int tid = threadIdx.x;
    float *out = a.part + ((size_t)r * slots + slot) * G * (D + 2);

    int64_t n = low ? (a.n_l ? a.n_l[r] : 0) : a.n_h[r];
    const int64_t cap = low ? a.stride_l
                            : (a.block_table ? (int64_t)a.blocks_per_seq * a.page_size : a.stride_h);
    if (n > cap) n = cap;
    const int64_t k0 = (int64_t)chunk * DEC_CHUNK;
    const int cnt = n - k0 < DEC_CHUNK ? (int)(n - k0) : DEC_CHUNK;
    if (cnt <= 0) {  // empty chunk: contributes nothing
        for (int i = tid; i < G * (D + 2); i += DEC_THREADS) out[i] = (i % (D + 2)) == 0 ? -INFINITY : 0.f;
        return;
    }
    const uint16_t *qrow = a.q + ((size_t)(ri.n * a.L + ri.l) * a.Hq + (size_t)ri.h * G) * D;
    for (int i = tid; i < G * D; i += DEC_THREADS) s_q[i / D][i % D] = bf16_to_f32(qrow[i]);
    __syncthreads();

    // Phase A: thread <-> key.
    float sc[DEC_MAX_G];
#pragma unroll
    for (int g = 0; g < DEC_MAX_G; ++g) sc[g] = 0.f;
    bool valid = tid < cnt;
    if (valid) {
        const int t = (int)(k0 + tid);
        if (!low) {
            const int64_t sl = bf16_slot(a, ri.n, t);
            s_slot[tid] = sl;
            valid = sl >= 0;
            if (valid) {
                const uint16_t *kr = a.K + ((size_t)r * a.stride_h + sl) * D;
                for (int c = 0; c < D; c += 8) {
                    const uint4 u = *reinterpret_cast<const uint4 *>(kr + c);
                    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float ka = bf16_to_f32((uint16_t)(w[e] & 0xFFFF));
                        const float kb = bf16_to_f32((uint16_t)(w[e] >> 16));
#pragma unroll
                        for (int g = 0; g < DEC_MAX_G; ++g)
                            if (g < G) sc[g] = fmaf(kb, s_q[g][c + 2 * e + 1], fmaf(ka, s_q[g][c + 2 * e], sc[g]));
                    }
                }
            }
        } else {
            s_slot[tid] = t;
            const int8_t *kr = a.Kq + ((size_t)r * a.stride_l + t) * D;
            const float ks = half_bits_to_f32(a.Ks[(size_t)r * a.stride_l + t]);
            for (int c = 0; c < D; c += 16) {
                const uint4 u = *reinterpret_cast<const uint4 *>(kr + c);
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const float kf = (float)(int8_t)((w[e] >> (8 * b)) & 0xFF) * ks;
#pragma unroll
                        for (int g = 0; g < DEC_MAX_G; ++g)
                            if (g < G) sc[g] = fmaf(kf, s_q[g][c + 4 * e + b], sc[g]);
                    }
                }
            }
        }
    }
    // Phase B: per-head chunk max and exp-sum (log2 domain).
    float mg[DEC_MAX_G], lg[DEC_MAX_G];
#pragma unroll
    for (int g = 0; g < DEC_MAX_G; ++g) {
        mg[g] = -INFINITY;
        lg[g] = 0.f;
        if (g < G) {
            const float v = valid ? sc[g] * a.c2 : -INFINITY;
            mg[g] = block_reduce(v, true, s_red);
            const float p = valid ? __builtin_amdgcn_exp2f(v - mg[g]) : 0.f;
            s_p[g][tid] = p;
            lg[g] = block_reduce(p, false, s_red);
        }
    }
    __syncthreads();
    // Phase C: thread <-> (dimension pair dp, key stripe).
    const int dp = tid % DP, stripe = tid / DP;
    float acc0[DEC_MAX_G], acc1[DEC_MAX_G];
#pragma unroll
    for (int g = 0; g < DEC_MAX_G; ++g) acc0[g] = acc1[g] = 0.f;
    for (int e = stripe; e < cnt; e += STRIPES) {
        const int64_t sl = s_slot[e];
        if (sl < 0) continue;
        float v0, v1;
        if (!low) {
            const uint32_t u = *reinterpret_cast<const uint32_t *>(a.V + ((size_t)r * a.stride_h + sl) * D + 2 * dp);
            v0 = bf16_to_f32((uint16_t)(u & 0xFFFF));
            v1 = bf16_to_f32((uint16_t)(u >> 16));
        } else {
            const float vs = half_bits_to_f32(a.Vs[(size_t)r * a.stride_l + sl]);
            const uint16_t u = *reinterpret_cast<const uint16_t *>(a.Vq + ((size_t)r * a.stride_l + sl) * D + 2 * dp);
            v0 = (float)(int8_t)(u & 0xFF) * vs;
            v1 = (float)(int8_t)(u >> 8) * vs;
        }
#pragma unroll
        for (int g = 0; g < DEC_MAX_G; ++g) {
            if (g < G) {
                const float p = s_p[g][e];
                acc0[g] = fmaf(p, v0, acc0[g]);
                acc1[g] = fmaf(p, v1, acc1[g]);
            }
        }
    }
#pragma unroll
    for (int g = 0; g < DEC_MAX_G; ++g) {
        if (g < G) {
            s_acc[stripe][g][2 * dp] = acc0[g];
            s_acc[stripe][g][2 * dp + 1] = acc1[g];
        }
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += DEC_THREADS) {
        const int g = i / D, c = i % D;
        float u = 0.f;
        for (int s = 0; s < STRIPES; ++s) u += s_acc[s][g][c];
        out[g * (D + 2) + 2 + c] = u;
    }
#pragma unroll
    for (int g = 0; g < DEC_MAX_G; ++g) {
        if (g < G && tid == 0) {
            out[g * (D + 2) + 0] = mg[g];
            out[g * (D + 2) + 1] = lg[g];
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
}

size_t decode_workspace_bytes(const kvc_dims *d, int64_t stride_h, int64_t stride_l) {
    const int G = d->n_q_heads / d->n_kv_heads;
    const int64_t ch = (stride_h + DEC_CHUNK - 1) / DEC_CHUNK;
    const int64_t cl = (stride_l + DEC_CHUNK - 1) / DEC_CHUNK;
    return (size_t)n_rows(d) * (ch + cl) * G * (d->head_dim + 2) * sizeof(float);
}

}  // namespace kvc

using namespace kvc;

extern "C" int kvc_decode_attn(const kvc_dims *dims, const uint16_t *q, const uint16_t *K,
                               const uint16_t *V, const int32_t *n_h, int64_t stride_h,
                               const int32_t *block_table, int32_t page_size, int32_t blocks_per_seq,
                               const int8_t *Kq, const int8_t *Vq, const uint16_t *Ks,
                               const uint16_t *Vs, const int32_t *n_l, int64_t stride_l,
                               uint16_t *o, float *lse, void *ws, size_t ws_bytes, void *stream) {
    int st = check_dims(dims, "kvc_decode_attn");
    if (st != KVC_OK) return st;
    if (!q || !K || !V || !n_h || !o) return fail(KVC_ERR_ARG, "kvc_decode_attn: NULL pointer");
    if (stride_h <= 0) return fail(KVC_ERR_ARG, "kvc_decode_attn: stride_h must be positive");
    const int G = dims->n_q_heads / dims->n_kv_heads;
    if (G > DEC_MAX_G)
        return fail(KVC_ERR_UNSUPPORTED, "kvc_decode_attn: GQA group %d exceeds %d", G, DEC_MAX_G);
    if (block_table && (page_size <= 0 || blocks_per_seq <= 0))
        return fail(KVC_ERR_ARG, "kvc_decode_attn: paged layout needs page_size and blocks_per_seq");
    const bool has_low = n_l != nullptr;
    if (has_low && (!Kq || !Vq || !Ks || !Vs || stride_l <= 0))
        return fail(KVC_ERR_ARG, "kvc_decode_attn: int8 partition needs Kq, Vq, Ks, Vs and stride_l");
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
    const int64_t rows = n_rows(dims);
    const int64_t blocks = rows * (a.chunks_h + a.chunks_l);
    if (blocks > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "kvc_decode_attn: grid too large");
    hipStream_t s = as_stream(stream);
    if (dims->head_dim == 128) {
        decode_partial<128><<<dim3((unsigned)blocks), dim3(DEC_THREADS), 0, s>>>(a);
        if ((st = check_launch("kvc_decode_attn partial")) != KVC_OK) return st;
        decode_merge<128><<<dim3((unsigned)(rows * G)), dim3(128), 0, s>>>(a);
    } else {
        decode_partial<64><<<dim3((unsigned)blocks), dim3(DEC_THREADS), 0, s>>>(a);
        if ((st = check_launch("kvc_decode_attn partial")) != KVC_OK) return st;
        decode_merge<64><<<dim3((unsigned)(rows * G)), dim3(64), 0, s>>>(a);
    }
    return check_launch("kvc_decode_attn merge");
}

extern "C" size_t kvc_decode_workspace_bytes(const kvc_dims *dims, int64_t max_h, int64_t stride_l) {
    if (check_dims(dims, "kvc_decode_workspace_bytes") != KVC_OK) return 0;
    if (max_h < 0 || stride_l < 0) {
        fail(KVC_ERR_ARG, "kvc_decode_workspace_bytes: negative capacity");
        return 0;
    }
    return decode_workspace_bytes(dims, max_h, stride_l);
}
