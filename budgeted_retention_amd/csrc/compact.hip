// kvc_compact_rerotate: gather the kept tokens of every row into contiguous
// pools, renumber them to bounded positions and re-rotate their keys exactly.
//
// PACE §3.2: kept tokens are renumbered in logical order to p' = base + rank
// and every kept key is rotated by R_{p'-p}; by Proposition 1 that is the key
// the engine would have cached at p'. The angle (p'-p)*theta_i is formed in
// fp64 from the integer position difference and reduced modulo 2*pi in fp64
// (Cody-Waite with a two-term 2*pi), so positions up to 2^31 stay exact to
// well below a bf16 ulp; the reduced angle's sine/cosine and the rotation run
// in fp32 and the result is rounded once to bf16. Values are bit copies
// (CommitKV §3.1 Eq. 4 applies the same index set to K, V and positions).
//
// Work split (plain path): a group of D/8 threads owns one token; thread `sub`
// rotates the frequency pairs 4sub..4sub+3 and their partners D/2 further on,
// so a group's loads cover the key and value rows contiguously. The tiered
// path keeps groups of D/4 threads with two pairs each.
//
// With an action array the kept entries are routed, in rank order, to the
// bf16 tier, the int8 tier (PASK Appendix B.5 symmetric per-token-per-head
// rule with 7 -> 127, separately for K and V) or dropped; one workgroup per
// row scans the actions to give every entry its slot in its tier.
#include <cmath>

#include "kvc_internal.h"

namespace kvc {

static constexpr int CMP_THREADS = 256;

__device__ __forceinline__ void reduced_sincos(double ang, float *s, float *c) {
    const double INV_2PI = 0.15915494309189535;
    const double TWO_PI_HI = 6.283185307179586;       // nearest double to 2*pi
    const double TWO_PI_LO = 2.4492935982947064e-16;  // 2*pi - TWO_PI_HI
    const double k = rint(ang * INV_2PI);
    double r = fma(-k, TWO_PI_HI, ang);
    r = fma(-k, TWO_PI_LO, r);
    sincosf((float)r, s, c);
}

// Rotates the two bf16 pairs packed in (lo, hi): lo holds x_i, x_{i+1} of the
// first half, hi the partners x_{i+D/2}, x_{i+1+D/2}.
__device__ __forceinline__ void rotate_pairs(uint32_t &lo, uint32_t &hi, double delta, double th0,
                                             double th1) {
    float s0, c0, s1, c1;
    reduced_sincos(delta * th0, &s0, &c0);
    reduced_sincos(delta * th1, &s1, &c1);
    const float x0 = bf16_to_f32((uint16_t)(lo & 0xFFFF)), x1 = bf16_to_f32((uint16_t)(lo >> 16));
    const float y0 = bf16_to_f32((uint16_t)(hi & 0xFFFF)), y1 = bf16_to_f32((uint16_t)(hi >> 16));
    const float nx0 = x0 * c0 - y0 * s0, ny0 = y0 * c0 + x0 * s0;
    const float nx1 = x1 * c1 - y1 * s1, ny1 = y1 * c1 + x1 * s1;
    lo = (uint32_t)f32_to_bf16(nx0) | ((uint32_t)f32_to_bf16(nx1) << 16);
    hi = (uint32_t)f32_to_bf16(ny0) | ((uint32_t)f32_to_bf16(ny1) << 16);
}

// Non-negative double -> IEEE half bits, round-to-nearest-even, from the
// exact double (no intermediate float rounding).
__device__ uint16_t f64_to_f16_rne(double x) {
    if (!(x > 0.0)) return 0;
    int e;
    const double m = frexp(x, &e);  // x = m * 2^e, m in [0.5, 1)
    if (e - 1 < -14) {               // below the smallest normal: grid 2^-24
        return (uint16_t)rint(ldexp(x, 24));  // 1024 lands exactly on 2^-14's encoding
    }
    double mant = rint(ldexp(m, 11));  // 11 significant bits, in [1024, 2048]
    if (mant == 2048.0) {
        mant = 1024.0;
        ++e;
    }
    const int field = e - 1 + 15;
    if (field >= 31) return 0x7C00;
    return (uint16_t)((field << 10) | ((int)mant - 1024));
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    const int ex = (h >> 10) & 31, mt = h & 1023;
    const float v = ex == 0 ? ldexpf((float)mt, -24) : ldexpf((float)(1024 + mt), ex - 25);
    return (h & 0x8000) ? -v : v;
}

// Maximum over the TPT adjacent lanes of a token (any TPT up to 64; some
// lanes of the wave may be inactive).
template <int TPT>
__device__ __forceinline__ float token_max(float v) {
#pragma unroll
    for (int m = TPT / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

// Code of x under scale s: round to nearest even, clamp to [-qmax, qmax].
__device__ __forceinline__ int8_t quant_code(float x, float s, float qmax) {
    float q = rintf(__fdiv_rn(x, s));
    q = fminf(fmaxf(q, -qmax), qmax);
    return (int8_t)(int)q;
}

// Scale bits for a row whose max |x| is amax: max(fp16(amax/qmax), 2^-24); zero row -> 1.0.
__device__ __forceinline__ uint16_t low_scale_bits(float amax, double qmax) {
    if (!(amax > 0.f)) return 0x3C00;
    uint16_t b = f64_to_f16_rne((double)amax / qmax);
    return b == 0 ? (uint16_t)1 : b;
}

// Two codes as one byte: the first in the low nibble (4-bit two's complement).
__device__ __forceinline__ uint32_t nibble_pair(int8_t c0, int8_t c1) {
    return ((uint32_t)c0 & 0xFu) | (((uint32_t)c1 & 0xFu) << 4);
}

struct CompactArgs {
    const uint16_t *K, *V;
    const int32_t *pos_in, *kept, *n_kept;
    const uint8_t *action;
    int64_t T, rows_per_seq;
    int kept_stride, out_stride, renumber_base, kept_page;
    double rope_base;
    uint16_t *Ko, *Vo;
    int32_t *po, *nh;
    int8_t *Kq, *Vq;
    uint16_t *Ks, *Vs;
    int32_t *pq, *nl;
    int low_bits;             // 8: int8 codes; 4: INT4 nibble pairs
    const int32_t *h_base, *l_base;
    const uint16_t *Kref;     // reference store of the current slots, or NULL
    const int32_t *pref;
    uint16_t *Kref_out;       // reference store of the kept slots (REF kernels)
    int32_t *pref_out;
    const float *score_in;    // per-slot payloads carried with the tokens, or NULL
    float *score_out;
    const uint8_t *tag_in;
    uint8_t *tag_out;
};

// Rotates four frequency pairs: lo holds x_i..x_{i+3} of the first half, hi
// their partners x_{i+D/2}..x_{i+3+D/2}; th[e] is the frequency of pair i+e.
__device__ __forceinline__ void rotate_quad(uint2 &lo, uint2 &hi, double delta, const double (&th)[4]) {
    uint32_t l[2] = {lo.x, lo.y}, h[2] = {hi.x, hi.y};
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        float s0, c0, s1, c1;
        reduced_sincos(delta * th[2 * w], &s0, &c0);
        reduced_sincos(delta * th[2 * w + 1], &s1, &c1);
        const float x0 = bf16_to_f32((uint16_t)(l[w] & 0xFFFF)), x1 = bf16_to_f32((uint16_t)(l[w] >> 16));
        const float y0 = bf16_to_f32((uint16_t)(h[w] & 0xFFFF)), y1 = bf16_to_f32((uint16_t)(h[w] >> 16));
        const float nx0 = x0 * c0 - y0 * s0, ny0 = y0 * c0 + x0 * s0;
        const float nx1 = x1 * c1 - y1 * s1, ny1 = y1 * c1 + x1 * s1;
        l[w] = (uint32_t)f32_to_bf16(nx0) | ((uint32_t)f32_to_bf16(nx1) << 16);
        h[w] = (uint32_t)f32_to_bf16(ny0) | ((uint32_t)f32_to_bf16(ny1) << 16);
    }
    lo = make_uint2(l[0], l[1]);
    hi = make_uint2(h[0], h[1]);
}

// Plain compaction. A group of D/8 threads owns one token; thread `sub`
// rotates the frequency pairs 4sub..4sub+3 (an 8-byte load from each half of
// the key) and copies 16 bytes of the value row. A workgroup takes CMP_UNROLL
// consecutive groups of ranks of one row: every thread first reads the kept
// indices of its CMP_UNROLL tokens, then issues all of their key and value
// loads, so each workgroup waits for two memory latencies in all.
static constexpr int CMP_UNROLL = 4;

// True when bf16(R_delta ref) lies within one bf16 step (plus 1e-5 of the
// reference row's largest magnitude, `refmax`) of the stored key, for the four
// pairs this thread holds.
__device__ __forceinline__ bool ref_pairs_match(uint2 rlo, uint2 rhi, uint2 klo, uint2 khi, double delta,
                                                const double (&th)[4], float refmax) {
    rotate_quad(rlo, rhi, delta, th);
    const uint32_t g[4] = {rlo.x, rlo.y, rhi.x, rhi.y}, k[4] = {klo.x, klo.y, khi.x, khi.y};
    bool ok = true;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float gv = bf16_to_f32((uint16_t)(g[w] >> (16 * h)));
            const float kv = bf16_to_f32((uint16_t)(k[w] >> (16 * h)));
            const float tol = fmaxf(fabsf(kv), 1.17549435e-38f) * 0.0078125f + 1e-5f * refmax;
            ok = ok && fabsf(gv - kv) <= tol;
        }
    }
    return ok;
}

__device__ __forceinline__ float bf16x4_maxabs(uint2 v) {
    const float a0 = fabsf(bf16_to_f32((uint16_t)(v.x & 0xFFFF))), a1 = fabsf(bf16_to_f32((uint16_t)(v.x >> 16)));
    const float a2 = fabsf(bf16_to_f32((uint16_t)(v.y & 0xFFFF))), a3 = fabsf(bf16_to_f32((uint16_t)(v.y >> 16)));
    return fmaxf(fmaxf(a0, a1), fmaxf(a2, a3));
}

// REF adds PACE's reference store (non-compounding re-rotation): a kept token
// whose slot holds a reference that passes the check is re-rotated from it
// (angle p' - p_ref); any other from its stored key, which becomes its
// reference at p. The kept slots' references are written beside the keys.
template <int D, bool REF>
__global__ void __launch_bounds__(CMP_THREADS) compact_plain(CompactArgs a, int blocks_per_row) {
    constexpr int TPT = D / 8;
    constexpr int TOK = CMP_THREADS / TPT;
    constexpr int U = CMP_UNROLL;
    const int64_t r = blockIdx.x / blocks_per_row;
    const int cb = blockIdx.x % blocks_per_row;
    const int kp = a.kept_page;
    const int64_t kr = kp ? r / a.rows_per_seq : r;  // row of the kept list
    int n = a.n_kept[kr];
    KVC_NOTE(n > a.kept_stride, KVC_CHK_COUNT);
    if (n > a.kept_stride) n = a.kept_stride;
    if (n < 0) n = 0;
    if (kp) n *= kp;
    int base = a.h_base ? a.h_base[r] : 0;
    if (base < 0) base = 0;
    const int room = a.out_stride - base > 0 ? a.out_stride - base : 0;
    KVC_NOTE(n > room, KVC_CHK_COUNT);
    if (n > room) n = room;
    if (cb == 0 && threadIdx.x == 0 && a.nh) a.nh[r] = base + n;
    const int sub = threadIdx.x % TPT, tin = threadIdx.x / TPT;
    const bool rot = a.renumber_base >= 0;
    double th[4] = {0.0, 0.0, 0.0, 0.0};
    if (rot || REF) {
#pragma unroll
        for (int e = 0; e < 4; ++e) th[e] = pow(a.rope_base, -2.0 * (4 * sub + e) / D);
    }
    const int rho0 = cb * (TOK * U) + tin;
    // Each token lives in its own struct value (no per-thread arrays, which
    // the compiler would place in LDS).
    struct Tok {
        int64_t j, p;
        uint2 lo, hi;
        uint4 v;
        uint2 rlo, rhi;  // the slot's reference (REF)
        int64_t pr;
        float sc;        // carried score and tag (thread sub == 0)
        uint32_t tg;
    };
    auto index = [&](int u) -> int64_t {
        const int rho = rho0 + u * TOK;
        if (rho >= n) return -1;
        int64_t j;
        if (kp) {
            const int64_t e = a.kept[(size_t)kr * a.kept_stride + rho / kp];
            j = e < 0 ? -1 : e * kp + rho % kp;
        } else {
            j = a.kept[(size_t)kr * a.kept_stride + rho];
            KVC_NOTE(j >= a.T, KVC_CHK_KEPT);
        }
        return j < a.T ? j : -1;
    };
    // entries past the kept count read token 0 of the row (always present) and are not stored
    auto fetch = [&](int64_t j) -> Tok {
        Tok t;
        t.j = j;
        const int64_t jj = KVC_IDX(j < 0 ? 0 : j, a.T, KVC_CHK_COMPACT);
        const size_t src = ((size_t)r * a.T + jj) * D;
        t.lo = *reinterpret_cast<const uint2 *>(a.K + src + 4 * sub);
        t.hi = *reinterpret_cast<const uint2 *>(a.K + src + D / 2 + 4 * sub);
        t.v = *reinterpret_cast<const uint4 *>(a.V + src + 8 * sub);
        t.p = a.pos_in ? (int64_t)a.pos_in[(size_t)r * a.T + jj] : jj;
        t.pr = -1;
        t.sc = 0.f;
        t.tg = 0u;
        if (sub == 0 && a.score_in) t.sc = a.score_in[(size_t)r * a.T + jj];
        if (sub == 0 && a.tag_in) t.tg = a.tag_in[(size_t)r * a.T + jj];
        if (REF && a.Kref) {
            t.rlo = *reinterpret_cast<const uint2 *>(a.Kref + src + 4 * sub);
            t.rhi = *reinterpret_cast<const uint2 *>(a.Kref + src + D / 2 + 4 * sub);
            t.pr = (int64_t)a.pref[(size_t)r * a.T + jj];
        }
        return t;
    };
    auto put = [&](Tok &t, int u) {
        if (t.j < 0) return;  // the same for the token's TPT threads
        const int rho = rho0 + u * TOK;
        const int slot = KVC_IDX(base + rho, a.out_stride, KVC_CHK_COMPACT);
        const size_t dst = ((size_t)r * a.out_stride + slot) * D;
        int64_t psrc = t.p;
        if (REF) {
            // the check before use; the token's TPT adjacent lanes agree on it
            bool use = false;
            if (t.pr >= 0) {
                float rm = fmaxf(bf16x4_maxabs(t.rlo), bf16x4_maxabs(t.rhi));
#pragma unroll
                for (int m = 1; m < TPT; m <<= 1) rm = fmaxf(rm, __shfl_xor(rm, m));
                int ok = ref_pairs_match(t.rlo, t.rhi, t.lo, t.hi, (double)(t.p - t.pr), th, rm) ? 1 : 0;
#pragma unroll
                for (int m = 1; m < TPT; m <<= 1) ok &= __shfl_xor(ok, m);
                use = ok != 0;
            }
            if (use) {
                psrc = t.pr;
            } else {
                t.rlo = t.lo;
                t.rhi = t.hi;
            }
            *reinterpret_cast<uint2 *>(a.Kref_out + dst + 4 * sub) = t.rlo;
            *reinterpret_cast<uint2 *>(a.Kref_out + dst + D / 2 + 4 * sub) = t.rhi;
            if (sub == 0) a.pref_out[(size_t)r * a.out_stride + slot] = (int32_t)psrc;
        }
        int64_t pn = t.p;
        if (rot) {
            pn = (int64_t)a.renumber_base + rho;
            if (REF) {
                t.lo = t.rlo;
                t.hi = t.rhi;
            }
            rotate_quad(t.lo, t.hi, (double)(pn - psrc), th);
        }
        *reinterpret_cast<uint2 *>(a.Ko + dst + 4 * sub) = t.lo;
        *reinterpret_cast<uint2 *>(a.Ko + dst + D / 2 + 4 * sub) = t.hi;
        *reinterpret_cast<uint4 *>(a.Vo + dst + 8 * sub) = t.v;
        if (sub == 0 && a.po) a.po[(size_t)r * a.out_stride + slot] = (int32_t)pn;
        if (sub == 0 && a.score_out) a.score_out[(size_t)r * a.out_stride + slot] = t.sc;
        if (sub == 0 && a.tag_out) a.tag_out[(size_t)r * a.out_stride + slot] = (uint8_t)t.tg;
    };
    static_assert(U == 4, "the token batch below is written out for four tokens");
    const int64_t j0 = index(0), j1 = index(1), j2 = index(2), j3 = index(3);
    Tok t0 = fetch(j0), t1 = fetch(j1), t2 = fetch(j2), t3 = fetch(j3);
    put(t0, 0);
    put(t1, 1);
    put(t2, 2);
    put(t3, 3);
}

template <int D>
__global__ void __launch_bounds__(CMP_THREADS) compact_tiered(CompactArgs a) {
    constexpr int TPT = D / 4;
    constexpr int TOK = CMP_THREADS / TPT;
    constexpr int NW = CMP_THREADS / 64;
    __shared__ int32_t s_j[CMP_THREADS], s_slot[CMP_THREADS];
    __shared__ uint8_t s_tier[CMP_THREADS];
    __shared__ uint32_t s_wave[NW + 1];

    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int n = a.n_kept[r];
    KVC_NOTE(n > a.kept_stride, KVC_CHK_COUNT);
    if (n > a.kept_stride) n = a.kept_stride;
    if (n < 0) n = 0;
    const int sub = tid % TPT, tin = tid / TPT;
    const bool rot = a.renumber_base >= 0;
    double th0 = 0.0, th1 = 0.0;
    if (rot) {
        th0 = pow(a.rope_base, -2.0 * (2 * sub) / D);
        th1 = pow(a.rope_base, -2.0 * (2 * sub + 1) / D);
    }
    int carry_h = a.h_base ? a.h_base[r] : 0, carry_l = a.l_base ? a.l_base[r] : 0;
    if (carry_h < 0) carry_h = 0;
    if (carry_l < 0) carry_l = 0;
    for (int base = 0; base < n; base += CMP_THREADS) {
        const int rho = base + tid;
        const int act = rho < n ? a.action[(size_t)r * a.kept_stride + rho] : 0;
        const uint32_t v = (uint32_t)(act == 2) | ((uint32_t)(act == 1) << 16);
        // exclusive scan of (H, L) counts over the block
        uint32_t x = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) s_wave[wave] = x;
        __syncthreads();
        if (tid == 0) {
            uint32_t c = 0;
            for (int w = 0; w < NW; ++w) {
                const uint32_t t = s_wave[w];
                s_wave[w] = c;
                c += t;
            }
            s_wave[NW] = c;
        }
        __syncthreads();
        const uint32_t ex = s_wave[wave] + x - v;
        const uint32_t tot = s_wave[NW];
        int slot = -1;
        if (act == 2) slot = carry_h + (int)(ex & 0xFFFFu);
        if (act == 1) slot = carry_l + (int)(ex >> 16);
        KVC_NOTE(slot >= a.out_stride, KVC_CHK_COUNT);
        if (slot >= a.out_stride) slot = -1;
        s_j[tid] = rho < n ? a.kept[(size_t)r * a.kept_stride + rho] : -1;
        KVC_NOTE(s_j[tid] >= a.T, KVC_CHK_KEPT);
        s_slot[tid] = slot;
        s_tier[tid] = (uint8_t)act;
        __syncthreads();
        for (int e = tin; e < CMP_THREADS; e += TOK) {
            const int64_t j = s_j[e];
            const int sl = s_slot[e];
            const int tier = s_tier[e];
            // Uniform across the TPT-thread group: all of it reads the same entry.
            if (sl < 0 || j < 0 || j >= a.T || (tier != 1 && tier != 2)) continue;
            const int slc = KVC_IDX(sl, a.out_stride, KVC_CHK_COMPACT);
            const int rho_e = base + e;
            const size_t src = ((size_t)r * a.T + KVC_IDX(j, a.T, KVC_CHK_COMPACT)) * D;
            uint32_t lo = *reinterpret_cast<const uint32_t *>(a.K + src + 2 * sub);
            uint32_t hi = *reinterpret_cast<const uint32_t *>(a.K + src + D / 2 + 2 * sub);
            const uint2 vv = *reinterpret_cast<const uint2 *>(a.V + src + 4 * sub);
            const int64_t p = a.pos_in ? (int64_t)a.pos_in[(size_t)r * a.T + j] : j;
            int64_t pn = p;
            if (rot) {
                pn = (int64_t)a.renumber_base + rho_e;
                rotate_pairs(lo, hi, (double)(pn - p), th0, th1);
            }
            const size_t dst = ((size_t)r * a.out_stride + slc) * D;
            if (tier == 2) {
                *reinterpret_cast<uint32_t *>(a.Ko + dst + 2 * sub) = lo;
                *reinterpret_cast<uint32_t *>(a.Ko + dst + D / 2 + 2 * sub) = hi;
                *reinterpret_cast<uint2 *>(a.Vo + dst + 4 * sub) = vv;
                if (sub == 0 && a.po) a.po[(size_t)r * a.out_stride + slc] = (int32_t)pn;
            } else {
                const float k0 = bf16_to_f32((uint16_t)(lo & 0xFFFF)), k1 = bf16_to_f32((uint16_t)(lo >> 16));
                const float k2 = bf16_to_f32((uint16_t)(hi & 0xFFFF)), k3 = bf16_to_f32((uint16_t)(hi >> 16));
                const float v0 = bf16_to_f32((uint16_t)(vv.x & 0xFFFF)), v1 = bf16_to_f32((uint16_t)(vv.x >> 16));
                const float v2 = bf16_to_f32((uint16_t)(vv.y & 0xFFFF)), v3 = bf16_to_f32((uint16_t)(vv.y >> 16));
                const float kmax = token_max<TPT>(fmaxf(fmaxf(fabsf(k0), fabsf(k1)), fmaxf(fabsf(k2), fabsf(k3))));
                const float vmax = token_max<TPT>(fmaxf(fmaxf(fabsf(v0), fabsf(v1)), fmaxf(fabsf(v2), fabsf(v3))));
                const bool q4 = a.low_bits == 4;
                const float qm = q4 ? 7.f : 127.f;
                const uint16_t ksb = low_scale_bits(kmax, qm), vsb = low_scale_bits(vmax, qm);
                const float ks = f16_to_f32(ksb), vs = f16_to_f32(vsb);
                const int8_t c0 = quant_code(k0, ks, qm), c1 = quant_code(k1, ks, qm);
                const int8_t c2 = quant_code(k2, ks, qm), c3 = quant_code(k3, ks, qm);
                const int8_t w0 = quant_code(v0, vs, qm), w1 = quant_code(v1, vs, qm);
                const int8_t w2 = quant_code(v2, vs, qm), w3 = quant_code(v3, vs, qm);
                if (q4) {
                    // dimensions 2sub, 2sub+1 -> byte sub; D/2+2sub, +1 -> byte D/4+sub;
                    // values 4sub..4sub+3 -> bytes 2sub, 2sub+1
                    const size_t dq = ((size_t)r * a.out_stride + slc) * (D / 2);
                    uint8_t *kq = reinterpret_cast<uint8_t *>(a.Kq) + dq;
                    uint8_t *vq = reinterpret_cast<uint8_t *>(a.Vq) + dq;
                    kq[sub] = (uint8_t)nibble_pair(c0, c1);
                    kq[D / 4 + sub] = (uint8_t)nibble_pair(c2, c3);
                    *reinterpret_cast<uint16_t *>(vq + 2 * sub) =
                        (uint16_t)(nibble_pair(w0, w1) | (nibble_pair(w2, w3) << 8));
                } else {
                    int8_t *kq = a.Kq + dst;
                    int8_t *vq = a.Vq + dst;
                    *reinterpret_cast<uint16_t *>(kq + 2 * sub) = (uint16_t)((uint8_t)c0 | ((uint32_t)(uint8_t)c1 << 8));
                    *reinterpret_cast<uint16_t *>(kq + D / 2 + 2 * sub) =
                        (uint16_t)((uint8_t)c2 | ((uint32_t)(uint8_t)c3 << 8));
                    *reinterpret_cast<uint32_t *>(vq + 4 * sub) = (uint32_t)(uint8_t)w0 | ((uint32_t)(uint8_t)w1 << 8) |
                                                                 ((uint32_t)(uint8_t)w2 << 16) |
                                                                 ((uint32_t)(uint8_t)w3 << 24);
                }
                if (sub == 0) {
                    a.Ks[(size_t)r * a.out_stride + slc] = ksb;
                    a.Vs[(size_t)r * a.out_stride + slc] = vsb;
                    if (a.pq) a.pq[(size_t)r * a.out_stride + slc] = (int32_t)pn;
                }
            }
        }
        carry_h += (int)(tot & 0xFFFFu);
        carry_l += (int)(tot >> 16);
        __syncthreads();
    }
    if (tid == 0) {
        if (a.nh) a.nh[r] = carry_h < a.out_stride ? carry_h : a.out_stride;
        if (a.nl) a.nl[r] = carry_l < a.out_stride ? carry_l : a.out_stride;
    }
}

KVC_CHECK_READER(check_read_compact)

}  // namespace kvc

using namespace kvc;

extern "C" int kvc_compact_rerotate(const kvc_dims *dims, const uint16_t *K, const uint16_t *V,
                                    const int32_t *pos_in, const int32_t *kept_idx,
                                    int32_t kept_stride, const int32_t *n_kept, int32_t renumber_base,
                                    double rope_base, const kvc_compact_out *out, void *stream) {
    int st = check_dims(dims, "kvc_compact_rerotate");
    if (st != KVC_OK) return st;
    if (!K || !V || !kept_idx || !n_kept || !out)
        return fail(KVC_ERR_ARG, "kvc_compact_rerotate: NULL pointer");
    if (kept_stride <= 0 || out->out_stride <= 0 || out->kept_page < 0)
        return fail(KVC_ERR_ARG, "kvc_compact_rerotate: strides must be positive (kept %d, out %d, page %d)",
                    kept_stride, out->out_stride, out->kept_page);
    if (out->kept_page > 0 && out->action)
        return fail(KVC_ERR_UNSUPPORTED, "kvc_compact_rerotate: shared page lists take no action array");
    if ((int64_t)kept_stride * (out->kept_page > 0 ? out->kept_page : 1) > (int64_t)INT32_MAX)
        return fail(KVC_ERR_ARG, "kvc_compact_rerotate: kept tokens overflow int32");
    if (renumber_base >= 0 && !(rope_base > 1.0))
        return fail(KVC_ERR_ARG, "kvc_compact_rerotate: rope_base %g must exceed 1", rope_base);
    if (renumber_base >= 0 &&
        (int64_t)renumber_base + (int64_t)kept_stride * (out->kept_page > 0 ? out->kept_page : 1) >
            (int64_t)INT32_MAX)
        return fail(KVC_ERR_ARG, "kvc_compact_rerotate: renumbered positions overflow int32");
    if (out->low_bits != 0 && out->low_bits != 8 && out->low_bits != 4)
        return fail(KVC_ERR_UNSUPPORTED, "kvc_compact_rerotate: low_bits %d (0, 8 or 4)", out->low_bits);
    if (out->action) {
        if (!out->Kq || !out->Vq || !out->Ks || !out->Vs || !out->K_out || !out->V_out)
            return fail(KVC_ERR_ARG, "kvc_compact_rerotate: tiered output needs bf16 and int8 pools");
    } else if (!out->K_out || !out->V_out) {
        return fail(KVC_ERR_ARG, "kvc_compact_rerotate: K_out/V_out are NULL");
    }
    if (out->K_ref_out || out->p_ref_out || out->K_ref || out->p_ref) {
        if (!out->K_ref_out || !out->p_ref_out)
            return fail(KVC_ERR_ARG, "kvc_compact_rerotate: the reference store needs K_ref_out and p_ref_out");
        if ((out->K_ref == nullptr) != (out->p_ref == nullptr))
            return fail(KVC_ERR_ARG, "kvc_compact_rerotate: K_ref and p_ref go together");
        if (out->action || out->kept_page > 0)
            return fail(KVC_ERR_UNSUPPORTED,
                        "kvc_compact_rerotate: the reference store takes neither actions nor page lists");
        if (!(rope_base > 1.0))
            return fail(KVC_ERR_ARG, "kvc_compact_rerotate: the reference check needs rope_base > 1 (got %g)",
                        rope_base);
    }
    if ((out->score_in == nullptr) != (out->score_out == nullptr) || (out->tag_in == nullptr) != (out->tag_out == nullptr))
        return fail(KVC_ERR_ARG, "kvc_compact_rerotate: carried scores and tags need both in and out");
    if (out->action && (out->score_out || out->tag_out))
        return fail(KVC_ERR_UNSUPPORTED, "kvc_compact_rerotate: the tiered path carries no scores or tags");
    CompactArgs a;
    a.K = K;
    a.V = V;
    a.pos_in = pos_in;
    a.kept = kept_idx;
    a.n_kept = n_kept;
    a.action = out->action;
    a.T = dims->n_tokens;
    a.rows_per_seq = (int64_t)dims->n_layers * dims->n_kv_heads;
    a.kept_page = out->kept_page;
    a.kept_stride = kept_stride;
    a.out_stride = out->out_stride;
    a.renumber_base = renumber_base;
    a.rope_base = rope_base;
    a.Ko = out->K_out;
    a.Vo = out->V_out;
    a.po = out->pos_out;
    a.nh = out->n_h;
    a.Kq = out->Kq;
    a.Vq = out->Vq;
    a.Ks = out->Ks;
    a.Vs = out->Vs;
    a.pq = out->pos_q;
    a.nl = out->n_l;
    a.low_bits = out->low_bits == 4 ? 4 : 8;
    a.h_base = out->h_base;
    a.l_base = out->l_base;
    a.Kref = out->K_ref;
    a.pref = out->p_ref;
    a.Kref_out = out->K_ref_out;
    a.pref_out = out->p_ref_out;
    a.score_in = out->score_in;
    a.score_out = out->score_out;
    a.tag_in = out->tag_in;
    a.tag_out = out->tag_out;
    const int64_t rows = n_rows(dims);
    hipStream_t s = as_stream(stream);
    if (!out->action) {
        const int tok = CMP_THREADS / (dims->head_dim / 8);
        const int64_t listed = (int64_t)kept_stride * (out->kept_page > 0 ? out->kept_page : 1);
        const int cap = (int)(listed < out->out_stride ? listed : out->out_stride);
        int bpr = (cap + CMP_UNROLL * tok - 1) / (CMP_UNROLL * tok);  // CMP_UNROLL tokens per group
        if (bpr < 1) bpr = 1;
        if (rows * bpr > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "kvc_compact_rerotate: grid too large");
        const dim3 grid((unsigned)(rows * bpr)), block(CMP_THREADS);
        const bool ref = out->K_ref_out != nullptr;
        if (dims->head_dim == 128) {
            if (ref)
                compact_plain<128, true><<<grid, block, 0, s>>>(a, bpr);
            else
                compact_plain<128, false><<<grid, block, 0, s>>>(a, bpr);
        } else {
            if (ref)
                compact_plain<64, true><<<grid, block, 0, s>>>(a, bpr);
            else
                compact_plain<64, false><<<grid, block, 0, s>>>(a, bpr);
        }
    } else {
        if (dims->head_dim == 128)
            compact_tiered<128><<<dim3((unsigned)rows), dim3(CMP_THREADS), 0, s>>>(a);
        else
            compact_tiered<64><<<dim3((unsigned)rows), dim3(CMP_THREADS), 0, s>>>(a);
    }
    return check_launch("kvc_compact_rerotate");
}
