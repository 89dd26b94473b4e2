// kvc_pool_scores: smoothing of the token scores of every row before top-B
// selection, as the SnapKV baseline does (PASK Appendix C.3, Table 8: average
// or max pooling with an odd kernel of 3, 5 or 7; the RocketKV baseline there
// max-pools with a kernel of 63).
//
// pooled[r][j] = max or mean of scores[r][j'] over |j' - j| <= kernel / 2,
// 0 <= j' < T: the window is cut at the row's ends. One workgroup takes 4096
// tokens of one row and stages them with their halo in LDS; each thread then
// reduces the windows of its tokens from LDS, in token order for the mean.
#include "kvc_internal.h"

namespace kvc {

static constexpr int POOL_CHUNK = 4096;
static constexpr int POOL_THREADS = 256;
static constexpr int POOL_MAX_KERNEL = 255;

__global__ void __launch_bounds__(POOL_THREADS)
    pool_kernel(const float *__restrict__ in, float *__restrict__ out, int64_t T, int kernel, int mode, int chunks) {
    __shared__ float s[POOL_CHUNK + POOL_MAX_KERNEL - 1];
    const int64_t r = blockIdx.x / chunks;
    const int c = blockIdx.x % chunks;
    const int h = kernel / 2;
    const int64_t j0 = (int64_t)c * POOL_CHUNK;
    const int n = T - j0 < POOL_CHUNK ? (int)(T - j0) : POOL_CHUNK;
    const int64_t base = j0 - h;  // token of s[0]
    const float *row = in + (size_t)r * T;
    for (int i = threadIdx.x; i < n + 2 * h; i += POOL_THREADS) {
        const int64_t j = base + i;
        s[i] = (j >= 0 && j < T) ? row[j] : 0.f;   // out-of-row cells are never read below
    }
    __syncthreads();
    for (int t = threadIdx.x; t < n; t += POOL_THREADS) {
        const int64_t j = j0 + t;
        const int lo = (int)((j - h < 0 ? 0 : j - h) - base);
        const int hi = (int)((j + h > T - 1 ? T - 1 : j + h) - base);
        float v;
        if (mode == KVC_POOL_MAX) {
            v = s[lo];
            for (int q = lo + 1; q <= hi; ++q) v = fmaxf(v, s[q]);
        } else {
            v = 0.f;
            for (int q = lo; q <= hi; ++q) v += s[q];
            v = __fdiv_rn(v, (float)(hi - lo + 1));
        }
        out[(size_t)r * T + KVC_IDX(j, T, KVC_CHK_POOL)] = v;
    }
}

KVC_CHECK_READER(check_read_pool)

}  // namespace kvc

using namespace kvc;

extern "C" int kvc_pool_scores(const kvc_dims *dims, const float *scores, int32_t kernel, int32_t mode,
                               float *pooled, void *stream) {
    int st = check_dims(dims, "kvc_pool_scores");
    if (st != KVC_OK) return st;
    if (!scores || !pooled) return fail(KVC_ERR_ARG, "kvc_pool_scores: NULL pointer");
    if (scores == pooled) return fail(KVC_ERR_ARG, "kvc_pool_scores: pooled must not alias scores");
    if (kernel < 1 || kernel > POOL_MAX_KERNEL || kernel % 2 == 0)
        return fail(KVC_ERR_ARG, "kvc_pool_scores: kernel %d must be odd, 1..%d", kernel, POOL_MAX_KERNEL);
    if (mode != KVC_POOL_MAX && mode != KVC_POOL_AVG)
        return fail(KVC_ERR_ARG, "kvc_pool_scores: mode %d", mode);
    const int64_t T = dims->n_tokens;
    const int64_t chunks = (T + POOL_CHUNK - 1) / POOL_CHUNK;
    const int64_t blocks = n_rows(dims) * chunks;
    if (blocks > (int64_t)INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "kvc_pool_scores: grid too large");
    pool_kernel<<<dim3((unsigned)blocks), dim3(POOL_THREADS), 0, as_stream(stream)>>>(scores, pooled, T, kernel,
                                                                                       mode, (int)chunks);
    return check_launch("kvc_pool_scores");
}
