// Status plumbing, version, workspace sizing and the small host-side policy
// helpers of the kvc ABI.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kvc_internal.h"

namespace kvc {

static thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int check_launch(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(KVC_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return KVC_OK;
}

int check_dims(const kvc_dims *d, const char *who) {
    if (!d) return fail(KVC_ERR_ARG, "%s: dims is NULL", who);
    if (d->n_seq <= 0 || d->n_layers <= 0 || d->n_kv_heads <= 0 || d->n_q_heads <= 0 ||
        d->head_dim <= 0 || d->n_tokens <= 0 || d->reserved != 0)
        return fail(KVC_ERR_ARG, "%s: dims must be positive (N=%d L=%d Hkv=%d Hq=%d d=%d T=%lld)", who,
                    d->n_seq, d->n_layers, d->n_kv_heads, d->n_q_heads, d->head_dim,
                    (long long)d->n_tokens);
    if (d->n_q_heads % d->n_kv_heads)
        return fail(KVC_ERR_ARG, "%s: Hq=%d is not a multiple of Hkv=%d", who, d->n_q_heads, d->n_kv_heads);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(KVC_ERR_UNSUPPORTED, "%s: head_dim %d unsupported (64 or 128)", who, d->head_dim);
    if (d->n_tokens > (int64_t)INT32_MAX - 1)
        return fail(KVC_ERR_UNSUPPORTED, "%s: T=%lld exceeds int32 token indices", who,
                    (long long)d->n_tokens);
    if (n_rows(d) > (int64_t)INT32_MAX)
        return fail(KVC_ERR_UNSUPPORTED, "%s: too many rows", who);
    return KVC_OK;
}

// Defined in score.hip and select.hip.
size_t score_workspace_bytes(const kvc_dims *d, int32_t W);
size_t select_workspace_bytes(const kvc_dims *d, int32_t B);

// The check words of the kernel sources (bounds-checked builds).
unsigned check_read_score();
unsigned check_read_select();
unsigned check_read_compact();
unsigned check_read_decode();
unsigned check_read_pool();
unsigned check_read_page();

}  // namespace kvc

using namespace kvc;

extern "C" int kvc_version(void) { return 0 * 10000 + 1 * 100 + 0; }

extern "C" const char *kvc_last_error(void) { return g_last_error; }

extern "C" int kvc_check_read(void *stream, uint32_t *sites) {
    if (!sites) return fail(KVC_ERR_ARG, "kvc_check_read: sites is NULL");
    *sites = 0u;
#ifdef KVC_CHECK
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return fail(KVC_ERR_HIP, "kvc_check_read: stream");
    const unsigned words[] = {check_read_score(), check_read_select(), check_read_compact(),
                              check_read_decode(), check_read_pool(), check_read_page()};
    for (unsigned w : words) {
        if (w == ~0u) return fail(KVC_ERR_HIP, "kvc_check_read: copy of a check word failed");
        *sites |= w;
    }
    return KVC_OK;
#else
    (void)stream;
    return fail(KVC_ERR_UNSUPPORTED, "kvc_check_read: the library was built without KVC_CHECK");
#endif
}

extern "C" size_t kvc_workspace_bytes(int op, const kvc_dims *dims, int32_t W, int32_t B) {
    (void)B;
    if (check_dims(dims, "kvc_workspace_bytes") != KVC_OK) return 0;
    switch (op) {
    case KVC_OP_SCORE:
        if (W <= 0 || W > dims->n_tokens) {
            fail(KVC_ERR_ARG, "kvc_workspace_bytes: W=%d out of range", W);
            return 0;
        }
        return score_workspace_bytes(dims, W);
    case KVC_OP_SELECT:
        return select_workspace_bytes(dims, B);
    default:
        fail(KVC_ERR_ARG, "kvc_workspace_bytes: unknown op %d", op);
        return 0;
    }
}

extern "C" int32_t kvc_layer_group(int32_t layer, int32_t n_layers, int32_t n_groups) {
    if (n_layers <= 0 || n_groups <= 0 || layer < 0 || layer >= n_layers) return -1;
    int32_t g = 0;
    for (int32_t c = 1; c < n_groups; ++c) {
        int64_t boundary = ((int64_t)c * n_layers + n_groups - 1) / n_groups;  // ceil(c*L/n)
        if (layer >= boundary) ++g;
    }
    return g;
}

extern "C" double kvc_foresight_bonus(double sigma, double lambda, double steps_ahead) {
    return sigma * (0.5 + 0.5 * std::exp(-lambda * steps_ahead));
}
