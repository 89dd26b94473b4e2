// Serial control steps of the path, run on the host: PASK's online
// structural controller and CommitKV's lifecycle classification. Both are
// small sequential loops whose outputs (per-token tier actions, candidate
// order) feed the GPU calls.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <numeric>
#include <vector>

#include "kvc.h"

namespace kvc {
int fail(int status, const char *fmt, ...);
}

using kvc::fail;

extern "C" int kvc_host_pask_costs(const int32_t *layers_per_group, int32_t n_groups, int32_t n_kv_heads,
                                   int32_t head_dim, int32_t low_bits, double *costs) {
    if (!layers_per_group || !costs || n_groups <= 0 || n_kv_heads <= 0 || head_dim <= 0 || low_bits <= 0)
        return fail(KVC_ERR_ARG, "kvc_host_pask_costs: bad arguments");
    for (int c = 0; c < n_groups; ++c) {
        if (layers_per_group[c] < 0) return fail(KVC_ERR_ARG, "kvc_host_pask_costs: negative layer count");
        // PASK Eq. 13: element and scale counts of the group's K and V rows
        const double n_c = 2.0 * layers_per_group[c] * n_kv_heads * head_dim;
        const double k_c = 2.0 * layers_per_group[c] * n_kv_heads;
        costs[3 * c + 0] = 0.0;                        // m(R)
        costs[3 * c + 1] = low_bits * n_c + 16.0 * k_c;  // m(L): codes + fp16 scales (Eq. 14)
        costs[3 * c + 2] = 16.0 * n_c;                 // m(H)
    }
    return KVC_OK;
}

// One token of PASK Algorithm 2 (§3.5, Eq. 11). Actions: 0 = R, 1 = L, 2 = H.
static double pask_token(const uint8_t *a0, const uint8_t *amin, const float *prio, bool critical,
                         double R_t, double gamma, const double *costs, int C, uint8_t *a) {
    auto cost = [&](const uint8_t *v) {
        double m = 0.0;
        for (int c = 0; c < C; ++c) m += costs[3 * c + v[c]];
        return m;
    };
    for (int c = 0; c < C; ++c) a[c] = std::max(a0[c], amin[c]);
    const double B_t = std::max(R_t - gamma, 0.0);
    // Demote in ascending stored priority until the cost fits or only floors remain.
    while (cost(a) > B_t) {
        int best = -1;
        float bp = 0.f;
        for (int c = 0; c < C; ++c) {
            if (a[c] > amin[c]) {
                const float p = prio[2 * c + (a[c] - 1)];  // the upgrade this demotion undoes
                if (best < 0 || p < bp) {
                    best = c;
                    bp = p;
                }
            }
        }
        if (best < 0) break;
        --a[best];
    }
    // Critical tags: promote in descending priority while the total still fits.
    if (critical) {
        for (;;) {
            int best = -1;
            float bp = 0.f;
            for (int c = 0; c < C; ++c) {
                if (a[c] < 2) {
                    const float p = prio[2 * c + a[c]];
                    if (best < 0 || p > bp) {
                        best = c;
                        bp = p;
                    }
                }
            }
            if (best < 0) break;
            const double delta = costs[3 * best + a[best] + 1] - costs[3 * best + a[best]];
            if (cost(a) + delta > B_t) break;
            ++a[best];
        }
    }
    return cost(a);
}

extern "C" int kvc_host_pask_control(const kvc_pask_table *tbl, const double *costs, double budget_fraction,
                                     double reserve, const uint8_t *tags, int32_t n_seq, int32_t n_tok,
                                     uint8_t *actions, double *ledger) {
    if (!tbl || !costs || !tags || !actions || n_seq <= 0 || n_tok < 0)
        return fail(KVC_ERR_ARG, "kvc_host_pask_control: bad arguments");
    const int C = tbl->n_groups;
    if (tbl->n_tags <= 0 || C <= 0 || !tbl->a0 || !tbl->amin || !tbl->prio || !tbl->critical)
        return fail(KVC_ERR_ARG, "kvc_host_pask_control: incomplete table");
    if (!(budget_fraction >= 0.0)) return fail(KVC_ERR_ARG, "kvc_host_pask_control: negative budget");
    double c_full = 0.0;
    for (int c = 0; c < C; ++c) c_full += costs[3 * c + 2];
    const double b = budget_fraction * c_full;  // per-token allowance
    for (int32_t n = 0; n < n_seq; ++n) {
        double R = b;  // R_1 = b
        if (ledger) ledger[(size_t)n * (n_tok + 1)] = R;
        for (int32_t t = 0; t < n_tok; ++t) {
            int z = tags[(size_t)n * n_tok + t];
            if (z >= tbl->n_tags) return fail(KVC_ERR_ARG, "kvc_host_pask_control: tag %d out of range", z);
            const double M = pask_token(tbl->a0 + (size_t)z * C, tbl->amin + (size_t)z * C,
                                        tbl->prio + (size_t)z * C * 2, tbl->critical[z] != 0, R, reserve,
                                        costs, C, actions + ((size_t)n * n_tok + t) * C);
            R = R - M + b;
            if (ledger) ledger[(size_t)n * (n_tok + 1) + t + 1] = R;
        }
    }
    return KVC_OK;
}

// Per-row physical actions of the generated tokens (PASK §3.2): the group's
// scheduled action for every layer of the group and every KV head, except the
// last `recent` tokens, which stay bf16 until they leave the window.
extern "C" int kvc_host_pask_row_actions(const uint8_t *actions, int32_t n_seq, int32_t n_tok, int32_t n_groups,
                                         int32_t n_layers, int32_t n_kv_heads, int32_t recent,
                                         uint8_t *row_actions) {
    if (!actions || !row_actions || n_seq <= 0 || n_tok < 0 || n_groups <= 0 || n_layers <= 0 ||
        n_kv_heads <= 0 || recent < 0)
        return fail(KVC_ERR_ARG, "kvc_host_pask_row_actions: bad arguments");
    const int32_t first_recent = recent < n_tok ? n_tok - recent : 0;
    for (int32_t n = 0; n < n_seq; ++n)
        for (int32_t l = 0; l < n_layers; ++l) {
            const int32_t g = kvc_layer_group(l, n_layers, n_groups);
            for (int32_t h = 0; h < n_kv_heads; ++h) {
                uint8_t *out = row_actions + (((size_t)n * n_layers + l) * n_kv_heads + h) * n_tok;
                const uint8_t *in = actions + (size_t)n * n_tok * n_groups + g;
                for (int32_t t = 0; t < first_recent; ++t) out[t] = in[(size_t)t * n_groups];
                for (int32_t t = first_recent; t < n_tok; ++t) out[t] = 2;   // H
            }
        }
    return KVC_OK;
}

extern "C" int kvc_host_event_pages(const int32_t *event_len, int32_t n_events, int32_t G, int64_t start,
                                    int32_t *first, int32_t *len, int32_t cap, int32_t *n_pages) {
    if (!event_len || !first || !len || !n_pages || n_events < 0 || G <= 0 || start < 0 || cap < 0)
        return fail(KVC_ERR_ARG, "kvc_host_event_pages: bad arguments");
    int64_t t = start, count = 0;
    for (int32_t i = 0; i < n_events; ++i) {
        const int64_t n_ev = event_len[i];
        if (n_ev <= 0) return fail(KVC_ERR_ARG, "kvc_host_event_pages: event %d has %lld tokens", i, (long long)n_ev);
        if (t + n_ev > INT32_MAX) return fail(KVC_ERR_ARG, "kvc_host_event_pages: tokens beyond 2^31 - 1");
        // cut from the event's first token: pages of G tokens, the last one shorter
        for (int64_t off = 0; off < n_ev; off += G, ++count)
            if (count < cap) {
                first[count] = (int32_t)(t + off);
                len[count] = (int32_t)(n_ev - off < G ? n_ev - off : G);
            }
        t += n_ev;
    }
    *n_pages = (int32_t)count;
    if (count > cap) return fail(KVC_ERR_ARG, "kvc_host_event_pages: %lld pages exceed cap %d", (long long)count, cap);
    return KVC_OK;
}

extern "C" int kvc_host_commit_candidates(const float *R_minus, const float *R_plus, int32_t n_pages,
                                          float tau_use, float tau_dead, float rho_use, float rho_dead,
                                          int32_t max_scan, uint8_t *state, int32_t *order, int32_t *n_order) {
    if (!R_minus || !R_plus || !state || !order || !n_order || n_pages <= 0 || max_scan <= 0)
        return fail(KVC_ERR_ARG, "kvc_host_commit_candidates: bad arguments");
    // Percentile rank: fraction of the other pages with a strictly smaller effect.
    auto percentiles = [&](const float *R, std::vector<double> &P) {
        std::vector<float> s(R, R + n_pages);
        std::sort(s.begin(), s.end());
        P.resize(n_pages);
        for (int32_t e = 0; e < n_pages; ++e) {
            const auto less = std::lower_bound(s.begin(), s.end(), R[e]) - s.begin();
            P[e] = n_pages > 1 ? (double)less / (n_pages - 1) : 0.0;
        }
    };
    std::vector<double> Pm, Pp;
    percentiles(R_minus, Pm);
    percentiles(R_plus, Pp);
    std::vector<int32_t> cand;
    for (int32_t e = 0; e < n_pages; ++e) {
        const bool Hm = R_minus[e] >= tau_use && Pm[e] >= rho_use;
        const bool Lm = R_minus[e] <= tau_dead && Pm[e] <= rho_dead;
        const bool Hp = R_plus[e] >= tau_use && Pp[e] >= rho_use;
        const bool Lp = R_plus[e] <= tau_dead && Pp[e] <= rho_dead;
        uint8_t st = KVC_LIFE_UNCERTAIN;
        if (Hm && Lp) st = KVC_LIFE_COMPLETION;
        else if (Lm && Lp) st = KVC_LIFE_DORMANT;
        else if (Lm && Hp) st = KVC_LIFE_NEWLY_ACTIVE;
        else if (Hm && Hp) st = KVC_LIFE_STILL_ACTIVE;
        state[e] = st;
        if (st == KVC_LIFE_COMPLETION) cand.push_back(e);
    }
    std::sort(cand.begin(), cand.end(), [&](int32_t x, int32_t y) {
        if (R_plus[x] != R_plus[y]) return R_plus[x] < R_plus[y];
        if (R_minus[x] != R_minus[y]) return R_minus[x] > R_minus[y];
        return x < y;
    });
    const int32_t n = std::min<int32_t>((int32_t)cand.size(), max_scan);
    for (int32_t i = 0; i < max_scan; ++i) order[i] = i < n ? cand[i] : -1;
    *n_order = n;
    return KVC_OK;
}

extern "C" int kvc_host_commit_protect(const float *R_minus, const int32_t *page_tokens, int32_t n_pending,
                                       int32_t budget, double eta, int32_t max_pages, uint8_t *protect,
                                       int32_t *n_protected) {
    if (!protect || !n_protected || n_pending < 0 || budget < 0 || max_pages < 0 || !(eta >= 0.0 && eta <= 1.0) ||
        (n_pending > 0 && (!R_minus || !page_tokens)))
        return fail(KVC_ERR_ARG, "kvc_host_commit_protect: bad arguments");
    const int64_t B_N = (int64_t)std::floor(eta * (double)budget);
    std::vector<int32_t> idx(n_pending);
    for (int32_t e = 0; e < n_pending; ++e) {
        idx[e] = e;
        protect[e] = 0;
        if (page_tokens[e] < 0) return fail(KVC_ERR_ARG, "kvc_host_commit_protect: negative page size");
    }
    std::sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) {
        if (R_minus[x] != R_minus[y]) return R_minus[x] > R_minus[y];
        return x < y;
    });
    int64_t used = 0;
    int32_t n = 0;
    for (int32_t e : idx) {  // a prefix of the order: the first page that does not fit ends it
        if (n >= max_pages || used + page_tokens[e] > B_N) break;
        protect[e] = 1;
        used += page_tokens[e];
        ++n;
    }
    *n_protected = n;
    return KVC_OK;
}

extern "C" int kvc_host_pace_renumber(int64_t m_next, int64_t shift, int32_t resident, int32_t limit,
                                      int32_t headroom, int32_t b_max, int32_t *renumber, int64_t *new_shift) {
    if (!renumber || !new_shift || resident < 0 || limit <= 0 || headroom < 0 || b_max < 0 || m_next < 0)
        return fail(KVC_ERR_ARG, "kvc_host_pace_renumber: bad arguments");
    if ((int64_t)limit <= (int64_t)b_max + headroom)
        return fail(KVC_ERR_ARG, "kvc_host_pace_renumber: limit %d must exceed B_max %d + headroom %d", limit, b_max,
                    headroom);
    if (resident > b_max) return fail(KVC_ERR_ARG, "kvc_host_pace_renumber: %d resident > B_max %d", resident, b_max);
    if (m_next - shift + headroom > (int64_t)limit) {
        *renumber = 1;
        *new_shift = m_next - resident;
    } else {
        *renumber = 0;
        *new_shift = shift;
    }
    return KVC_OK;
}
