/*
 * kvc -- budgeted KV-cache compaction on AMD MI355X (gfx950).
 *
 * C ABI of libkvc.so. The operations follow three pages on budgeted KV
 * retention:
 *   PASK     -- "Parser Transitions Already Reveal Structural Responsibility:
 *               KV Persistence for Structured Generation"
 *   PACE     -- "PACE: Keeping the Right Tokens in the KV Cache Is Not Enough
 *               for Long-Horizon LLM Agents"
 *   CommitKV -- "CommitKV: Lifecycle-Aware KV Cache Compression via Commit
 *               Transitions for Multi-Turn Agents"
 *
 * Conventions shared by every call:
 *  - Tensor arguments are DEVICE pointers to contiguous, row-major buffers
 *    that the caller owns; the library never allocates or frees device
 *    memory. bf16 tensors are passed as uint16_t bit patterns, fp16 scales
 *    likewise.
 *  - A "row" is one (sequence, layer, KV head) triple, r = (n*L + l)*Hkv + h.
 *    Query head g of a row's GQA group is absolute head h*G + g, G = Hq/Hkv.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call checks
 *    its arguments on the host, then only enqueues work on `stream`: it does
 *    not synchronise, so results are valid once the stream reaches them.
 *  - Argument errors return before anything is enqueued. KVC_ERR_HIP reports
 *    a failed launch. kvc_last_error() returns a thread-local description of
 *    the last non-OK status.
 *  - The library keeps no state between calls; calls on different streams
 *    may run concurrently if their buffers do not overlap.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvc_status {
    KVC_OK = 0,
    KVC_WARN_FLOOR_EXCESS = 1,  /* sink + recent alone exceed the budget: all protected tokens kept */
    KVC_ERR_ARG = -1,           /* NULL pointer, negative size, inconsistent shape */
    KVC_ERR_UNSUPPORTED = -2,   /* shape outside what the kernels handle (head_dim, W*G, ...) */
    KVC_ERR_WORKSPACE = -3,     /* workspace missing or smaller than kvc_workspace_bytes() */
    KVC_ERR_HIP = -4            /* the HIP runtime rejected a launch */
} kvc_status;

/* Shape of the cache buffers handed to a call. */
typedef struct kvc_dims {
    int32_t n_seq;       /* N */
    int32_t n_layers;    /* L: layers present in the buffers of this call */
    int32_t n_kv_heads;  /* Hkv */
    int32_t n_q_heads;   /* Hq, a multiple of Hkv */
    int32_t head_dim;    /* d: 64 or 128 */
    int32_t reserved;    /* must be 0 */
    int64_t n_tokens;    /* T: cached tokens per row */
} kvc_dims;

/* Library version, major*10000 + minor*100 + patch. */
int kvc_version(void);

/* Thread-local text for the last non-OK status returned on this thread. */
const char *kvc_last_error(void);

/*
 * Bounds-checked builds (the library compiled with -DKVC_CHECK, built as
 * libkvc_check.so beside libkvc.so; kernels otherwise the same). The global
 * indices the kernels compute from data (key and token indices of the gathers,
 * kept slots and output positions of the scatters, pool slots) are checked
 * against their ranges, and caller data the kernels clamp (kept indices at or
 * past the cache, counts above their buffers, page spans, block-table
 * entries) is noted; an index out of range is reported and replaced by one in
 * range instead of being used.
 * kvc_check_read synchronises `stream`, stores in *sites the bits of every
 * kind of access reported since the last read (0: none; bits 0-5: score,
 * select, compaction, decode, pooling, page kernels; bits 8-11: kept index,
 * count, page span, block-table entry) and clears them. In other builds it
 * returns KVC_ERR_UNSUPPORTED and stores 0.
 */
int kvc_check_read(void *stream, uint32_t *sites);

/* Operation ids for kvc_workspace_bytes(). */
enum { KVC_OP_SCORE = 1, KVC_OP_SELECT = 2 };

/* Device workspace (bytes) that operation `op` needs for these dims, window W
 * and budget B; 0 if it needs none. Returns 0 and sets the error on bad args. */
size_t kvc_workspace_bytes(int op, const kvc_dims *dims, int32_t W, int32_t B);

/*
 * Observation-window attention score (PASK §3.1 Eq. 1 attention; the
 * SnapKV-style window of PASK Appendix C and CommitKV's pre-commit window,
 * CommitKV §3.1 Eq. 5; causal rule of CommitKV Eq. 6).
 *
 * For every row and every cached token j < T:
 *   scores[r][j] = sum_{g<G} sum_{w<W} softmax_j( q_{g,w} . k_j / sqrt(d) )
 * where query (g, w) sits at position T-W+w and sees keys j <= T-W+w.
 *
 *   K       bf16 [N][L][Hkv][T][d]  cached (already rotated) keys
 *   Q_obs   bf16 [N][L][Hq][W][d]   rotated queries of the last W positions
 *   W       1 <= W <= T, W*G <= 256
 *   scores  fp32 [N][L][Hkv][T]     output, sums to W*G per row
 *   ws      device workspace of kvc_workspace_bytes(KVC_OP_SCORE, dims, W, 0) bytes;
 *           its first 32-bit word is the call's status once the stream has
 *           reached the end of the call (kvc_score_status)
 * Supported: d in {64, 128}. Deterministic (no float atomics).
 *
 * K is read twice: a statistics pass, then the scores. With
 * kvc_score_options(1, ...), rows of d = 128, W*G = 128 and 32,768 <= T <=
 * about 106,000 (a 100K-token Qwen3-8B-shaped row) read K once instead: a
 * persistent kernel, one workgroup per CU (a cooperative launch), keeps each
 * row's exponentials on chip until the row's normalisers are merged across
 * the chip. Every wait in it is bounded; a wait that runs out (only possible
 * if the workgroups were not all resident) ends the kernel early and sets
 * the status word. On MI355X it is measured slower than the two passes, so
 * it is off by default.
 */
int kvc_score(const kvc_dims *dims, const uint16_t *K, const uint16_t *Q_obs, int32_t W,
              float *scores, void *ws, size_t ws_bytes, void *stream);

/*
 * Options of kvc_score (process-wide; set them while no kvc_score call is
 * being enqueued): single_read = 1 uses the single-read kernel where it
 * applies, 0 (default) always reads K twice; wait_us bounds every wait of the
 * single-read kernel (default 200000); diag_no_merge = 1 stops the kernel's
 * merges so that every wait for merged values runs out (a test of the
 * give-up path; 0 in normal use). Returns KVC_ERR_ARG on bad values.
 */
int kvc_score_options(int32_t single_read, int64_t wait_us, int32_t diag_no_merge);

/*
 * Synchronises `stream` and reads the status word of the last kvc_score call
 * on workspace `ws` (NULL: the last kvc_score_noalloc call on the current
 * device). KVC_OK, or KVC_ERR_HIP when the single-read kernel gave up (the
 * scores of the rows it did not finish are undefined).
 */
int kvc_score_status(const void *ws, void *stream);

/*
 * kvc_score for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. It
 * takes no workspace; its scratch is a static device array of the library,
 * kvc_score_noalloc_max_bytes() bytes (16 MiB) on every GPU the library runs
 * on, held until the process ends. Same arguments, kernels and results as
 * kvc_score; calls whose workspace (kvc_workspace_bytes(KVC_OP_SCORE, ...))
 * would exceed the array return KVC_ERR_WORKSPACE before touching the device.
 * The call allocates nothing and enqueues on `stream` only.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (other streams, other threads) race and must be serialised by the caller.
 */
int kvc_score_noalloc(const kvc_dims *dims, const uint16_t *K, const uint16_t *Q_obs, int32_t W,
                      float *scores, void *stream);
size_t kvc_score_noalloc_max_bytes(void);

/* Pooling modes of kvc_pool_scores. */
enum { KVC_POOL_MAX = 0, KVC_POOL_AVG = 1 };

/*
 * Score pooling along the token axis (PASK Appendix C.3, Table 8: the SnapKV
 * baseline smooths its window scores by average or max pooling with an odd
 * kernel of 3, 5 or 7; the RocketKV baseline max-pools with a kernel of 63),
 * applied between kvc_score and kvc_select.
 *
 *   pooled[r][j] = max (KVC_POOL_MAX) or mean (KVC_POOL_AVG) of scores[r][j']
 *                  over |j' - j| <= kernel/2 and 0 <= j' < T
 * The window is cut at the row's ends: no padding enters the max or the mean.
 * The mean sums in token order in fp32 and divides once. Max ignores NaN
 * unless every value is NaN.
 *
 *   scores, pooled  fp32 [N][L][Hkv][T]; pooled must not alias scores
 *   kernel          odd, 1..255 (1 copies the scores)
 */
int kvc_pool_scores(const kvc_dims *dims, const float *scores, int32_t kernel, int32_t mode, float *pooled,
                    void *stream);

/*
 * Retention policy for kvc_select: bonus and protection floor per
 * (tag, layer group) from a frozen table (PASK §3.5 Eq. 11 lookup, PASK
 * Appendix A.2 layer groups; PACE §3.1 Eq. 2 foresight bonus, precomputed per
 * span tag), plus sink and recent-window protection (PASK Appendix B.2;
 * PACE Table 1 counts them inside the budget).
 */
typedef struct kvc_policy {
    int32_t n_sink;             /* tokens j < n_sink are protected */
    int32_t n_recent;           /* tokens j >= T - n_recent are protected */
    int32_t budget;             /* B: tokens kept per row, protected ones included */
    int32_t n_tags;             /* rows of the tables (>= 1); tag values >= n_tags read as 0 */
    int32_t n_groups;           /* columns of the tables (>= 1) */
    int32_t layer_base;         /* model index of the first layer in this call */
    int32_t n_layers_model;     /* model depth used for the group rule */
    int32_t tag_rows;           /* 0: tags [N][T], shared by a sequence's rows; 1: tags
                                   [N][L][Hkv][T], one per row (a resident cache whose slots
                                   hold different tokens in different rows) */
    const uint8_t *tags;        /* device u8 tag per token (layout by tag_rows), or NULL (all tag 0) */
    const float *tag_bonus;     /* device fp32 [n_tags][n_groups], or NULL (no bonus) */
    const uint8_t *tag_floor;   /* device u8 [n_tags][n_groups] 1 = protected, or NULL */
} kvc_policy;

/* Layer group of model layer `layer` among `n_groups` groups of an
 * n_layers-deep model: #{c in 1..n_groups-1 : layer >= ceil(c*n_layers/n_groups)}
 * (PASK Appendix A.2 generalised). Returns -1 on bad arguments. */
int32_t kvc_layer_group(int32_t layer, int32_t n_layers, int32_t n_groups);

/* PACE §3.1 Eq. 2 foresight bonus sigma*(1/2 + 1/2*exp(-lambda*steps_ahead))
 * for a span whose next reader is steps_ahead >= 0 steps away. Host helper
 * for filling tag_bonus. */
double kvc_foresight_bonus(double sigma, double lambda, double steps_ahead);

/*
 * Top-B selection under the budget (PACE §2 problem statement and §3.1
 * "keep the top-B by the sum"; PASK Appendix B.4 tie rule and floor excess;
 * CommitKV §3.1 Eq. 4 index set).
 *
 * Per row: total[j] = scores[j] + tag_bonus[tag_j][group(layer)];
 * protected[j] = j < n_sink || j >= T - n_recent || tag_floor[tag_j][group].
 * Kept set = every protected token plus the best unprotected tokens by
 * (total descending, index ascending) until `budget` tokens are kept; all T
 * if T <= budget; only the protected ones if they alone reach the budget.
 *
 *   scores     fp32 [N][L][Hkv][T]   (NaN totals rank lowest)
 *   kept_idx   int32 [N][L][Hkv][kept_stride]  ascending kept token indices;
 *              only the first min(n_kept, kept_stride) entries are written
 *   kept_stride  >= min(budget, T); >= T when tag_floor is given and T >
 *              budget (a floor can protect any token, and every protected
 *              token is kept, so only a full-length list holds them all);
 *              KVC_ERR_ARG otherwise
 *   n_kept     int32 [N][L][Hkv]  number of kept tokens. Excess caused by
 *              table floors is reported here only: n_kept > budget (the host
 *              cannot see the tags without a copy, and the call does not
 *              synchronise). Size the compaction's out_stride to hold n_kept.
 *   ws         device workspace of kvc_workspace_bytes(KVC_OP_SELECT, dims, 0, B)
 *              bytes. It is 0 (ws may be NULL) unless the rows are long: T >=
 *              262144, or fewer than 128 rows of T >= 32768. Such rows are
 *              split over several workgroups whose histograms and counts meet
 *              in the workspace; the call returns KVC_ERR_WORKSPACE before
 *              enqueueing anything if it is missing or too small. The
 *              workspace is overwritten; calls sharing one must not overlap.
 * Returns KVC_WARN_FLOOR_EXCESS (after enqueueing) when n_sink + n_recent
 * alone exceed the budget and T > budget: the one excess the host can see.
 */
int kvc_select(const kvc_dims *dims, const float *scores, const kvc_policy *policy,
               int32_t *kept_idx, int32_t kept_stride, int32_t *n_kept,
               void *ws, size_t ws_bytes, void *stream);

/* Outputs of kvc_compact_rerotate. Strides are in tokens per row. */
typedef struct kvc_compact_out {
    /* Per kept entry action, device u8 [N][L][Hkv][kept_stride]:
     * 0 = release, 1 = int8 tier, 2 = bf16 tier (PASK §3.2 {R, L, H}).
     * NULL = every kept token goes to the bf16 tier. */
    const uint8_t *action;
    int32_t out_stride;   /* capacity per row of every output pool below */
    /* 0: kept_idx / n_kept are per row ([N][L][Hkv][kept_stride] token
     * indices, [N][L][Hkv] counts). p > 0: they are per sequence
     * ([N][kept_stride] page indices, [N] page counts) and every layer and
     * head of sequence n keeps the tokens e*p .. e*p+p-1 of each listed page
     * e, in list order (CommitKV §3.1 Eq. 4: one index set for the token
     * axis). p > 0 requires action == NULL. */
    int32_t kept_page;
    /* Per-row first slot of this call's writes, device int32 [N][L][Hkv] or
     * NULL (= 0): appends after what an earlier call wrote (pass that call's
     * n_h / n_l). Must not alias the n_h / n_l outputs. */
    const int32_t *h_base;
    const int32_t *l_base;
    /* bf16 tier */
    uint16_t *K_out;      /* bf16 [N][L][Hkv][out_stride][d] */
    uint16_t *V_out;      /* bf16 [N][L][Hkv][out_stride][d] */
    int32_t *pos_out;     /* int32 [N][L][Hkv][out_stride], may be NULL */
    int32_t *n_h;         /* int32 [N][L][Hkv] rows written to the bf16 tier, may be NULL */
    /* int8 tier (required only when `action` is given) */
    int8_t *Kq;           /* int8 [N][L][Hkv][out_stride][d] */
    int8_t *Vq;           /* int8 [N][L][Hkv][out_stride][d] */
    uint16_t *Ks;         /* fp16 [N][L][Hkv][out_stride] per-token K scale */
    uint16_t *Vs;         /* fp16 [N][L][Hkv][out_stride] per-token V scale */
    int32_t *pos_q;       /* int32 [N][L][Hkv][out_stride], may be NULL */
    int32_t *n_l;         /* int32 [N][L][Hkv] rows written to the int8 tier, may be NULL */
    /* Reference store (PACE §3.2, non-compounding re-rotation; Appendix D):
     * per cache slot, the key that the slot's key was derived from and that
     * key's position. K_ref_out != NULL turns it on; only the plain path takes
     * it (action == NULL, kept_page == 0; else KVC_ERR_UNSUPPORTED), and
     * rope_base must exceed 1 even when renumber_base < 0.
     * Kept token j uses its reference when p_ref[j] >= 0 and the reference
     * passes the check before use: every element of bf16(R_{p - p_ref[j]}
     * K_ref[j]) within max(|K|, 2^-126) * 2^-7 + 1e-5 * max|K_ref[j]| of the
     * stored K[j]. Then K' = bf16(R_{p' - p_ref[j]} K_ref[j]) and the
     * reference is carried; otherwise K' = bf16(R_{p' - p} K[j]) and K[j] at
     * p becomes the reference. With renumber_base < 0 keys are copied and
     * only the store is rewritten. K_ref_out[rho] / p_ref_out[rho] follow the
     * kept order like K_out (from h_base). K_ref / p_ref NULL: no references
     * yet (each kept key starts one). Outputs must not alias the inputs. */
    const uint16_t *K_ref;    /* bf16 [N][L][Hkv][T][d], NULL together with p_ref */
    const int32_t *p_ref;     /* int32 [N][L][Hkv][T], < 0 = no reference */
    uint16_t *K_ref_out;      /* bf16 [N][L][Hkv][out_stride][d], or NULL */
    int32_t *p_ref_out;       /* int32 [N][L][Hkv][out_stride], with K_ref_out */
    /* Per-slot payloads that move with the kept tokens, in rank order like
     * K_out (plain path only, else KVC_ERR_UNSUPPORTED): a running score, such
     * as H2O's cumulative attention that PACE §3.1 adds the bonus to, and the
     * slot's tag for per-row policies (kvc_policy.tag_rows = 1). In and out
     * go together; NULL = not carried. */
    const float *score_in;    /* fp32 [N][L][Hkv][T] */
    float *score_out;         /* fp32 [N][L][Hkv][out_stride] */
    const uint8_t *tag_in;    /* u8 [N][L][Hkv][T] */
    uint8_t *tag_out;         /* u8 [N][L][Hkv][out_stride] */
    /* Low tier format (PASK Appendix B.5): 0 or 8 = int8 codes, Kq / Vq
     * [..][out_stride][d] with 7 -> 127; 4 = INT4, codes in [-7, 7], two
     * signed nibbles per byte (dimension 2i in the low nibble of byte i),
     * Kq / Vq [..][out_stride][d/2]. Scales as for int8. */
    int32_t low_bits;
} kvc_compact_out;

/*
 * Gather, renumber and exact re-rotation (PACE §3.2 "Bounded positions",
 * Proposition 1; CommitKV §3.1 Eq. 4 for the shared index set; PASK
 * Appendix B.5 for the int8 tier with 7 -> 127).
 *
 * For the rank rho-th kept token j = kept_idx[r][rho] (rho < n_kept[r]):
 *   p  = pos_in ? pos_in[r][j] : j
 *   p' = renumber_base + rho            (renumber_base >= 0)
 *   K' = bf16_rne( R_{p'-p} K[j] )      split-half RoPE, theta_i = rope_base^(-2i/d),
 *                                       angle (p'-p)*theta_i formed in fp64
 *   V' = V[j] (bit copy),  pos' = p'
 * With renumber_base < 0 positions are kept (p' = p) and K' = K[j] bit-exact.
 * The kept entries are then routed by `action` in rank order (stable):
 * bf16 tier rows are written as above; int8 tier rows get, separately for K'
 * and V', scale s = max(fp16_rne(max|x|/127), 2^-24) (a zero row: s = 1,
 * codes 0) and codes clamp(rne(x/s), -127, 127); released rows are dropped.
 *
 *   K, V      bf16 [N][L][Hkv][T][d]
 *   pos_in    int32 [N][L][Hkv][T] physical positions, or NULL (position = index)
 *   kept_idx  int32 [N][L][Hkv][kept_stride], n_kept int32 [N][L][Hkv] (from kvc_select);
 *             with out->kept_page = p > 0, [N][kept_stride] page indices and
 *             [N] page counts shared by the sequence's rows: rank rho is token
 *             kept_idx[n][rho / p] * p + rho % p
 *   Entries beyond min(n_kept, kept_stride) or past out_stride are ignored;
 *   an index outside [0, T) is skipped and leaves its slot as it was. n_h /
 *   n_l report base + the entries taken (skipped ones included).
 */
int kvc_compact_rerotate(const kvc_dims *dims, const uint16_t *K, const uint16_t *V,
                         const int32_t *pos_in, const int32_t *kept_idx, int32_t kept_stride,
                         const int32_t *n_kept, int32_t renumber_base, double rope_base,
                         const kvc_compact_out *out, void *stream);

/* Device workspace (bytes) kvc_decode_attn needs: `max_h` is the number of
 * bf16-partition tokens a row can address (stride_h, or blocks_per_seq *
 * page_size for a paged layout), `stride_l` the int8 capacity (0 if none). */
size_t kvc_decode_workspace_bytes(const kvc_dims *dims, int64_t max_h, int64_t stride_l);

/*
 * Decode attention over a compacted cache (PASK §3.1 Eq. 1 attention; PASK
 * Appendix B.5 disjoint bf16/low-precision partitions with fp32 statistics,
 * bf16 output and the Eq. 15 merge; grouped-query heads).
 *
 * For every row r and query head g of its group (absolute head h*G + g):
 *   o = sum_t softmax_t(q . k_t / sqrt(d)) v_t
 * over the union of the row's bf16 tokens (n_h[r] of them) and low-precision tokens
 * (n_l[r], dequantised as code * fp16 scale); every cached token is visible.
 *
 *   q            bf16 [N][L][Hq][d] (already rotated to the query position)
 *   K, V         bf16 [N][L][Hkv][stride_h][d]
 *   n_h          int32 [N][L][Hkv], clamped to the addressable tokens
 *   block_table  int32 [N][blocks_per_seq] or NULL. When given, token t of row
 *                (n, l, h) lives in slot block_table[n][t / page_size] *
 *                page_size + t % page_size of that row's storage (paged
 *                layout); slots outside [0, stride_h) are skipped.
 *   Kq, Vq       low-precision codes: low_bits 8 = int8 [N][L][Hkv][stride_l][d];
 *                low_bits 4 = INT4 nibble pairs [N][L][Hkv][stride_l][d/2] (PASK
 *                Appendix B.5, as kvc_compact_out.low_bits); Ks, Vs fp16 [N][L][Hkv][stride_l]
 *   n_l          int32 [N][L][Hkv], or NULL for no low-precision partition
 *   low_bits     8 or 4 (read only with n_l)
 *   o            bf16 [N][L][Hq][d] output; a row with no tokens gives o = 0
 *   lse          fp32 [N][L][Hq] natural-log normaliser (max + log sum), or NULL
 *   ws           kvc_decode_workspace_bytes(dims, max_h, stride_l) bytes
 * Supported: d in {64, 128}, G = Hq/Hkv <= 16.
 */
int kvc_decode_attn(const kvc_dims *dims, const uint16_t *q, const uint16_t *K, const uint16_t *V,
                    const int32_t *n_h, int64_t stride_h, const int32_t *block_table,
                    int32_t page_size, int32_t blocks_per_seq, const int8_t *Kq, const int8_t *Vq,
                    const uint16_t *Ks, const uint16_t *Vs, const int32_t *n_l, int64_t stride_l,
                    int32_t low_bits, uint16_t *o, float *lse, void *ws, size_t ws_bytes, void *stream);

/* Device workspace (bytes) kvc_decode_attn_h2o needs for a pool of stride_h
 * tokens per row. */
size_t kvc_decode_h2o_workspace_bytes(const kvc_dims *dims, int64_t stride_h);

/*
 * Decode attention with H2O cumulative attention (PACE §2 background: H2O
 * keeps the tokens with the largest attention received; PACE §3.1: the
 * foresight bonus is added to that cumulative score).
 *
 * The same attention as kvc_decode_attn over one unpaged bf16 pool, and for
 * every row r and cached token t < n_h[r]:
 *   acc[r][t] += sum over the row's G query heads g of softmax_t(q_g . k_t / sqrt(d))
 * (each call adds exactly G to a non-empty row). acc is read and written in
 * place; the caller sets the score of a newly cached token to 0 before the
 * step whose query attends to it. Softmax weights are formed in fp32 from the
 * merged normaliser; the running sum is fp32.
 *
 *   q, K, V, n_h, stride_h, o, lse  as kvc_decode_attn
 *   acc   fp32 [N][L][Hkv][stride_h]
 *   ws    kvc_decode_h2o_workspace_bytes(dims, stride_h) bytes
 * Supported: d in {64, 128}, G <= 16.
 */
int kvc_decode_attn_h2o(const kvc_dims *dims, const uint16_t *q, const uint16_t *K, const uint16_t *V,
                        const int32_t *n_h, int64_t stride_h, float *acc, uint16_t *o, float *lse,
                        void *ws, size_t ws_bytes, void *stream);

/* Device workspace (bytes) of kvc_page_effect / kvc_page_retire for a window
 * of W queries starting at position q_first. */
size_t kvc_page_workspace_bytes(const kvc_dims *dims, int32_t W, int64_t q_first);

/*
 * Pages (CommitKV §3.1, "Agent events and commit transitions": every event is
 * partitioned into contiguous pages of at most G tokens, cut at event
 * boundaries). The page calls below take either
 *   uniform pages:  page_first = page_len = NULL; page e of every sequence is
 *                   tokens [e*page_size, (e+1)*page_size); or
 *   event pages:    page_first, page_len device int32 [N][n_pages]; page e of
 *                   sequence n is tokens [page_first[n][e],
 *                   page_first[n][e] + page_len[n][e]), and page_size is the
 *                   longest a page may be (G). Entries are clamped to [0, T)
 *                   and to page_size; a page of length 0 has effect 0 and
 *                   score 0. Pages in token order without overlap run
 *                   fastest; any order is correct.
 */

/*
 * CommitKV page deletion effect (CommitKV §3.2, Eq. 6 renormalisation and
 * Eq. 7 relative change; the window of Eq. 5).
 *
 * For the chosen layer, window query w of query head hq sits at position
 * q_first + w and attends to the cached tokens j <= q_first + w (attention
 * weights a_j, output o). For every page E (e < n_pages) and every sequence n:
 *   effect_rel[n][e] = max over the layer's query heads and window queries of
 *                      ||o - o^{\E}|| / ||o||,  o - o^{\E} = sum_{j in E} a_j (v_j - o) / (1 - alpha_E)
 *   effect_abs[n][e] = the same maximum of ||o - o^{\E}||
 * A page whose deletion leaves nothing visible (alpha_E = 1) gets +inf; a
 * page no query sees gets 0.
 *
 *   K, V      bf16 [N][L][Hkv][T][d];  Q_win bf16 [N][L][Hq][W][d] (rotated)
 *   layer     0 <= layer < L;  q_first + W <= T;  W*G <= 256
 *   pages     uniform: page_size divides 64, n_pages*page_size <= T;
 *             event pages: 1 <= page_size <= 64
 *   effect_rel fp32 [N][n_pages];  effect_abs fp32 [N][n_pages] or NULL
 *   ws        kvc_page_workspace_bytes(dims, W, q_first) bytes
 */
int kvc_page_effect(const kvc_dims *dims, int32_t layer, const uint16_t *K, const uint16_t *V,
                    const uint16_t *Q_win, int32_t W, int64_t q_first, int32_t page_size,
                    const int32_t *page_first, const int32_t *page_len, int32_t n_pages,
                    float *effect_rel, float *effect_abs, void *ws, size_t ws_bytes, void *stream);

/*
 * CommitKV greedy joint retirement (CommitKV §3.3, Eq. 11). Per sequence n,
 * candidates order[n][0..n_cand) (page indices; -1 = no candidate) are
 * examined in that order; candidate E is accepted iff the effect, in the
 * sense of kvc_page_effect, of deleting E together with every page accepted
 * before it is <= tau_joint. The joint deletion treats all their tokens as
 * one set (Eq. 6 with the combined weights).
 *
 *   accepted   u8 [N][n_cand] 1 = retired;  joint_rel fp32 [N][n_cand] or NULL
 *              (the joint effect tested for each candidate, -1 for none)
 *   Other arguments as kvc_page_effect; page_size <= 16 (either kind).
 */
int kvc_page_retire(const kvc_dims *dims, int32_t layer, const uint16_t *K, const uint16_t *V,
                    const uint16_t *Q_win, int32_t W, int64_t q_first, int32_t page_size,
                    const int32_t *page_first, const int32_t *page_len, int32_t n_pages,
                    const int32_t *order, int32_t n_cand, float tau_joint, uint8_t *accepted,
                    float *joint_rel, void *ws, size_t ws_bytes, void *stream);

/*
 * Page scores for the compression checkpoint (CommitKV §3.3: pages accepted
 * for retirement are excluded and the retained index set, Eq. 13, is applied
 * to keys, values and positions alike, Eq. 4, so one page set serves every
 * layer and head of a sequence). For every sequence n and page e < n_pages:
 *   page_score[n][e] = sum over the page's tokens j (in order) of
 *                      sum over layers l and KV heads h (in order) of scores[n][l][h][j]
 * in fp32, and -inf for every page order[n][c] with accepted[n][c] != 0 (the
 * outputs of kvc_page_retire; entries outside [0, n_pages) are ignored).
 * Ranking the page scores with kvc_select (dims with T = n_pages, one layer,
 * one head) then keeps the best non-retired pages.
 *
 *   scores      fp32 [N][L][Hkv][T] (from kvc_score)
 *   page_size   1..1024;  uniform pages: n_pages*page_size <= T
 *   order, accepted  int32 / u8 [N][n_cand], both NULL for no exclusion
 *   page_score  fp32 [N][n_pages]
 */
int kvc_page_scores(const kvc_dims *dims, const float *scores, int32_t page_size,
                    const int32_t *page_first, const int32_t *page_len, int32_t n_pages,
                    const int32_t *order, const uint8_t *accepted, int32_t n_cand, float *page_score,
                    void *stream);

/*
 * Pages kept under a token budget (CommitKV §3.3, Eq. 13: the retained index
 * set holds at most B tokens; with event pages, §3.1, pages differ in
 * length). For every sequence n the pages are ranked by (page_score
 * descending, page index ascending), a NaN score below every other (-inf,
 * the score of a retired page, ranks below every finite one); the kept pages
 * are the longest prefix of that ranking whose lengths sum to at most
 * `budget`: the first page that does not fit ends it.
 *
 *   page_score   fp32 [N][n_pages] (from kvc_page_scores)
 *   pages        uniform or event pages as for the calls above (lengths
 *                clamped the same way); 1 <= page_size <= 4096,
 *                1 <= n_pages < 2^20
 *   budget       tokens, >= 0
 *   kept         int32 [N][kept_stride]: the first kept_stride kept pages in
 *                ascending order
 *   n_kept       int32 [N]: the number of kept pages (may exceed kept_stride;
 *                the rest are not written)
 *   n_tokens     int32 [N] or NULL: their total length (<= budget), which
 *                kvc_page_tokens then expands
 * With uniform pages of page_size tokens and a budget of k*page_size this is
 * kvc_select's top-k over the page scores.
 */
int kvc_page_select(const kvc_dims *dims, const float *page_score, int32_t page_size,
                    const int32_t *page_first, const int32_t *page_len, int32_t n_pages, int32_t budget,
                    int32_t *kept, int32_t kept_stride, int32_t *n_kept, int32_t *n_tokens, void *stream);

/*
 * Token list of per-sequence page lists: the retained index set of CommitKV
 * §3.3 Eq. 13 as one set of token indices for every layer and head (Eq. 4).
 * For sequence n the listed pages pages[n][0 .. min(n_listed[n], list_stride))
 * (for instance kvc_select's kept list over page scores) are expanded in list
 * order, each page's tokens in order; indices outside [0, n_pages) add
 * nothing. kvc_compact_rerotate with out->kept_page = 1 then compacts those
 * tokens, which is how event pages are compacted.
 *
 *   pages       int32 [N][list_stride];  n_listed int32 [N]
 *   tokens      int32 [N][out_stride]: the first out_stride token indices
 *   n_tokens    int32 [N]: the number of tokens of the listed pages (may
 *               exceed out_stride; the rest are not written)
 *   Page arguments as for the calls above, page_size <= 2^20 (dims: n_seq
 *   and n_tokens only).
 */
int kvc_page_tokens(const kvc_dims *dims, int32_t page_size, const int32_t *page_first,
                    const int32_t *page_len, int32_t n_pages, const int32_t *pages, const int32_t *n_listed,
                    int32_t list_stride, int32_t *tokens, int32_t *n_tokens, int32_t out_stride, void *stream);

/* ------------------------------------------------------------------------
 * Host-side serial control (plain C on host memory; no GPU work). Their
 * outputs feed the `action` argument of kvc_compact_rerotate and the `order`
 * argument of kvc_page_retire.
 * ---------------------------------------------------------------------- */

/* PASK Appendix B.3 payload costs (Eq. 13-14) per layer group, in bits:
 * costs[c][0..2] = m(R), m(L), m(H) with n_c = 2*layers*Hkv*d and
 * k_c = 2*layers*Hkv, m(H) = 16 n_c, m(L) = low_bits*n_c + 16 k_c, m(R) = 0.
 * costs is host double [n_groups][3]. */
int kvc_host_pask_costs(const int32_t *layers_per_group, int32_t n_groups, int32_t n_kv_heads,
                        int32_t head_dim, int32_t low_bits, double *costs);

/* Frozen PASK policy table (PASK §3.5 lookup), host memory. Actions are
 * 0 = release (R), 1 = low precision (L), 2 = bf16 (H). */
typedef struct kvc_pask_table {
    int32_t n_tags, n_groups;
    const uint8_t *a0;        /* [n_tags][n_groups] base action */
    const uint8_t *amin;      /* [n_tags][n_groups] floor action */
    const float *prio;        /* [n_tags][n_groups][2] stored priority of the upgrades R->L, L->H */
    const uint8_t *critical;  /* [n_tags] 1 = critical tag (promotions allowed) */
} kvc_pask_table;

/*
 * PASK online structural control, Algorithm 2 (§3.5, Eq. 11) per generated
 * token: a = max(a0, amin); B_t = [R_t - reserve]_+; demote the eligible
 * adjacent step with the smallest stored priority (never below the floor)
 * until M(a) <= B_t or only floors remain; for critical tags promote in
 * descending priority while the cost still fits (stopping at the first that
 * does not); R_{t+1} = R_t - M(a) + b with b = budget_fraction * C_full and
 * R_1 = b. The priority of a demotion is that of the upgrade it undoes;
 * priority ties go to the lower group.
 *   tags     host u8 [n_seq][n_tok];  actions host u8 [n_seq][n_tok][n_groups]
 *   ledger   host double [n_seq][n_tok + 1] (R_1 .. R_{n_tok+1}) or NULL
 */
int kvc_host_pask_control(const kvc_pask_table *tbl, const double *costs, double budget_fraction,
                          double reserve, const uint8_t *tags, int32_t n_seq, int32_t n_tok,
                          uint8_t *actions, double *ledger);

/*
 * Event pages of one sequence (CommitKV §3.1, "Agent events and commit
 * transitions": every completed event is partitioned into contiguous pages
 * of at most G tokens, so no page spans two events). Events follow one
 * another from token `start`; event i has event_len[i] >= 1 tokens and is
 * cut from its first token into pages of G tokens, the last one shorter.
 * Page p is tokens [first[p], first[p] + len[p]), in token order: the
 * page_first / page_len of the page calls (sequences whose page counts agree
 * are stacked as [N][n_pages]).
 *   event_len   host int32 [n_events]
 *   G           >= 1 (the page calls' page_size)
 *   first, len  host int32 [cap]
 *   n_pages     out: the number of pages. When it exceeds cap the call
 *               returns KVC_ERR_ARG after writing the first cap pages, with
 *               the full count in *n_pages. Tokens must stay below 2^31.
 */
int kvc_host_event_pages(const int32_t *event_len, int32_t n_events, int32_t G, int64_t start,
                         int32_t *first, int32_t *len, int32_t cap, int32_t *n_pages);

/*
 * Per-row physical actions of the generated tokens (PASK §3.2: the layers of
 * a group share the group's action but keep their own KV tensors; recent
 * tokens remain high precision and scheduled releases happen after they
 * leave the window; Appendix B.3 accounts for the recent window apart from
 * the scheduled payload, so the ledger of kvc_host_pask_control still
 * charges the scheduled action). For sequence n, layer l, KV head h and
 * generated token t:
 *   row_actions[n][l][h][t] = 2 (H)                          if t >= n_tok - recent
 *                           = actions[n][t][kvc_layer_group(l, n_layers, n_groups)]  otherwise
 * The result is the `action` argument of kvc_compact_rerotate for the
 * generated tokens (kept list 0 .. n_tok - 1).
 *   actions      host u8 [n_seq][n_tok][n_groups] (kvc_host_pask_control)
 *   row_actions  host u8 [n_seq][n_layers][n_kv_heads][n_tok]
 */
int kvc_host_pask_row_actions(const uint8_t *actions, int32_t n_seq, int32_t n_tok, int32_t n_groups,
                              int32_t n_layers, int32_t n_kv_heads, int32_t recent, uint8_t *row_actions);

/* CommitKV lifecycle states (CommitKV §3.2 Eq. 10). */
enum {
    KVC_LIFE_UNCERTAIN = 0,
    KVC_LIFE_COMPLETION = 1,
    KVC_LIFE_DORMANT = 2,
    KVC_LIFE_NEWLY_ACTIVE = 3,
    KVC_LIFE_STILL_ACTIVE = 4
};

/*
 * CommitKV lifecycle classification and candidate order (CommitKV §3.2
 * Eq. 9-10, §3.3). Percentile rank P(E) = #{E' : R(E') < R(E)} / (n_pages-1);
 * high: R >= tau_use and P >= rho_use; low: R <= tau_dead and P <= rho_dead.
 * Completion candidates (high before, low after) are ordered by R_plus
 * ascending, then R_minus descending, then page index; the first max_scan
 * go to `order` (padded with -1), their count to *n_order.
 *   R_minus, R_plus host fp32 [n_pages]; state host u8 [n_pages];
 *   order host int32 [max_scan].
 */
int kvc_host_commit_candidates(const float *R_minus, const float *R_plus, int32_t n_pages, float tau_use,
                               float tau_dead, float rho_use, float rho_dead, int32_t max_scan,
                               uint8_t *state, int32_t *order, int32_t *n_order);

/*
 * Pending-page protection at a compression checkpoint (CommitKV §3.3
 * "Protecting incomplete transitions", Eq. 12), on the host. Pages whose
 * pre-commit effect R_minus is known but whose post-commit measurement is
 * still to come are protected in order of decreasing R_minus (ties: lower
 * index) while their tokens total at most B_N = floor(eta * budget) and at
 * most max_pages pages are taken (the page's setup protects at most 16); the
 * first page that does not fit ends the walk. The protected pages are then
 * kept at the checkpoint (Eq. 13), e.g. as a floor tag in kvc_select.
 *
 *   R_minus, page_tokens  [n_pending] host arrays
 *   protect               u8 [n_pending] output, 1 = protected; *n_protected their count
 */
int kvc_host_commit_protect(const float *R_minus, const int32_t *page_tokens, int32_t n_pending,
                            int32_t budget, double eta, int32_t max_pages, uint8_t *protect,
                            int32_t *n_protected);

/*
 * Bounded positions (PACE §3.2, Renumbering and "Choosing L"), on the host.
 * Called after an eviction that leaves `resident` tokens per row, with
 * m_next the logical position of the next token and `shift` the sequence's
 * current shift (next physical position m_next - shift).
 *   KVC_ERR_ARG unless limit > b_max + headroom (b_max: the largest resident
 *   row, budget plus eviction interval; headroom: the most tokens appended
 *   between two checks) and resident <= b_max.
 *   *renumber = 1 when m_next - shift + headroom > limit: renumber the
 *   resident rows to 0..resident-1 (kvc_compact_rerotate with renumber_base
 *   0) and continue at physical position `resident`: *new_shift =
 *   m_next - resident. Otherwise *renumber = 0, *new_shift = shift.
 */
int kvc_host_pace_renumber(int64_t m_next, int64_t shift, int32_t resident, int32_t limit, int32_t headroom,
                           int32_t b_max, int32_t *renumber, int64_t *new_shift);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
