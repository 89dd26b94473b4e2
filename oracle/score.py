"""Observation-window attention score (test infrastructure).

For one (sequence, layer, KV head) row the cached keys K (T x d, already
rotated) are scored by the softmax attention that the last W cached queries
of every query head in the KV head's GQA group pay to them, summed over the
window and over the group:

    s[r, j]  = q_r . k_j / sqrt(d)                       (PASK §3.1, Eq. 1)
    a[r, j]  = softmax over the keys visible to r        (causal: j <= pos_r)
    score[j] = sum_r a[r, j]

The window is the final W query positions, as in the SnapKV scorer the PASK
page runs as a baseline (Appendix C) and CommitKV's pre-commit window
Q^- (§3.1, Eq. 5). The causal rule is CommitKV's "p_i <= p" (§3.2, Eq. 6).
Query rows are ordered (g, w): row r = g*W + w for query head g of the
group and window slot w, whose position is T - W + w.
"""
import numpy as np


def window_positions(T, W):
    """Positions of the W observation queries: T-W .. T-1."""
    return np.arange(T - W, T, dtype=np.int64)


def attention_weights(K, Q, q_pos, k_pos=None):
    """a[r, j] = softmax_j(q_r . k_j / sqrt(d)) over keys with k_pos <= q_pos[r].

    K: [T, d] float64, Q: [R, d] float64, q_pos: [R] ints,
    k_pos: [T] ints (default: 0..T-1). Invisible entries are exactly 0.
    """
    K = np.asarray(K, np.float64)
    Q = np.asarray(Q, np.float64)
    T, d = K.shape
    if k_pos is None:
        k_pos = np.arange(T, dtype=np.int64)
    s = (Q @ K.T) / np.sqrt(d)
    visible = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def obs_window_score(K, Qgrp, W):
    """score[j] for one row.

    K: [T, d] float64 cached keys. Qgrp: [G, W, d] float64 rotated queries of
    the group's G query heads at the final W positions. Returns [T] float64.
    """
    Qgrp = np.asarray(Qgrp, np.float64)
    G, W_, d = Qgrp.shape
    assert W_ == W
    T = K.shape[0]
    q_pos = np.tile(window_positions(T, W), G)          # row r = g*W + w
    a = attention_weights(K, Qgrp.reshape(G * W, d), q_pos)
    return a.sum(axis=0)


def pool_scores(score, kernel, mode):
    """Smoothing of a row's scores along the token axis before selection
    (PASK Appendix C.3, Table 8: SnapKV's pooling, avg or max with an odd
    kernel of 3, 5 or 7; the RocketKV baseline there scores the prefix with an
    odd max-pool kernel of 63).

    pooled[j] = max or mean of score[j'] over |j' - j| <= kernel // 2 with
    0 <= j' < T. Reading: the window is cut at the row's ends (no padding
    values enter the max or the mean). kernel 1 is the identity.
    """
    s = np.asarray(score, np.float64)
    T, h = s.shape[0], kernel // 2
    out = np.empty(T)
    for j in range(T):
        win = s[max(0, j - h):min(T, j + h + 1)]
        out[j] = win.max() if mode == "max" else win.mean()
    return out
