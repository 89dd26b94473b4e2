"""H2O cumulative-attention scoring and eviction during decode (test infrastructure).

PACE §2 (background): H2O keeps the tokens with the largest attention received
so far plus a recent window, and the policy decides every few decoded tokens
which B entries to keep. PACE §3.1: the foresight bonus (Eq. 2) is added to
that cumulative attention score and eviction keeps the top-B by the sum.

Readings:

* The cumulative score of a cached token in one (layer, KV head) row is the
  sum, over decode steps and over the G query heads of the row's group, of
  the softmax weight the head's query gives the token. The group sum is the
  same aggregation the observation-window score uses.
* A decoded token is cached before its query attends, so it receives weight
  from its own step; its cumulative score starts at 0.
* Eviction runs every E decoded tokens over the resident row: totals =
  cumulative score + bonus of the slot's tag, sink / recent / floor
  protection by slot order (renumbering keeps the logical order), top-B by
  the same rule as the window-score path. The kept slots carry their
  cumulative scores and tags with them.
"""
import numpy as np

from . import policy, select


def attention_mass(q_group, K):
    """Sum over the group's query heads of each key's softmax weight.

    q_group: [G, d]; K: [n, d] (float64, n >= 1). Returns [n]. Each head's
    weights sum to one, so the result sums to G.
    """
    q_group = np.asarray(q_group, np.float64)
    K = np.asarray(K, np.float64)
    s = K @ q_group.T / np.sqrt(K.shape[1])        # [n, G]
    w = np.exp(s - s.max(axis=0, keepdims=True))
    w /= w.sum(axis=0, keepdims=True)
    return w.sum(axis=1)


def accumulate(acc, q_group, K):
    """One decode step's update of a row's cumulative scores: acc + mass."""
    return np.asarray(acc, np.float64) + attention_mass(q_group, K)


def evict(acc, tags, bonus_tbl, floor_tbl, group, n_sink, n_recent, B):
    """Kept slots (ascending) of a resident row under the budget."""
    total, prot = policy.totals_and_protection(acc, tags, bonus_tbl, floor_tbl, group, n_sink, n_recent)
    kept, _ = select.select_top_b(total, prot, B)
    return kept
