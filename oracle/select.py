"""Top-B selection under the budget (test infrastructure).

The kept set is every protected token plus the best of the rest by
(total descending, position ascending), until B tokens are kept:

* B counts the protected tokens (PACE Table 1: "B = 2,048 tokens, including
  4 sink and 128 recent").
* Ties go to the earlier position (PASK Appendix B.4: ties follow token
  position).
* Floors take precedence over the budget (PASK §3.5); when more than B tokens
  are protected, all of them are kept and the excess is reported
  (PASK Appendix B.4: floor excess is recorded).
* When T <= B every token is kept.
* The kept indices are returned in ascending order, so the same index set can
  be applied to keys, values and positions in order (CommitKV §3.1, Eq. 4).
"""
import numpy as np


def select_top_b(total, protected, B):
    """Return (kept ascending int64 indices, floor_excess bool)."""
    total = np.asarray(total, np.float64)
    protected = np.asarray(protected, bool)
    T = total.shape[0]
    if T <= B:
        return np.arange(T, dtype=np.int64), False
    P = np.flatnonzero(protected)
    if P.size >= B:
        return P.astype(np.int64), P.size > B
    rest = np.flatnonzero(~protected)
    # lexsort sorts by the last key first: total descending, then index ascending
    order = np.lexsort((rest, -total[rest]))
    chosen = rest[order[: B - P.size]]
    return np.sort(np.concatenate([P, chosen])).astype(np.int64), False
