"""Bounded positions: when to renumber a resident row (test infrastructure).

PACE §3.2 ("Bounded positions", Renumbering): each resident slot keeps a
physical position; new tokens are written at m_hat = m - c for a per-sequence
shift c. When the next physical position would come within a headroom H of a
limit L (checked after each eviction), the resident row is renumbered to
0..R-1 in logical order and the shift is advanced so that the next token
continues at m_hat = R. "Choosing L": the limit must exceed the largest
resident row B_max (the budget plus the eviction interval) plus H, the most
tokens appended between two checks (a prefill chunk).

Reading: "within a headroom H" is m_hat + H > L (the next H tokens would
reach a position >= L).
"""


def admissible(limit, b_max, headroom):
    """The limit rule L > B_max + H."""
    return limit > b_max + headroom


def after_eviction(m_next, shift, resident, limit, headroom):
    """Decision after an eviction that left `resident` tokens, the next token
    being logical position m_next. Returns (renumber, new_shift): renumber
    is True when m_next - shift + headroom > limit, and then the next token
    continues at physical position `resident` (new_shift = m_next - resident)."""
    if m_next - shift + headroom > limit:
        return True, m_next - resident
    return False, shift


def simulate(total, budget, chunk, limit, headroom):
    """Renumbers in a session of `total` tokens appended `chunk` at a time,
    with an eviction back to `budget` resident tokens after every chunk (the
    policy evicts after each prefill chunk) and the limit checked after each
    eviction. Returns the number of renumbers and the largest physical
    position written."""
    shift, resident, m, renumbers, top = 0, 0, 0, 0, -1
    while m < total:
        n = min(chunk, total - m)
        top = max(top, m + n - 1 - shift)
        resident += n
        m += n
        resident = min(resident, budget)
        ren, shift2 = after_eviction(m, shift, resident, limit, headroom)
        if ren:
            renumbers += 1
            shift = shift2
    return renumbers, top
