"""Gather, renumber and exact re-rotation (test infrastructure).

PACE §3.2 ("Bounded positions"): the kept tokens of a row are renumbered in
logical order to p' in {0, ..., R-1} (order-preserving, gap-collapsing), and
every kept key is re-rotated from its position p to p'. Proposition 1: for a
cached key k~ = R_p k, R_{p'-p} k~ = R_{p'} k, so the renumbered key is the
one the engine would have cached at p'. The next query continues at R.

CommitKV §3.1, Eq. 4 applies one index set to keys, values and positions.
When renumbering is off (CommitKV and PASK keep absolute positions) keys are
copied unchanged.

Here the rotation by p'-p is applied directly with float64 angles, and the
re-rotated key is rounded once to bf16.
"""
import numpy as np

from . import numfmt, rope


def compact_row(K_bits, V_bits, pos, kept, renumber_base, base):
    """One row.

    K_bits, V_bits: [T, d] uint16 bf16 bits; pos: [T] ints (physical position
    of every slot); kept: [n] ascending slot indices; renumber_base: first new
    position (p' = renumber_base + rank), or a negative value to keep
    positions and skip rotation; base: RoPE base.
    Returns (K' bits [n, d], V' bits [n, d], pos' [n] int64).
    """
    kept = np.asarray(kept, dtype=np.int64)
    K_sel = np.asarray(K_bits)[kept]
    V_sel = np.asarray(V_bits)[kept].copy()
    p_old = np.asarray(pos, dtype=np.int64)[kept]
    if renumber_base < 0:
        return K_sel.copy(), V_sel, p_old
    p_new = renumber_base + np.arange(kept.size, dtype=np.int64)
    k = numfmt.bf16_bits_to_f64(K_sel)
    k_new = rope.rotate(k, p_new - p_old, base)
    return numfmt.f64_to_bf16_bits(k_new), V_sel, p_new
