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


# ---------------------------------------------------------------- reference store
#
# PACE §3.2 ("Non-compounding re-rotation") and Appendix D: re-rotating the
# stored bf16 key at every renumber adds one rounding per position change, so
# long-lived keys drift. PACE copies each resident key into a reference store
# at its first renumber, with the position p_ref it is valid at, and derives
# every later position from that copy, so a key carries about two roundings
# however often it moves. Entries move with their slots when rows are
# compacted and are checked against the stored key before use.
#
# Readings: the store holds the key bits the slot held at its first renumber
# (the key it was cached with) and that key's position. A reference is used
# when p_ref >= 0 and rotating it to the slot's current position reproduces the
# stored key within one bf16 step per element, plus 1e-5 of the reference
# row's largest magnitude (the fp32/fp64 rotation and sine differences); a
# reference that fails the check is treated as absent and the stored key
# becomes the new reference.


def ref_matches(K_bits_row, Kref_bits_row, p, p_ref, base):
    """The check before use: bf16(R_{p - p_ref} K_ref) agrees with the stored key."""
    if p_ref < 0:
        return False
    ref = numfmt.bf16_bits_to_f64(np.asarray(Kref_bits_row))
    got = numfmt.bf16_bits_to_f64(numfmt.f64_to_bf16_bits(rope.rotate(ref, p - p_ref, base)))
    stored = numfmt.bf16_bits_to_f64(np.asarray(K_bits_row))
    tol = np.maximum(np.abs(stored), 2.0 ** -126) * 2.0 ** -7 + 1e-5 * np.abs(ref).max()
    return bool(np.all(np.abs(got - stored) <= tol))


def compact_row_ref(K_bits, V_bits, pos, kept, renumber_base, base, Kref_bits=None, pref=None):
    """compact_row with a reference store.

    Kref_bits [T, d] uint16 and pref [T] ints are the store of the current
    slots (pref < 0 or None: no reference yet). Returns (K', V', pos', Kref',
    pref'): the renumbered keys derived from each token's reference (or from
    its stored key, which becomes the reference), and the store of the kept
    slots in rank order.
    """
    kept = np.asarray(kept, dtype=np.int64)
    K_bits = np.asarray(K_bits)
    pos = np.asarray(pos, dtype=np.int64)
    n = kept.size
    src = np.empty((n, K_bits.shape[1]), dtype=np.uint16)
    psrc = np.empty(n, dtype=np.int64)
    for r, j in enumerate(kept):
        pr = -1 if pref is None else int(pref[j])
        if Kref_bits is not None and ref_matches(K_bits[j], Kref_bits[j], pos[j], pr, base):
            src[r], psrc[r] = np.asarray(Kref_bits)[j], pr
        else:
            src[r], psrc[r] = K_bits[j], pos[j]
    V_sel = np.asarray(V_bits)[kept].copy()
    if renumber_base < 0:
        return K_bits[kept].copy(), V_sel, pos[kept], src, psrc
    p_new = renumber_base + np.arange(n, dtype=np.int64)
    k_new = rope.rotate(numfmt.bf16_bits_to_f64(src), p_new - psrc, base)
    return numfmt.f64_to_bf16_bits(k_new), V_sel, p_new, src, psrc
