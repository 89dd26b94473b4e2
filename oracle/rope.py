"""Rotary position embedding R_p, split-half layout (test infrastructure).

PACE §2 ("Rotary positions", Eq. 1): a vector at position p is rotated
pairwise per frequency theta_i by the angle p*theta_i, so that
<R_m q, R_n k> = <q, R_{n-m} k> and R_a R_b = R_{a+b}. PACE §3.5 names the
layout it covers: full-rotary, split-half RoPE. For head width d and
i < d/2 the pair is (x_i, x_{i+d/2}) and theta_i = base**(-2i/d).

Angles are formed in float64 from an integer position: at positions near
2**20 a float32 angle would be off by a sizeable fraction of a radian.
"""
import numpy as np


def inv_freq(d, base):
    """theta_i = base**(-2i/d) for i in [0, d/2), float64."""
    if d % 2:
        raise ValueError("split-half RoPE needs an even head width")
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / d)


def rotate(x, pos, base):
    """Apply R_pos to x (float64, last axis = head width d).

    ``pos`` broadcasts against x's leading axes (integer or float64 array);
    positions may be negative, which rotates backwards.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq(d, base)
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)
