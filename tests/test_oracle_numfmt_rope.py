"""Pins for the oracle's number formats and RoPE (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import numfmt, rope


def test_bf16_rounding_matches_torch_cast_on_float32_inputs():
    # For float32-representable inputs one RNE step to bf16 is exactly torch's cast.
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),     # bf16 subnormals
        (rng.standard_normal(2000) * 1e38).astype(np.float32),      # near overflow
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf], np.float32),
    ])
    # exact ties: 1 + 2**-8 (half ulp) rounds to even (1.0); 1 + 3*2**-8 rounds up
    x = np.concatenate([x, np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8)], np.float32)])
    ours = numfmt.f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_rounding_is_single_rounding_from_float64():
    # 1 + 2**-8 + 2**-30 lies just above a tie: direct rounding goes up, while a
    # float32 intermediate (which drops 2**-30) would tie-break down to 1.0.
    x = np.array([1 + 2**-8 + 2**-30])
    assert numfmt.round_bf16(x)[0] == 1 + 2**-7


def test_bf16_widening_is_exact():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ours = numfmt.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


def test_fp16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(5000).astype(np.float32) * 0.01
    ours = numfmt.f64_to_fp16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


@pytest.mark.parametrize("d,base", [(64, 1e4), (128, 1e6)])
def test_inv_freq_endpoints(d, base):
    th = rope.inv_freq(d, base)
    assert th.shape == (d // 2,)
    assert th[0] == 1.0
    assert th[-1] == pytest.approx(base ** (-(d - 2) / d), rel=1e-15)
    assert np.all(np.diff(th) < 0)


def test_rope_matches_complex_multiplication():
    # Textbook form: pair (x_i, x_{i+d/2}) as z = x_i + i x_{i+d/2}; R_p z = z * exp(i p theta_i).
    rng = np.random.default_rng(3)
    d, base = 128, 1e6
    x = rng.standard_normal((7, d))
    p = np.array([0, 1, 17, 4095, 100000, 900001, 1048575])
    z = x[:, : d // 2] + 1j * x[:, d // 2:]
    zr = z * np.exp(1j * p[:, None] * rope.inv_freq(d, base)[None, :])
    ref = np.concatenate([zr.real, zr.imag], axis=1)
    np.testing.assert_allclose(rope.rotate(x, p, base), ref, rtol=0, atol=1e-12)


def test_rope_basis_vector_split_half_layout():
    d = 8
    e0 = np.zeros(d)
    e0[1] = 1.0                                 # pair i = 1 -> partner index 1 + d/2 = 5
    th = rope.inv_freq(d, 10000.0)[1]
    out = rope.rotate(e0, 3, 10000.0)
    exp = np.zeros(d)
    exp[1], exp[5] = np.cos(3 * th), np.sin(3 * th)
    np.testing.assert_allclose(out, exp, atol=1e-15)


def test_rope_group_laws():
    # PACE Eq. 1: R_a R_b = R_{a+b} and <R_m q, R_n k> = <q, R_{n-m} k>; R_0 = I; norms kept.
    rng = np.random.default_rng(4)
    d, base = 128, 1e6
    x = rng.standard_normal((5, d))
    a = np.array([3, 70000, -5, 123456, 0])
    b = np.array([9, 30000, 5, 900000, 0])
    np.testing.assert_allclose(rope.rotate(rope.rotate(x, b, base), a, base),
                               rope.rotate(x, a + b, base), atol=1e-11)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for m, n in [(0, 5), (4000, 100), (1048575, 2047)]:
        lhs = rope.rotate(q, m, base) @ rope.rotate(k, n, base)
        rhs = q @ rope.rotate(k, n - m, base)
        assert lhs == pytest.approx(rhs, abs=1e-9)   # angles near 1e6 rad: ~1e6 * 2**-53 each
    np.testing.assert_array_equal(rope.rotate(x, 0, base), x)
    np.testing.assert_allclose(np.linalg.norm(rope.rotate(x, a, base), axis=1),
                               np.linalg.norm(x, axis=1), rtol=1e-14)
