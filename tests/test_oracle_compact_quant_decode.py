"""Pins for the oracle's compaction/re-rotation, int8 codes and decode attention (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import compact, decode, numfmt, quant, rope


def _bf16(x):
    return numfmt.f64_to_bf16_bits(x)


def test_rerotation_matches_direct_rotation_prop1():
    # PACE Prop. 1: R_{p'-p} (R_p k) = R_{p'} k. Both sides pass through one bf16
    # rounding of the cached key, so they agree within about two bf16 roundings.
    rng = np.random.default_rng(11)
    T, d, base = 3000, 128, 1e6
    k = rng.standard_normal((T, d))
    pos = np.arange(T) * 333 + 17                      # positions up to ~1e6
    cached = _bf16(rope.rotate(k, pos, base))
    kept = np.sort(rng.choice(T, 256, replace=False))
    Kn, _, pn = compact.compact_row(cached, cached, pos, kept, 0, base)
    np.testing.assert_array_equal(pn, np.arange(256))
    want = rope.rotate(k[kept], pn, base)
    got = numfmt.bf16_bits_to_f64(Kn)
    err = np.abs(got - want) / (np.abs(want).max(axis=1, keepdims=True))
    assert err.max() < 2 * 2.0 ** -8


def test_rerotation_zero_shift_and_no_renumber_are_bit_copies():
    rng = np.random.default_rng(12)
    T, d = 100, 64
    K = _bf16(rng.standard_normal((T, d)))
    V = _bf16(rng.standard_normal((T, d)))
    kept = np.arange(10, 30)
    Kn, Vn, pn = compact.compact_row(K, V, np.arange(T), kept, 10, 1e4)   # p' = p
    np.testing.assert_array_equal(Kn, K[kept])
    np.testing.assert_array_equal(Vn, V[kept])
    Kn, Vn, pn = compact.compact_row(K, V, np.arange(T) + 5, kept, -1, 1e4)
    np.testing.assert_array_equal(Kn, K[kept])
    np.testing.assert_array_equal(pn, kept + 5)


def test_rerotation_round_trip():
    rng = np.random.default_rng(13)
    T, d, base = 64, 128, 1e6
    K = _bf16(rng.standard_normal((T, d)))
    kept = np.arange(T)
    far = np.arange(T) + 700000
    K1, _, p1 = compact.compact_row(K, K, far, kept, 0, base)      # rotate by -700000
    K2, _, _ = compact.compact_row(K1, K1, p1, kept, 700000, base)  # and back
    a, b = numfmt.bf16_bits_to_f64(K2), numfmt.bf16_bits_to_f64(K)
    assert np.max(np.abs(a - b) / np.abs(b).max(axis=1, keepdims=True)) < 2 * 2.0 ** -8


def test_renumbered_suffix_decodes_like_original_positions():
    # Shift invariance: keep the last B tokens, renumber them to 0..B-1 and place the
    # query at m_hat = m - (T - B); attention equals that at the original positions.
    rng = np.random.default_rng(14)
    T, B, d, base = 5000, 512, 64, 1e4
    k = rng.standard_normal((T, d))
    v = _bf16(rng.standard_normal((T, d)))
    q = rng.standard_normal(d)
    m = T
    K = _bf16(rope.rotate(k, np.arange(T), base))
    kept = np.arange(T - B, T)
    Kn, Vn, pn = compact.compact_row(K, v, np.arange(T), kept, 0, base)
    o_new, _ = decode.decode_head(rope.rotate(q, m - (T - B), base),
                                  numfmt.bf16_bits_to_f64(Kn), numfmt.bf16_bits_to_f64(Vn))
    o_old, _ = decode.decode_head(rope.rotate(q, m, base),
                                  numfmt.bf16_bits_to_f64(K[kept]), numfmt.bf16_bits_to_f64(v[kept]))
    np.testing.assert_allclose(o_new, o_old, atol=5e-3)


def _argmin_code(x, s, qmax):
    # independent definition: the integer in [-qmax, qmax] closest to x/s (ties to even)
    c = np.arange(-qmax, qmax + 1)
    err = np.abs(x - c * s)
    best = err.min()
    cand = c[np.isclose(err, best, rtol=0, atol=0)]
    return cand[0] if cand.size == 1 else cand[cand % 2 == 0][0]


def test_int8_codes_brute_force_and_bounds():
    rng = np.random.default_rng(15)
    X = numfmt.round_bf16(rng.standard_normal((40, 16)) * rng.uniform(0.01, 10, (40, 1)))
    codes, sb = quant.quantize_rows(X)
    for t in range(X.shape[0]):
        s = numfmt.fp16_bits_to_f64(sb[t])
        amax = np.abs(X[t]).max()
        assert sb[t] == numfmt.f64_to_fp16_bits(amax / 127)
        for i in range(X.shape[1]):
            assert codes[t, i] == _argmin_code(X[t, i], s, 127)
        unclipped = np.abs(X[t]) <= 127 * s
        assert np.all(np.abs(X[t] - codes[t] * s)[unclipped] <= s / 2 + 1e-300)
        i = np.argmax(np.abs(X[t]))
        assert abs(int(codes[t, i])) in (126, 127)


def test_int8_zero_row_and_tiny_scale():
    codes, s = quant.quantize_row(np.zeros(8))
    assert np.all(codes == 0) and numfmt.fp16_bits_to_f64(s) == 1.0
    x = np.zeros(8)
    x[3] = 2.0 ** -40                                  # scale would underflow fp16
    codes, s = quant.quantize_row(x)
    assert numfmt.fp16_bits_to_f64(s) == 2.0 ** -24
    assert codes[3] == 0


def test_decode_full_attention_matches_torch_sdpa():
    rng = np.random.default_rng(16)
    n, d = 300, 64
    q, K, V = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    o, _ = decode.decode_head(q, K, V)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None], torch.from_numpy(K)[None, None],
        torch.from_numpy(V)[None, None])[0, 0, 0].numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_decode_partition_merge_eq15_and_empty_partition():
    rng = np.random.default_rng(17)
    d = 32
    q = rng.standard_normal(d)
    parts = [(rng.standard_normal((n, d)), rng.standard_normal((n, d))) for n in (5, 0, 40, 1)]
    o_union, _ = decode.decode_partitions(q, parts)
    stats = []
    for K, V in parts:
        if len(K) == 0:
            continue
        s = K @ q / np.sqrt(d)
        vj = s.max()
        e = np.exp(s - vj)
        stats.append((vj, e.sum(), e @ V))
    np.testing.assert_allclose(decode.merge_partitions(stats), o_union, rtol=1e-12)
    o_noempty, _ = decode.decode_partitions(q, [p for p in parts if len(p[0])])
    np.testing.assert_array_equal(o_union, o_noempty)


def test_decode_single_token_returns_value():
    v = np.array([[0.5, -2.0, 3.25]])
    o, lse = decode.decode_head(np.array([1.0, 2.0, 3.0]), np.array([[1.0, 1.0, 1.0]]), v)
    np.testing.assert_array_equal(o, v[0])
    assert lse == pytest.approx(6.0 / np.sqrt(3))


# ---------------------------------------------------------------- reference store pins

def _churn(k, p0, steps, base, rng, store):
    """Renumber a set of keys `steps` times to fresh positions (eviction churn):
    with the store every key is re-derived from its first cached copy,
    without it the stored bf16 key is re-rotated each time."""
    K = _bf16(rope.rotate(k, p0, base))
    pos = p0.copy()
    Kref, pref = (None, None) if store else (None, None)
    for _ in range(steps):
        kept = np.arange(k.shape[0])
        rb = int(rng.integers(0, 6000))                        # new block of positions below L
        if store:
            K, _, pos, Kref, pref = compact.compact_row_ref(K, K, pos, kept, rb, base, Kref, pref)
        else:
            K, _, pos = compact.compact_row(K, K, pos, kept, rb, base)
    want = rope.rotate(k, pos, base)
    got = numfmt.bf16_bits_to_f64(K)
    return np.linalg.norm(got - want, axis=1) / np.linalg.norm(want, axis=1)


def test_reference_store_stops_drift_like_pace_appendix_d():
    # PACE Appendix D: naive re-rotation's mean relative key error grows with the
    # number of renumbers (0.011 after 23, 0.019 after 71: ratio 1.73, about
    # sqrt(71/23) = 1.76, one rounding per renumber adding up like a random walk);
    # §3.2: with the reference store the error stays at about two roundings
    # (max 0.003 after 60 renumbers, against 0.031 without).
    rng = np.random.default_rng(31)
    n, d, base = 200, 128, 1e6
    k = rng.standard_normal((n, d))
    p0 = rng.integers(0, 1_000_000, n)
    e23 = _churn(k, p0, 23, base, np.random.default_rng(1), False).mean()
    e71 = _churn(k, p0, 71, base, np.random.default_rng(2), False).mean()
    assert 1.5 < e71 / e23 < 2.0                                  # ~ sqrt(71/23): compounding
    naive60 = _churn(k, p0, 60, base, np.random.default_rng(3), False)
    store60 = _churn(k, p0, 60, base, np.random.default_rng(3), True)
    store1 = _churn(k, p0, 1, base, np.random.default_rng(3), True)
    assert store60.max() < 3 * 2.0 ** -8                           # about two bf16 roundings
    assert store60.max() < 1.5 * store1.max()                      # flat in the number of renumbers
    assert naive60.max() > 4 * store60.max()


def test_reference_store_first_renumber_and_checks():
    rng = np.random.default_rng(32)
    T, d, base = 300, 64, 1e4
    K = _bf16(rng.standard_normal((T, d)))
    V = _bf16(rng.standard_normal((T, d)))
    pos = np.arange(T) + 5000
    kept = np.sort(rng.choice(T, 40, replace=False))
    # first renumber: the stored keys become the references, at their positions
    K1, V1, p1, R1, q1 = compact.compact_row_ref(K, V, pos, kept, 0, base)
    Kn, Vn, pn = compact.compact_row(K, V, pos, kept, 0, base)
    np.testing.assert_array_equal(K1, Kn)
    np.testing.assert_array_equal(V1, Vn)
    np.testing.assert_array_equal(R1, K[kept])
    np.testing.assert_array_equal(q1, pos[kept])
    # second renumber from the references: one rotation from the original key
    kept2 = np.arange(0, 40, 3)
    K2, _, p2, R2, q2 = compact.compact_row_ref(K1, V1, p1, kept2, 100, base, R1, q1)
    direct = _bf16(rope.rotate(numfmt.bf16_bits_to_f64(K[kept][kept2]), p2 - pos[kept][kept2], base))
    np.testing.assert_array_equal(K2, direct)
    np.testing.assert_array_equal(R2, K[kept][kept2])
    # a stale reference (the slot was reused by another key) fails the check
    bad = R1.copy()
    bad[5] = _bf16(rng.standard_normal(d))
    assert not compact.ref_matches(K1[5], bad[5], p1[5], q1[5], base)
    assert compact.ref_matches(K1[6], R1[6], p1[6], q1[6], base)
    K3, _, _, R3, q3 = compact.compact_row_ref(K1, V1, p1, np.array([5, 6]), 0, base, bad, q1)
    np.testing.assert_array_equal(R3[0], K1[5])                    # the stored key is the new reference
    assert q3[0] == p1[5] and q3[1] == q1[6]
    # positions kept (no renumbering): keys copied, references carried
    K4, _, p4, R4, q4 = compact.compact_row_ref(K1, V1, p1, kept2, -1, base, R1, q1)
    np.testing.assert_array_equal(K4, K1[kept2])
    np.testing.assert_array_equal(R4, R1[kept2])


def test_int4_rule_on_a_hand_worked_row_pask_b5():
    # PASK Appendix B.5 with 7: amax 0.7 -> scale fp16(0.1) = 0.0999755859375;
    # 0.7/s = 7.0017 -> 7, -0.35/s = -3.5009 -> -4, 0 -> 0, 0.1/s = 1.0002 -> 1,
    # -0.7/s -> -7; packed low nibble first: (7, -4) -> 0xC7, (0, 1) -> 0x10,
    # (-7, pad 0) -> 0x09.
    x = np.array([0.7, -0.35, 0.0, 0.1, -0.7])
    codes, s_bits = quant.quantize_row(x, qmax=7)
    assert numfmt.fp16_bits_to_f64(s_bits) == 0.0999755859375
    np.testing.assert_array_equal(codes, [7, -4, 0, 1, -7])
    packed = quant.pack_nibbles(codes)
    np.testing.assert_array_equal(packed, np.array([0xC7, 0x10, 0x09], np.uint8))
    np.testing.assert_array_equal(quant.unpack_nibbles(packed, 5), codes)
    # zero row: zero codes, unit scale
    c0, s0 = quant.quantize_row(np.zeros(6), qmax=7)
    assert s0 == 0x3C00 and not c0.any() and not quant.pack_nibbles(c0).any()


def test_int4_round_trip_and_bounds():
    rng = np.random.default_rng(7)
    X = numfmt.bf16_bits_to_f64(numfmt.f64_to_bf16_bits(rng.standard_normal((200, 128)) * 3))
    codes, scales = quant.quantize_rows(X, qmax=7)
    assert codes.min() >= -7 and codes.max() <= 7
    s = numfmt.fp16_bits_to_f64(scales)
    err = np.abs(quant.dequantize_rows(codes, scales) - X)
    assert np.all(err <= s[:, None] * 0.5 + np.abs(X).max(axis=1, keepdims=True) * 2.0 ** -10)
    assert np.all(np.abs(codes).max(axis=1) == 7)                  # the row maximum maps to +-7
    allc = np.arange(-8, 8)
    np.testing.assert_array_equal(quant.unpack_nibbles(quant.pack_nibbles(np.tile(allc, (3, 1))), 16),
                                  np.tile(allc, (3, 1)))
