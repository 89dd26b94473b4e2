"""Pins for the bounded-position rule (CPU only)."""
from oracle import positions


def test_smallest_admissible_power_of_two_is_8192_pace_choosing_l():
    # PACE §3.2 "Choosing L": B = 2,048 and 4,096-token chunks make L = 8,192 the
    # smallest admissible power of two (B_max = budget + interval, interval < 2,048)
    for interval in (1, 128, 2047):
        ok = [L for L in (2 ** k for k in range(10, 16)) if positions.admissible(L, 2048 + interval, 4096)]
        assert ok[0] == 8192
    assert not positions.admissible(8192, 2048 + 2048, 4096)


def test_positions_stay_below_the_limit_and_renumbers_match_the_session_counts():
    # PACE: ~23 renumbers per 100K-token session, 242 at 1M and 480 at 2M with
    # L = 8K, a 2,048-token budget and H = 4,096 (the prefill chunk), sessions
    # growing by ~2,000-token steps; physical positions never reach L. The
    # spacing of renumbers is then about 4,000 tokens.
    for total, pages_count in ((100_000, 23), (1_000_000, 242), (2_000_000, 480)):
        n, top = positions.simulate(total, 2048, 2000, 8192, 4096)
        assert top < 8192
        assert abs(n - pages_count) <= 0.1 * pages_count + 2, (total, n)


def test_after_eviction_decision():
    assert positions.after_eviction(10_000, 4000, 2048, 8192, 2048) == (False, 4000)   # m_hat 6000 + 2048 < 8193
    assert positions.after_eviction(10_200, 4000, 2048, 8192, 2048) == (True, 10_200 - 2048)
