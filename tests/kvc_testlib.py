"""Shared helpers for the parity tests: run the HIP path through the C ABI and
the float64 oracle on the same drawn inputs, and compare them by the rules
the workloads fix (kept sets exact up to near-threshold swaps, floating
outputs within stated tolerances)."""
import numpy as np
import torch

from oracle import compact as o_compact
from oracle import numfmt, policy as o_policy, score as o_score, select as o_select

SCORE_RTOL, SCORE_ATOL = 1e-3, 1e-6     # fp32 path; far inside the 1e-2 rel / 2e-2 abs bar
TIE_REL = 1e-3                          # swaps allowed within 1e-3 relative of the B-th total


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16/fp16 tensor -> uint16 numpy bits (on host)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def f64(t: torch.Tensor) -> np.ndarray:
    return numfmt.bf16_bits_to_f64(bits(t))


def gpu_path(dims_args, K, V, Q, W, policy, renumber_base, rope_base, kept_stride=None,
             out_stride=None, pos_in=None):
    """score -> select -> compact on the GPU. Returns a dict of host arrays."""
    from budgeted_retention_amd import kvc
    N, L, Hkv, Hq, d, T = dims_args
    dims = kvc.make_dims(N, L, Hkv, Hq, d, T)
    rows = N * L * Hkv
    dev = K.device
    ks = kept_stride or min(policy.budget, T)
    os_ = out_stride or ks
    ws = kvc.workspace(kvc.KVC_OP_SCORE, dims, W, 0, dev)
    scores = torch.empty((N, L, Hkv, T), dtype=torch.float32, device=dev)
    kvc.kvc_score(dims, K, Q, W, scores, ws)
    kept = torch.full((rows, ks), -1, dtype=torch.int32, device=dev)
    n_kept = torch.zeros(rows, dtype=torch.int32, device=dev)
    st = kvc.kvc_select(dims, scores, policy, kept, ks, n_kept)
    Ko = torch.zeros((rows, os_, d), dtype=torch.bfloat16, device=dev)
    Vo = torch.zeros_like(Ko)
    po = torch.full((rows, os_), -1, dtype=torch.int32, device=dev)
    nh = torch.zeros(rows, dtype=torch.int32, device=dev)
    out = kvc.CompactOut(os_, Ko, Vo, po, nh)
    kvc.kvc_compact_rerotate(dims, K, V, pos_in, kept, ks, n_kept, renumber_base, rope_base, out)
    torch.cuda.synchronize()
    return dict(status=st, scores=scores.cpu().numpy().reshape(rows, T), kept=kept.cpu().numpy(),
                n_kept=n_kept.cpu().numpy(), K=bits(Ko), V=bits(Vo), pos=po.cpu().numpy(),
                n_h=nh.cpu().numpy())


def assert_same_bits(a, b, path="out"):
    """Two runs of the same GPU path on the same inputs produced identical bits
    (dicts, lists, torch tensors on any device, numpy arrays, scalars)."""
    if isinstance(a, dict):
        assert a.keys() == b.keys(), path
        for k in a:
            assert_same_bits(a[k], b[k], f"{path}.{k}")
    elif isinstance(a, (list, tuple)):
        assert len(a) == len(b), path
        for i, (x, y) in enumerate(zip(a, b)):
            assert_same_bits(x, y, f"{path}[{i}]")
    elif torch.is_tensor(a):
        assert a.dtype == b.dtype and a.shape == b.shape, path
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), path
    elif isinstance(a, np.ndarray):
        assert a.dtype == b.dtype and a.shape == b.shape, path
        assert np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8)), path
    else:
        assert a == b or (a != a and b != b), path


def oracle_bonus_table(steps_ahead, sigma, lam):
    """[n_tags][1] float64 bonus table: tag 0 = no span, tag k+1 = span k (PACE Eq. 2)."""
    return np.array([[0.0]] + [[o_policy.foresight_bonus(sigma, lam, s)] for s in steps_ahead])


def oracle_row(K_row, Q_grp, W, tags, bonus_tbl, floor_tbl, group, n_sink, n_recent, B):
    """Oracle score/total/protection/kept for one row (float64)."""
    s = o_score.obs_window_score(K_row, Q_grp, W)
    tot, prot = o_policy.totals_and_protection(s, tags, bonus_tbl, floor_tbl, group, n_sink, n_recent)
    kept, excess = o_select.select_top_b(tot, prot, B)
    return s, tot, prot, kept, excess


def check_scores(g, o):
    np.testing.assert_allclose(g, o, rtol=1e-2, atol=2e-2)            # the workload bar
    np.testing.assert_allclose(g, o, rtol=SCORE_RTOL, atol=SCORE_ATOL)  # what fp32 reaches


def check_kept(g_kept, g_n, o_kept, tot, prot, B):
    """Kept sets equal except swaps among unprotected tokens whose oracle total lies
    within TIE_REL of the B-th total; the GPU set is ascending and holds every
    protected token."""
    g = np.asarray(g_kept[:g_n], dtype=np.int64)
    assert g_n == o_kept.size, (g_n, o_kept.size)
    assert np.all(np.diff(g) > 0), "kept indices not strictly ascending"
    assert set(np.flatnonzero(prot)).issubset(set(g.tolist())), "a protected token was dropped"
    diff = np.setxor1d(g, o_kept)
    if diff.size == 0:
        return 0
    free = np.setdiff1d(o_kept, np.flatnonzero(prot))
    thr = tot[free].min()
    near = np.abs(tot[diff] - thr) <= TIE_REL * abs(thr)
    assert near.all() and not prot[diff].any(), (
        f"{diff.size} kept-set differences, far from threshold {thr}: "
        f"{diff[~near][:10]} totals {tot[diff[~near]][:10]}")
    return diff.size


def check_compaction(gK, gV, gpos, K_bits, V_bits, pos, kept, renumber_base, rope_base):
    """GPU gather/re-rotation of `kept` against the oracle's on the same kept set:
    values bit-exact, positions exact, keys within one bf16 rounding step (the
    tolerance bar is 2e-2 abs / 1e-2 rel)."""
    oK, oV, op = o_compact.compact_row(K_bits, V_bits, pos, kept, renumber_base, rope_base)
    n = kept.size
    np.testing.assert_array_equal(gV[:n], oV)
    np.testing.assert_array_equal(gpos[:n], op)
    a, b = numfmt.bf16_bits_to_f64(gK[:n]), numfmt.bf16_bits_to_f64(oK)
    np.testing.assert_allclose(a, b, rtol=1e-2, atol=2e-2)
    # tighter than the bar: one bf16 rounding step of the output plus the fp32
    # sine/cosine/rotation error, which scales with the row's magnitude (a rotated
    # component can cancel to a small value whose own ulp is tiny)
    ulp = np.maximum(np.abs(b), 2.0 ** -126) * 2.0 ** -7
    slack = 1e-5 * np.abs(numfmt.bf16_bits_to_f64(K_bits[kept])).max(axis=1, keepdims=True)
    assert np.all(np.abs(a - b) <= ulp + slack), np.max((np.abs(a - b) - ulp) / slack)
    if renumber_base < 0:
        np.testing.assert_array_equal(gK[:n], oK)
