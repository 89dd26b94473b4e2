"""GPU parity of score pooling (PASK Appendix C.3, Table 8) against the
float64 oracle, through the C ABI: max pooling is exact, the mean is within
fp32 summation error (1e-6 relative), and selection on pooled scores keeps
the oracle's set."""
import numpy as np
import pytest
import torch

from budgeted_retention_amd import synth
from oracle import score as o_score
import kvc_testlib as tl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,kernel", [(4096, 3), (4097, 7), (10_000, 63), (100, 255), (5, 7), (9000, 1)])
@pytest.mark.parametrize("mode", ["max", "avg"])
def test_pool_rows(T, kernel, mode):
    from budgeted_retention_amd import kvc
    rows = 3
    rng = np.random.default_rng(T + kernel)
    s = rng.gamma(0.5, 1.0, (rows, T)).astype(np.float32)
    dims = kvc.make_dims(1, 1, rows, rows, 64, T)
    out = torch.full((rows, T), -7.0, dtype=torch.float32, device="cuda")
    kvc.kvc_pool_scores(dims, torch.from_numpy(s).cuda(), kernel,
                        kvc.KVC_POOL_MAX if mode == "max" else kvc.KVC_POOL_AVG, out)
    g = out.cpu().numpy()
    for r in range(rows):
        want = o_score.pool_scores(s[r].astype(np.float64), kernel, mode)
        if mode == "max":
            np.testing.assert_array_equal(g[r], want)
        else:
            np.testing.assert_allclose(g[r], want, rtol=1e-6 * max(1, kernel / 8), atol=1e-7)


def test_pooled_selection_on_the_tiny_workload():
    """kvc_score -> kvc_pool_scores (max, 7) -> kvc_select against the oracle's
    window score, pooling and top-B on the same inputs."""
    from budgeted_retention_amd import kvc
    w = synth.WORKLOADS["tiny"]
    inp = synth.make_compaction_inputs(w, "cuda")
    N, L, Hkv, Hq, d, T, W, B = (w.n_seq, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim, w.n_tokens,
                                 w.window, w.budget)
    G = Hq // Hkv
    dims = kvc.make_dims(N, L, Hkv, Hq, d, T)
    scores = torch.empty((N * L * Hkv, T), dtype=torch.float32, device="cuda")
    kvc.kvc_score(dims, inp.K, inp.Q_obs, W, scores, kvc.workspace(kvc.KVC_OP_SCORE, dims, W, 0, "cuda"))
    pooled = torch.empty_like(scores)
    kvc.kvc_pool_scores(dims, scores, 7, kvc.KVC_POOL_MAX, pooled)
    pol = kvc.Policy(w.n_sink, w.n_recent, B, 1, 1, 0, L, None, torch.zeros((1, 1), device="cuda"))
    kept = torch.full((N * L * Hkv, B), -1, dtype=torch.int32, device="cuda")
    nk = torch.zeros(N * L * Hkv, dtype=torch.int32, device="cuda")
    kvc.kvc_select(dims, pooled, pol, kept, B, nk)
    torch.cuda.synchronize()
    z = np.zeros((1, 1))
    for r in range(N * L * Hkv):
        n, l, h = r // (L * Hkv), (r // Hkv) % L, r % Hkv
        s = o_score.obs_window_score(tl.f64(inp.K[n, l, h]), tl.f64(inp.Q_obs[n, l, h * G:(h + 1) * G]), W)
        p = o_score.pool_scores(s, 7, "max")
        from oracle import policy as o_policy, select as o_select
        tot, prot = o_policy.totals_and_protection(p, None, z, z.astype(np.uint8), 0, w.n_sink, w.n_recent)
        o_kept, _ = o_select.select_top_b(tot, prot, B)
        tl.check_kept(kept[r].cpu().numpy(), int(nk[r]), o_kept, tot, prot, B)


def test_pool_single_token_rows():
    from budgeted_retention_amd import kvc
    s = torch.tensor([[3.5], [-1.0]], dtype=torch.float32, device="cuda")
    dims = kvc.make_dims(1, 1, 2, 2, 64, 1)
    for mode in (kvc.KVC_POOL_MAX, kvc.KVC_POOL_AVG):
        out = torch.empty_like(s)
        kvc.kvc_pool_scores(dims, s, 63, mode, out)
        torch.cuda.synchronize()
        assert torch.equal(out, s)


@pytest.mark.parametrize("mode", ["max", "avg"])
def test_pool_full_session_shape_sampled_rows(mode):
    """The launch bench.py times: 36 layers x 8 KV heads of 100,000-token
    score rows, kernel 7; three rows checked against the oracle entry by entry."""
    from budgeted_retention_amd import kvc
    L, Hkv, T, kernel = 36, 8, 100_000, 7
    rows = L * Hkv
    gen = torch.Generator(device="cuda").manual_seed(20261229)
    s = torch.rand((rows, T), generator=gen, device="cuda", dtype=torch.float32) ** 4   # many small, few large
    dims = kvc.make_dims(1, L, Hkv, 4 * Hkv, 128, T)
    out = torch.full((rows, T), -7.0, dtype=torch.float32, device="cuda")
    kvc.kvc_pool_scores(dims, s, kernel, kvc.KVC_POOL_MAX if mode == "max" else kvc.KVC_POOL_AVG, out)
    torch.cuda.synchronize()
    for r in (0, 143, rows - 1):
        src = s[r].cpu().numpy()
        want = o_score.pool_scores(src.astype(np.float64), kernel, mode)
        got = out[r].cpu().numpy()
        if mode == "max":
            np.testing.assert_array_equal(got, want)
        else:
            np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-7)
