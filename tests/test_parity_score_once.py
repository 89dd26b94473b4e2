"""GPU parity of kvc_score's single-read kernel (rows of d = 128, W*G = 128,
32,768 <= T <= ~106,000: the window score of PASK §3.1 Eq. 1 over CommitKV's
window, §3.1 Eq. 5, causal by CommitKV Eq. 6) against the float64 oracle and
against the two-pass path, through the C ABI.

The kernel keeps each key's exponentials in fp16 (round to nearest even,
relative error at most 2^-11) against a per-tile power-of-two reference, so a
score's relative error is at most ~5e-4 plus fp32 rounding: inside the 1e-3
relative bar the tests hold every fp32 score path to. The kernel is an option
(kvc_score_options), off by default; each test switches it on for its calls."""
import numpy as np
import pytest
import torch

from budgeted_retention_amd import synth
from oracle import numfmt, score as o_score
import kvc_testlib as tl

pytestmark = pytest.mark.gpu


def _scores(dims_args, K, Q, W, single_read=True):
    from budgeted_retention_amd import kvc
    N, L, Hkv, Hq, d, T = dims_args
    dims = kvc.make_dims(N, L, Hkv, Hq, d, T)
    ws = kvc.workspace(kvc.KVC_OP_SCORE, dims, W, 0, K.device)
    out = torch.full((N, L, Hkv, T), float("nan"), dtype=torch.float32, device=K.device)
    kvc.kvc_score_options(single_read)
    try:
        kvc.kvc_score(dims, K, Q, W, out, ws)
        kvc.kvc_score_status(ws)
    finally:
        kvc.kvc_score_options(False)
    return out.reshape(N * L * Hkv, T)


def _oracle_rows(K, Q, W, G, rows, L, Hkv):
    out = {}
    for r in rows:
        l, h = r // Hkv % L, r % Hkv
        n = r // (L * Hkv)
        out[r] = o_score.obs_window_score(tl.f64(K[n, l, h]), tl.f64(Q[n, l, h * G:(h + 1) * G]), W)
    return out


@pytest.mark.parametrize("T,L,Hkv", [(100_000, 4, 8), (32_768, 1, 5), (40_001, 7, 1), (106_000, 2, 3)])
def test_single_read_matches_oracle_and_two_pass(T, L, Hkv):
    """Ragged lengths: one split tile per row (32,768), a masked tail spread over
    split tiles and a row count not divisible by three (40,001 x 7), 241 split
    tiles per row (106,000); every row against the two-pass path, sampled rows
    against the oracle."""
    G, W, d = 4, 32, 128
    print(f"single read T={T} rows={L * Hkv}", flush=True)
    K = synth.normal_bf16((1, L, Hkv, T, d), T + 1, "cuda")
    Q = synth.normal_bf16((1, L, Hkv * G, W, d), T + 2, "cuda")
    dims = (1, L, Hkv, Hkv * G, d, T)
    one = _scores(dims, K, Q, W).cpu().numpy()
    two = _scores(dims, K, Q, W, single_read=False).cpu().numpy()
    assert np.isfinite(one).all()
    np.testing.assert_allclose(one, two, rtol=1e-3, atol=1e-7)
    np.testing.assert_allclose(one.sum(-1), W * G, rtol=1e-4)
    rows = sorted({0, L * Hkv // 2, L * Hkv - 1})
    for r, o in _oracle_rows(K, Q, W, G, rows, L, Hkv).items():
        tl.check_scores(one[r], o)


@pytest.mark.parametrize("profile", ["late_jump", "climb", "spike"])
def test_single_read_logit_ranges(profile):
    """Keys scaled so the logits leave every early reference far behind: a jump
    by 24x two thirds in, a climb by 2^(6 j / T), and one key 40x larger than
    the rest (its query rows' weight sits on it)."""
    G, W, d, T, L, Hkv = 4, 32, 128, 40_001, 1, 2
    K = synth.normal_bf16((1, L, Hkv, T, d), 7, "cpu").float()
    Q = synth.normal_bf16((1, L, Hkv * G, W, d), 8, "cpu")
    j = torch.arange(T, dtype=torch.float32)
    if profile == "late_jump":
        scale = torch.where(j >= 27_000, 24.0, 1.0)
    elif profile == "climb":
        scale = 2.0 ** (6.0 * j / T)
    else:
        scale = torch.where(j == 12_345, 40.0, 1.0)
    K = (K * scale[:, None]).to(torch.bfloat16)
    dims = (1, L, Hkv, Hkv * G, d, T)
    one = _scores(dims, K.cuda(), Q.cuda(), W).cpu().numpy()
    for r, o in _oracle_rows(K, Q, W, G, range(L * Hkv), L, Hkv).items():
        tl.check_scores(one[r], o)


def test_single_read_is_deterministic():
    G, W, d, T, L, Hkv = 4, 32, 128, 50_000, 3, 4
    # _scores switches the single-read kernel on for the call
    K = synth.normal_bf16((1, L, Hkv, T, d), 31, "cuda")
    Q = synth.normal_bf16((1, L, Hkv * G, W, d), 32, "cuda")
    dims = (1, L, Hkv, Hkv * G, d, T)
    a, b = _scores(dims, K, Q, W), _scores(dims, K, Q, W)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_single_read_gives_up_and_recovers():
    """With the merges switched off from the host, every wait for merged values
    runs out (50 us each): the kernel ends, the status reports it, and the next
    call with the default options is correct."""
    from budgeted_retention_amd import _lib, kvc
    G, W, d, T, L, Hkv = 4, 32, 128, 40_000, 2, 2
    K = synth.normal_bf16((1, L, Hkv, T, d), 41, "cuda")
    Q = synth.normal_bf16((1, L, Hkv * G, W, d), 42, "cuda")
    dims = kvc.make_dims(1, L, Hkv, Hkv * G, d, T)
    ws = kvc.workspace(kvc.KVC_OP_SCORE, dims, W, 0, K.device)
    out = torch.zeros((1, L, Hkv, T), dtype=torch.float32, device="cuda")
    kvc.kvc_score_options(True, 50, True)
    try:
        kvc.kvc_score(dims, K, Q, W, out, ws)
        with pytest.raises(_lib.KvcError):
            kvc.kvc_score_status(ws)
        kvc.kvc_score_options(True, 200000, False)
        kvc.kvc_score(dims, K, Q, W, out, ws)
        kvc.kvc_score_status(ws)
    finally:
        kvc.kvc_score_options(False)
    o = out.reshape(L * Hkv, T).cpu().numpy()
    for r, ref in _oracle_rows(K, Q, W, G, [0, L * Hkv - 1], L, Hkv).items():
        tl.check_scores(o[r], ref)
