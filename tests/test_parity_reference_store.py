"""GPU parity of the reference store in kvc_compact_rerotate (PACE §3.2,
non-compounding re-rotation, with the check before use; Appendix D, drift
under eviction churn) against the float64 oracle, through the C ABI.

Each slot's reference is the key its cached key was derived from and that
key's position. Inputs are drawn from seeded generators; crafted slots are
made with the oracle's own rotation (valid references), with random bits
(stale references), with a position off by one, or with no reference. The
check's decision is compared exactly (the reference positions written out);
it is far from its tolerance edge on every crafted slot, so the kernel's fp32
rotation and the oracle's fp64 one take the same decision. Keys follow the
compaction bar: one bf16 step plus 1e-5 of the source row's magnitude.
"""
import numpy as np
import pytest
import torch

from budgeted_retention_amd import synth
from oracle import compact as o_compact, numfmt, rope
import kvc_testlib as tl

pytestmark = pytest.mark.gpu


def _dev_bits(a):
    if torch.is_tensor(a):
        return a
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _dev_i32(a):
    if a is None or torch.is_tensor(a):
        return a
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _gpu(K, V, pos, kept, n_kept, renumber_base, base, Kref=None, pref=None, out_stride=None, h_base=None):
    """One compaction with the store on; K, V, Kref [rows][T][d] uint16 bits
    (host or device bf16), pos / pref [rows][T], kept [rows][ks]. Returns host arrays."""
    from budgeted_retention_amd import kvc
    rows, T, d = K.shape
    ks = kept.shape[1]
    os_ = out_stride or ks
    dims = kvc.make_dims(1, 1, rows, rows, d, T)
    dK, dV = _dev_bits(K), _dev_bits(V)
    dR = None if Kref is None else _dev_bits(Kref)
    Ko = torch.zeros((rows, os_, d), dtype=torch.bfloat16, device="cuda")
    Vo, Ro = torch.zeros_like(Ko), torch.zeros_like(Ko)
    po = torch.full((rows, os_), -7, dtype=torch.int32, device="cuda")
    qo = torch.full((rows, os_), -7, dtype=torch.int32, device="cuda")
    nh = torch.zeros(rows, dtype=torch.int32, device="cuda")
    out = kvc.CompactOut(os_, Ko, Vo, po, nh, h_base=_dev_i32(h_base), K_ref=dR, p_ref=_dev_i32(pref),
                         K_ref_out=Ro, p_ref_out=qo)
    kvc.kvc_compact_rerotate(dims, dK, dV, _dev_i32(pos), _dev_i32(kept), ks, _dev_i32(n_kept),
                             renumber_base, base, out)
    torch.cuda.synchronize()
    return dict(K=tl.bits(Ko), V=tl.bits(Vo), pos=po.cpu().numpy(), Kref=tl.bits(Ro), pref=qo.cpu().numpy(),
                n_h=nh.cpu().numpy(), dev=(Ko, Vo, po, Ro, qo))


def _close_keys(g, o, src_bits):
    """Kernel keys against the oracle's: one bf16 step plus 1e-5 of the source row's magnitude."""
    a, b = numfmt.bf16_bits_to_f64(g), numfmt.bf16_bits_to_f64(o)
    np.testing.assert_allclose(a, b, rtol=1e-2, atol=2e-2)
    ulp = np.maximum(np.abs(b), 2.0 ** -126) * 2.0 ** -7
    slack = 1e-5 * np.abs(numfmt.bf16_bits_to_f64(src_bits)).max(axis=1, keepdims=True)
    assert np.all(np.abs(a - b) <= ulp + slack)


def _check_row(res, r, K, V, pos, kept_r, rb, base, Kref=None, pref=None, h0=0):
    oK, oV, op, oR, oq = o_compact.compact_row_ref(K[r], V[r], pos[r], kept_r, rb, base,
                                                   None if Kref is None else Kref[r],
                                                   None if pref is None else pref[r])
    n = kept_r.size
    sl = slice(h0, h0 + n)
    np.testing.assert_array_equal(res["pref"][r][sl], oq)          # the check's decisions
    np.testing.assert_array_equal(res["Kref"][r][sl], oR)          # references are bit copies
    np.testing.assert_array_equal(res["V"][r][sl], oV)
    np.testing.assert_array_equal(res["pos"][r][sl], op)
    if rb < 0:
        np.testing.assert_array_equal(res["K"][r][sl], oK)
    else:
        _close_keys(res["K"][r][sl], oK, oR)
    assert res["n_h"][r] == h0 + n
    return oK, oV, op, oR, oq


@pytest.mark.parametrize("d,T,n_keep", [(128, 3001, 700), (64, 1000, 333)])
def test_first_renumber_starts_the_store(d, T, n_keep):
    """No references yet: keys re-rotated from the stored keys (as without the
    store), which become the references at their old positions; appended at
    per-row offsets, with a ragged tail of workgroups."""
    rows = 3
    K = tl.bits(synth.normal_bf16((rows, T, d), 41 + d))
    V = tl.bits(synth.normal_bf16((rows, T, d), 42 + d))
    rng = np.random.default_rng(d)
    pos = np.sort(rng.choice(1_000_000, (rows, T), replace=False), axis=1)
    kept, n, _ = synth.kept_and_actions(rows, T, n_keep, seed=d, with_actions=False)
    h0 = np.array([0, 5, 64], np.int32)
    res = _gpu(K, V, pos, kept, n, 0, 1e6, out_stride=n_keep + 64, h_base=h0)
    for r in range(rows):
        kr = kept[r, : n[r]].astype(np.int64)
        _check_row(res, r, K, V, pos, kr, 0, 1e6, h0=h0[r])
        np.testing.assert_array_equal(res["pref"][r][h0[r]: h0[r] + kr.size], pos[r][kr])
        # the same keys as a compaction without the store
        oK, _, _ = o_compact.compact_row(K[r], V[r], pos[r], kr, 0, 1e6)
        _close_keys(res["K"][r][h0[r]: h0[r] + kr.size], oK, K[r][kr])


def _crafted_store(rows, T, d, base, seed):
    """Slots of five kinds, in a seeded random order: 0 valid reference,
    1 stale reference (random bits), 2 reference position off by one,
    3 no reference (p_ref = -1), 4 valid reference at distance zero."""
    rng = np.random.default_rng(seed)
    kind = rng.integers(0, 5, (rows, T))
    Kref = numfmt.f64_to_bf16_bits(rng.standard_normal((rows, T, d)))
    pref = rng.integers(0, 500_000, (rows, T))
    pos = pref + rng.integers(1, 500_000, (rows, T))
    pos[kind == 4] = pref[kind == 4]
    K = np.empty_like(Kref)
    for r in range(rows):
        K[r] = numfmt.f64_to_bf16_bits(rope.rotate(numfmt.bf16_bits_to_f64(Kref[r]), pos[r] - pref[r], base))
    stale = kind == 1
    K[stale] = numfmt.f64_to_bf16_bits(rng.standard_normal((int(stale.sum()), d)))
    pref = np.where(kind == 2, pref + 1, pref)
    pref = np.where(kind == 3, -1, pref)
    return K, Kref, pos, pref, kind


@pytest.mark.parametrize("d,base", [(128, 1e6), (64, 1e4)])
def test_valid_stale_and_missing_references(d, base):
    rows, T, n_keep = 2, 2500, 1100
    K, Kref, pos, pref, kind = _crafted_store(rows, T, d, base, seed=d)
    V = tl.bits(synth.normal_bf16((rows, T, d), 50 + d))
    kept, n, _ = synth.kept_and_actions(rows, T, n_keep, seed=60 + d, with_actions=False)
    res = _gpu(K, V, pos, kept, n, 17, base, Kref=Kref, pref=pref)
    for r in range(rows):
        kr = kept[r, : n[r]].astype(np.int64)
        _, _, _, _, oq = _check_row(res, r, K, V, pos, kr, 17, base, Kref, pref)
        used = np.isin(kind[r][kr], (0, 4))
        np.testing.assert_array_equal(oq == pref[r][kr], used)          # the crafted kinds were decided as built
        assert used.any() and (~used).any()


def test_no_renumber_copies_keys_and_carries_store():
    rows, T, d, base = 2, 900, 128, 1e6
    K, Kref, pos, pref, kind = _crafted_store(rows, T, d, base, seed=3)
    V = tl.bits(synth.normal_bf16((rows, T, d), 70))
    kept, n, _ = synth.kept_and_actions(rows, T, 300, seed=71, with_actions=False)
    res = _gpu(K, V, pos, kept, n, -1, base, Kref=Kref, pref=pref)
    for r in range(rows):
        _check_row(res, r, K, V, pos, kept[r, : n[r]].astype(np.int64), -1, base, Kref, pref)


def test_churn_error_stays_flat_like_pace_appendix_d():
    """60 renumbers of the same keys to fresh positions, slots permuted each
    time. The kernel's chain and the oracle's run side by side, each on its
    own outputs: the check's decisions and the references agree exactly at
    every step, keys stay within the compaction bar of the oracle's, and the
    error against the exactly rotated key stays at about two bf16 roundings,
    while re-rotating the stored key each time drifts."""
    from budgeted_retention_amd import kvc
    rows, n, d, base, steps = 2, 256, 128, 1e6, 60
    rng = np.random.default_rng(77)
    k = rng.standard_normal((rows, n, d))
    p0 = rng.integers(0, 1_000_000, (rows, n))
    K0 = np.stack([numfmt.f64_to_bf16_bits(rope.rotate(k[r], p0[r], base)) for r in range(rows)])
    V0 = tl.bits(synth.normal_bf16((rows, n, d), 78))
    oK, oV, op = K0.copy(), V0.copy(), p0.copy()
    oR, oq = [None] * rows, [None] * rows
    gK, gV, gp = _dev_bits(K0), _dev_bits(V0), torch.from_numpy(p0.astype(np.int32)).cuda()
    gR = gq = None
    nK = _dev_bits(K0)                                   # the store-less chain
    np_ = torch.from_numpy(p0.astype(np.int32)).cuda()
    truth_k = k.copy()
    for s in range(steps):
        perm = np.stack([rng.permutation(n) for _ in range(rows)]).astype(np.int32)
        rb = int(rng.integers(0, 6000))
        cnt = np.full(rows, n, np.int32)
        res = _gpu(gK, gV, gp, perm, cnt, rb, base, Kref=gR, pref=gq)
        for r in range(rows):
            oK[r], oV[r], op[r], oR[r], oq[r] = o_compact.compact_row_ref(
                oK[r], oV[r], op[r], perm[r], rb, base, oR[r], oq[r])
            np.testing.assert_array_equal(res["pref"][r], oq[r])
            np.testing.assert_array_equal(res["Kref"][r], oR[r])
            np.testing.assert_array_equal(res["V"][r], oV[r])
            np.testing.assert_array_equal(res["pos"][r], op[r])
            _close_keys(res["K"][r], oK[r], oR[r])
        gK, gV, gp, gR, gq = res["dev"]
        # store-less chain on the same permutation
        out = kvc.CompactOut(n, torch.empty_like(nK), torch.empty_like(nK),
                             torch.empty_like(np_), torch.zeros(rows, dtype=torch.int32, device="cuda"))
        dims = kvc.make_dims(1, 1, rows, rows, d, n)
        kvc.kvc_compact_rerotate(dims, nK, nK, np_, torch.from_numpy(perm).cuda(), n,
                                 torch.from_numpy(cnt).cuda(), rb, base, out)
        nK, np_ = out.K_out, out.pos_out
        truth_k = np.stack([truth_k[r][perm[r]] for r in range(rows)])
    torch.cuda.synchronize()
    pos_final = gp.cpu().numpy()
    np.testing.assert_array_equal(pos_final, np_.cpu().numpy())
    want = np.stack([rope.rotate(truth_k[r], pos_final[r], base) for r in range(rows)])
    err = lambda KK: (np.linalg.norm(tl.f64(KK) - want, axis=2) / np.linalg.norm(want, axis=2))
    e_store, e_naive = err(gK), err(nK)
    assert e_store.max() < 3 * 2.0 ** -8
    assert e_naive.max() > 4 * e_store.max()


def test_qwen3_8b_100k_shape_two_compactions_sampled_rows():
    """The 100K shape (288 rows of 100,000 tokens, d = 128, B = 2048) in the
    plain launch configuration: a first compaction starts the store; 2048
    new tokens (no references) are appended after the kept ones and a second
    compaction keeps 2048 of the 4096. Sampled rows against the oracle, each
    side on its own first-step outputs."""
    w = synth.WORKLOADS["qwen3_8b_100k"]
    rows, T, d, B = w.rows, w.n_tokens, w.head_dim, w.budget
    sample = [0, 137, rows - 1]
    K = synth.normal_bf16((rows, T, d), 901, "cuda")
    V = synth.normal_bf16((rows, T, d), 902, "cuda")
    Khost = {r: tl.bits(K[r]) for r in sample}
    Vhost = {r: tl.bits(V[r]) for r in sample}
    g = torch.Generator(device="cpu")
    g.manual_seed(903)
    kept = torch.rand((rows, T), generator=g).argsort(dim=1)[:, :B].sort(dim=1).values.to(torch.int32)
    pos = torch.arange(T, dtype=torch.int32, device="cuda").repeat(rows, 1)
    cnt = np.full(rows, B, np.int32)
    res1 = _gpu(K, V, pos, kept.numpy(), cnt, 0, w.rope_base, out_stride=2 * B)
    del K, V, pos
    o1 = {}
    for r in sample:
        kr = kept[r].numpy().astype(np.int64)
        o1[r] = o_compact.compact_row_ref(Khost[r], Vhost[r], np.arange(T), kr, 0, w.rope_base)
        np.testing.assert_array_equal(res1["pref"][r][:B], kr)
        np.testing.assert_array_equal(res1["Kref"][r][:B], o1[r][3])
        _close_keys(res1["K"][r][:B], o1[r][0], o1[r][3])
        np.testing.assert_array_equal(res1["V"][r][:B], o1[r][1])
    # second compaction over [kept 2048 | appended 2048]
    Ko, Vo, po, Ro, qo = res1["dev"]
    newK = synth.normal_bf16((rows, B, d), 904, "cuda")
    newV = synth.normal_bf16((rows, B, d), 905, "cuda")
    Ko[:, B:] = newK
    Vo[:, B:] = newV
    po[:, B:] = torch.arange(B, 2 * B, dtype=torch.int32, device="cuda")
    qo[:, B:] = -1
    kept2 = torch.rand((rows, 2 * B), generator=g).argsort(dim=1)[:, :B].sort(dim=1).values.to(torch.int32)
    res2 = _gpu(Ko, Vo, po, kept2.numpy(), cnt, 0, w.rope_base, Kref=Ro, pref=qo)
    nK, nV = tl.bits(newK), tl.bits(newV)
    for r in sample:
        K1 = np.concatenate([o1[r][0], nK[r]])
        V1 = np.concatenate([o1[r][1], nV[r]])
        p1 = np.concatenate([o1[r][2], np.arange(B, 2 * B)])
        R1 = np.concatenate([o1[r][3], np.zeros_like(nK[r])])
        q1 = np.concatenate([o1[r][4], np.full(B, -1)])
        k2 = kept2[r].numpy().astype(np.int64)
        oK, oV, op, oR, oq = o_compact.compact_row_ref(K1, V1, p1, k2, 0, w.rope_base, R1, q1)
        np.testing.assert_array_equal(res2["pref"][r], oq)
        np.testing.assert_array_equal(res2["Kref"][r], oR)
        np.testing.assert_array_equal(res2["V"][r], oV)
        np.testing.assert_array_equal(res2["pos"][r], op)
        _close_keys(res2["K"][r], oK, oR)
        old = k2 < B
        assert np.all(oq[old] == o1[r][4][k2[old]]) and np.all(oq[~old] == p1[k2[~old]])


def test_empty_rows_and_clamped_counts():
    """A row that keeps nothing writes nothing; a kept count above the list or
    the output room is clamped; references follow the same slots."""
    rows, T, d = 3, 500, 64
    K = tl.bits(synth.normal_bf16((rows, T, d), 81))
    V = tl.bits(synth.normal_bf16((rows, T, d), 82))
    pos = np.tile(np.arange(T), (rows, 1)) + 100
    kept = np.tile(np.arange(0, 400, 2, dtype=np.int32), (rows, 1))      # 200 listed per row
    n = np.array([0, 200, 10_000], np.int32)                              # empty, full, above the list
    res = _gpu(K, V, pos, kept, n, 0, 1e4, out_stride=150, h_base=np.array([0, 0, 20], np.int32))
    assert res["n_h"].tolist() == [0, 150, 150]
    assert np.all(res["pref"][0] == -7)                                   # nothing written
    _check_row(res, 1, K, V, pos, kept[1, :150].astype(np.int64), 0, 1e4, h0=0)
    _check_row(res, 2, K, V, pos, kept[2, :130].astype(np.int64), 0, 1e4, h0=20)
    assert np.all(res["pref"][2][:20] == -7)
