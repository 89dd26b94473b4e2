"""GPU parity of H2O cumulative-attention decode and eviction (PACE §2
background, §3.1: cumulative attention plus the foresight bonus, top-B every
few decoded tokens) against the float64 oracle, through the C ABI.

The attention output and normaliser are those of kvc_decode_attn. The
cumulative scores are fp32 on the GPU: each step's weights come from the
merged normaliser (relative error ~1e-6) and the running sum adds one fp32
rounding per step, so after s steps they agree with the float64 oracle to
1e-4 relative plus 1e-6 absolute, far inside the 1e-2 / 2e-2 bar. Evictions
follow the kept-set bar (swaps only within 1e-3 relative of the B-th total).
A row whose kept set differs by such a swap has a different resident set
from then on; its later cycles are not compared (the check counts them).
"""
import numpy as np
import pytest
import torch

from budgeted_retention_amd import synth
from oracle import decode as o_decode, h2o, numfmt, policy as o_policy
import kvc_testlib as tl

pytestmark = pytest.mark.gpu

MASS_RTOL, MASS_ATOL = 1e-4, 1e-6


def _h2o_call(dims, q, K, V, n_h, stride, acc):
    from budgeted_retention_amd import kvc
    N, L, Hq, d = dims.n_seq, dims.n_layers, dims.n_q_heads, dims.head_dim
    o = torch.empty((N, L, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((N, L, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, kvc.kvc_decode_h2o_workspace_bytes(dims, stride)), dtype=torch.uint8, device="cuda")
    kvc.kvc_decode_attn_h2o(dims, q, K, V, n_h, stride, acc, o, ws, lse)
    o2 = torch.empty_like(o)
    lse2 = torch.empty_like(lse)
    ws2 = torch.empty(max(1, kvc.kvc_decode_workspace_bytes(dims, stride, 0)), dtype=torch.uint8, device="cuda")
    kvc.kvc_decode_attn(dims, q, K, V, n_h, stride, o2, ws2, lse2)
    torch.cuda.synchronize()
    return o, lse, o2, lse2


@pytest.mark.parametrize("d,Hkv,Hq,stride,counts", [
    (128, 2, 8, 1031, [0, 1, 255, 256, 257, 1031]),     # G = 4, ragged chunk tails, an empty row
    (64, 1, 7, 600, [600, 333, 17]),                     # G = 7, three layers
    (128, 4, 4, 300, [300, 1, 299, 128]),                # G = 1
])
def test_decode_h2o_adds_each_keys_attention_mass(d, Hkv, Hq, stride, counts):
    from budgeted_retention_amd import kvc
    L = len(counts) // Hkv
    rows = L * Hkv
    G = Hq // Hkv
    dims = kvc.make_dims(1, L, Hkv, Hq, d, stride)
    K = synth.normal_bf16((rows, stride, d), 11 + d, "cuda")
    V = synth.normal_bf16((rows, stride, d), 12 + d, "cuda")
    q = synth.normal_bf16((1, L, Hq, d), 13 + d, "cuda")
    n_h = torch.tensor(counts, dtype=torch.int32, device="cuda")
    acc0 = torch.from_numpy(np.random.default_rng(d).gamma(0.5, 3.0, (rows, stride)).astype(np.float32)).cuda()
    acc = acc0.clone()
    o, lse, o2, lse2 = _h2o_call(dims, q, K, V, n_h, stride, acc)
    # the attention itself is kvc_decode_attn's, bit for bit
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse, lse2)
    a, a0 = acc.cpu().numpy().astype(np.float64), acc0.cpu().numpy().astype(np.float64)
    Kh, Vh, qh = tl.f64(K), tl.f64(V), tl.f64(q)
    for r in range(rows):
        n = counts[r]
        l, h = r // Hkv, r % Hkv
        np.testing.assert_array_equal(a[r, n:], a0[r, n:])          # slots past n_h untouched
        if n == 0:
            continue
        qg = qh[0, l, h * G:(h + 1) * G]
        want = h2o.attention_mass(qg, Kh[r, :n])
        np.testing.assert_allclose(a[r, :n] - a0[r, :n], want, rtol=MASS_RTOL, atol=MASS_ATOL * 10)
        np.testing.assert_allclose(a[r, :n], a0[r, :n] + want, rtol=MASS_RTOL, atol=MASS_ATOL)
        assert abs((a[r, :n] - a0[r, :n]).sum() - G) < 1e-4 + n * 2e-6      # each head's weights sum to 1
        for g in range(G):
            ref, ref_lse = o_decode.decode_head(qg[g], Kh[r, :n], Vh[r, :n])
            np.testing.assert_allclose(tl.f64(o)[0, l, h * G + g], ref, rtol=1e-2, atol=2e-2)
            assert abs(lse.cpu().numpy()[0, l, h * G + g] - ref_lse) < 1e-4 * max(1.0, abs(ref_lse))


def _oracle_cycles(w, inp, cycles, rec, final, sigma=1e3, lam=0.35):
    """Each row through the oracle's decode / eviction loop on its own state;
    compared with the recorded GPU cycles. Returns the number of rows whose
    later cycles were skipped after an allowed near-tie swap."""
    N, L, Hkv, Hq, d = w.n_seq, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim
    B, E, G = w.budget, w.interval, w.group
    vals = [0.0] + [o_policy.foresight_bonus(sigma, lam, s) for s in inp.steps_ahead]
    bonus = np.array(vals).reshape(-1, 1)
    floor = np.zeros_like(bonus, np.uint8)
    Kb, Vb = tl.bits(inp.K), tl.bits(inp.V)
    Knb, Vnb = tl.bits(inp.K_new), tl.bits(inp.V_new)
    qh = tl.f64(inp.q)
    pos0, acc0, tags0 = inp.pos.cpu().numpy(), inp.acc.cpu().numpy(), inp.tags.cpu().numpy()
    new_pos = int(pos0[:, B:].min())
    diverged = 0
    for r in range(w.rows):
        n, l, h = r // (L * Hkv), (r // Hkv) % L, r % Hkv
        K, V = Kb[r].copy(), Vb[r].copy()
        pos, acc, tags = pos0[r].astype(np.int64), acc0[r].astype(np.float64), tags0[r].astype(np.int64)
        same = True
        for c in range(cycles):
            K[B:], V[B:] = Knb[c, r], Vnb[c, r]
            pos[B:] = new_pos + c * E + np.arange(E)
            acc[B:] = 0.0
            tags[B:] = 0
            Kf = numfmt.bf16_bits_to_f64(K)
            for e in range(E):
                acc[:B + e + 1] = h2o.accumulate(acc[:B + e + 1], qh[c, e, n, l, h * G:(h + 1) * G], Kf[:B + e + 1])
            g = rec[c]
            np.testing.assert_array_equal(g["pos"][r], pos)
            np.testing.assert_array_equal(g["tags"][r], tags)
            np.testing.assert_allclose(g["acc"][r], acc, rtol=MASS_RTOL, atol=MASS_ATOL)
            kept = h2o.evict(acc, tags, bonus, floor, 0, w.n_sink, w.n_recent, B)
            tot, prot = o_policy.totals_and_protection(acc, tags, bonus, floor, 0, w.n_sink, w.n_recent)
            swaps = tl.check_kept(g["kept"][r], g["n_kept"][r], kept, tot, prot, B)
            K, V, pos, acc, tags = K[kept], V[kept], pos[kept], acc[kept], tags[kept]
            K = np.concatenate([K, np.zeros((E, d), np.uint16)])
            V = np.concatenate([V, np.zeros((E, d), np.uint16)])
            pos, acc, tags = (np.concatenate([pos, np.zeros(E, np.int64)]), np.concatenate([acc, np.zeros(E)]),
                              np.concatenate([tags, np.zeros(E, np.int64)]))
            if swaps:
                same = False
                diverged += 1
                break
        if same:
            np.testing.assert_array_equal(final["K"][r][:B], K[:B])        # positions kept: bit copies
            np.testing.assert_array_equal(final["V"][r][:B], V[:B])
            np.testing.assert_array_equal(final["pos"][r][:B], pos[:B])
            np.testing.assert_array_equal(final["tags"][r][:B], tags[:B])
            np.testing.assert_allclose(final["acc"][r][:B], acc[:B], rtol=MASS_RTOL, atol=MASS_ATOL)
            np.testing.assert_array_equal(final["Kr"][r][:B], K[:B])       # the store: each key at its own position
            np.testing.assert_array_equal(final["pr"][r][:B], pos[:B])
    return diverged


def _host(res):
    conv = lambda v: v if not torch.is_tensor(v) else (tl.bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy())  # noqa: E731
    rec = [{k: conv(v) for k, v in c.items()} for c in res["cycles"]]
    final = {k: (tl.bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in res["final"].items()}
    return rec, final


def test_h2o_small_cycles_match_oracle():
    from budgeted_retention_amd import pipelines
    w = synth.H2O_WORKLOADS["h2o_small"]
    cycles = 6
    inp = synth.make_h2o_inputs(w, cycles, "cuda")
    res = pipelines.run_h2o(w, inp, cycles, record=True)
    torch.cuda.synchronize()
    rec, final = _host(res)
    assert all((c["n_kept"] == w.budget).all() for c in rec)
    diverged = _oracle_cycles(w, inp, cycles, rec, final)
    assert diverged <= 1
    # the foresight spans outrank every cumulative score: all tagged slots stay resident
    for r in range(w.rows):
        assert (final["tags"][r][:w.budget] > 0).sum() == w.n_spans * w.span_slots


def test_pace_h2o_decode_shape_one_cycle_sampled_rows():
    """The 288-row resident cache (2048 + 32 slots, d = 128, G = 4): one cycle of
    32 decode steps and an eviction, in the configuration bench.py times;
    sampled rows against the oracle."""
    from budgeted_retention_amd import pipelines
    w = synth.H2O_WORKLOADS["pace_h2o_decode"]
    inp = synth.make_h2o_inputs(w, 1, "cuda")
    res = pipelines.run_h2o(w, inp, 1, record=True)
    torch.cuda.synchronize()
    rec, final = _host(res)
    assert (rec[0]["n_kept"] == w.budget).all()
    sample = [0, 137, w.rows - 1]
    sub = lambda a: a[sample] if isinstance(a, np.ndarray) and a.shape[0] == w.rows else a  # noqa: E731
    rec_s = [{k: sub(v) for k, v in c.items()} for c in rec]
    final_s = {k: sub(v) for k, v in final.items()}

    class _Rows:   # the sampled rows' inputs, as a small workload of len(sample) rows
        pass
    small = _Rows()
    idx = torch.tensor(sample, device="cuda")
    for k in ("K", "V", "pos", "acc", "tags"):
        setattr(small, k, getattr(inp, k).index_select(0, idx))
    small.K_new, small.V_new = inp.K_new.index_select(1, idx), inp.V_new.index_select(1, idx)
    # queries of the sampled rows' (layer, KV head) groups, laid out as rows of one layer
    G = w.group
    qs = []
    for r in sample:
        l, h = (r // w.n_kv_heads) % w.n_layers, r % w.n_kv_heads
        qs.append(inp.q[:, :, 0, l, h * G:(h + 1) * G])
    small.q = torch.stack(qs, dim=2).reshape(1, w.interval, 1, 1, len(sample) * G, w.head_dim)
    small.steps_ahead = inp.steps_ahead
    import dataclasses
    ws = dataclasses.replace(w, n_layers=1, n_kv_heads=len(sample), n_q_heads=len(sample) * G)
    assert _oracle_cycles(ws, small, 1, rec_s, final_s) == 0


def test_decode_h2o_counts_above_the_pool_are_clamped():
    from budgeted_retention_amd import kvc
    rows, S, d = 2, 300, 64
    dims = kvc.make_dims(1, 1, rows, 2 * rows, d, S)
    K = synth.normal_bf16((rows, S, d), 91, "cuda")
    V = synth.normal_bf16((rows, S, d), 92, "cuda")
    q = synth.normal_bf16((1, 1, 2 * rows, d), 93, "cuda")
    acc = torch.zeros((rows, S), dtype=torch.float32, device="cuda")
    n_h = torch.tensor([S + 77, S], dtype=torch.int32, device="cuda")
    o, lse, o2, lse2 = _h2o_call(dims, q, K, V, n_h, S, acc)
    a = acc.cpu().numpy()
    assert np.isfinite(a).all()
    for r in range(rows):
        want = h2o.attention_mass(tl.f64(q)[0, 0, 2 * r:2 * r + 2], tl.f64(K)[r])
        np.testing.assert_allclose(a[r], want, rtol=MASS_RTOL, atol=MASS_ATOL)


def _oracle_cycles_bounded(w, inp, cycles, rec, final, sigma=1e3, lam=0.35):
    """As _oracle_cycles with PACE's bounded positions: the oracle's own
    renumber decisions (oracle.positions), compaction with the reference store
    (oracle.compact.compact_row_ref). After a renumber the kernel's keys differ
    from the oracle's by one bf16 rounding, so later running scores are held
    to the workload bar and kept sets to swaps within 1e-2 relative; a row
    with a swap is not compared further. Returns (rows compared to the end,
    number of renumbers)."""
    from oracle import compact as o_compact, positions
    N, L, Hkv, Hq, d = w.n_seq, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim
    B, E, G = w.budget, w.interval, w.group
    vals = [0.0] + [o_policy.foresight_bonus(sigma, lam, s) for s in inp.steps_ahead]
    bonus = np.array(vals).reshape(-1, 1)
    floor = np.zeros_like(bonus, np.uint8)
    Kb, Vb = tl.bits(inp.K), tl.bits(inp.V)
    Knb, Vnb = tl.bits(inp.K_new), tl.bits(inp.V_new)
    qh = tl.f64(inp.q)
    pos0, acc0, tags0 = inp.pos.cpu().numpy(), inp.acc.cpu().numpy(), inp.tags.cpu().numpy()
    new_pos = int(pos0[:, B:].min())
    full, renumbers = 0, 0
    for r in range(w.rows):
        n, l, h = r // (L * Hkv), (r // Hkv) % L, r % Hkv
        K, V = Kb[r].copy(), Vb[r].copy()
        pos, acc, tags = pos0[r].astype(np.int64), acc0[r].astype(np.float64), tags0[r].astype(np.int64)
        Kref, pref = np.zeros_like(K), np.full(K.shape[0], -1, np.int64)
        shift, renumbered, ok = 0, False, True
        for c in range(cycles):
            g = rec[c]
            K[B:], V[B:] = Knb[c, r], Vnb[c, r]
            pos[B:] = new_pos + c * E - shift + np.arange(E)
            acc[B:], tags[B:], pref[B:] = 0.0, 0, -1
            Kf = numfmt.bf16_bits_to_f64(K)
            for e in range(E):
                acc[:B + e + 1] = h2o.accumulate(acc[:B + e + 1], qh[c, e, n, l, h * G:(h + 1) * G], Kf[:B + e + 1])
            np.testing.assert_array_equal(g["pos"][r], pos)
            assert pos.max() < w.limit
            if renumbered:
                np.testing.assert_allclose(g["acc"][r], acc, rtol=1e-2, atol=2e-2)
            else:
                np.testing.assert_allclose(g["acc"][r], acc, rtol=MASS_RTOL, atol=MASS_ATOL)
            kept = h2o.evict(acc, tags, bonus, floor, 0, w.n_sink, w.n_recent, B)
            gk = g["kept"][r][: g["n_kept"][r]].astype(np.int64)
            if not np.array_equal(gk, kept):
                tot, _ = o_policy.totals_and_protection(acc, tags, bonus, floor, 0, w.n_sink, w.n_recent)
                thr = tot[kept].min()
                diff = np.setxor1d(gk, kept)
                assert np.all(np.abs(tot[diff] - thr) <= (1e-2 if renumbered else 1e-3) * abs(thr))
                ok = False
                break
            ren, shift = positions.after_eviction(new_pos + (c + 1) * E, shift, B, w.limit, E)
            assert g["renumber"] == ren
            renumbers += int(ren and r == 0)
            K, V, pos, Kref, pref = o_compact.compact_row_ref(K, V, pos, kept, 0 if ren else -1, w.rope_base,
                                                             Kref, pref)
            acc, tags = acc[kept], tags[kept]
            renumbered |= ren
            pad = lambda a, v: np.concatenate([a, np.full((E,) + a.shape[1:], v, a.dtype)])  # noqa: E731
            K, V, Kref = pad(K, 0), pad(V, 0), pad(Kref, 0)
            pos, pref, acc, tags = pad(pos, 0), pad(pref, -1), pad(acc, 0.0), pad(tags, 0)
        if not ok:
            continue
        full += 1
        np.testing.assert_array_equal(final["pos"][r][:B], pos[:B])
        np.testing.assert_array_equal(final["pr"][r][:B], pref[:B])
        np.testing.assert_array_equal(final["Kr"][r][:B], Kref[:B])          # references are bit copies
        np.testing.assert_array_equal(final["V"][r][:B], V[:B])
        _close = numfmt.bf16_bits_to_f64
        a, b = _close(final["K"][r][:B]), _close(K[:B])
        np.testing.assert_allclose(a, b, rtol=1e-2, atol=2e-2)
    return full, renumbers


def test_h2o_small_bounded_positions_with_reference_store():
    """PACE's decode loop with H2O eviction, bounded positions (L = 128 here,
    headroom E) and renumbering through the reference store, against the
    oracle's own loop."""
    from budgeted_retention_amd import pipelines
    w = synth.H2O_WORKLOADS["h2o_small_bounded"]
    cycles = 10
    inp = synth.make_h2o_inputs(w, cycles, "cuda")
    res = pipelines.run_h2o(w, inp, cycles, record=True)
    torch.cuda.synchronize()
    rec, final = _host(res)
    assert sum(c["renumber"] for c in rec) >= 2                   # the limit was reached more than once
    assert all(c["pos"].max() < w.limit for c in rec)
    full, renumbers = _oracle_cycles_bounded(w, inp, cycles, rec, final)
    assert renumbers == sum(c["renumber"] for c in rec)
    assert full >= w.rows // 2, full
