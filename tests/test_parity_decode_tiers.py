"""GPU parity: kvc_decode_attn (bf16 pool, int8 or INT4 pool, paged layout)
and the low-precision/bf16/release tiers of kvc_compact_rerotate, against the
float64 oracle. INT4 codes (PASK Appendix B.5: two signed nibbles per byte)
are packed by the oracle where a test needs them as input."""
import numpy as np
import pytest
import torch

from budgeted_retention_amd import synth
from oracle import compact as o_compact, decode as o_decode, numfmt, quant as o_quant
import kvc_testlib as tl

pytestmark = pytest.mark.gpu


def _gpu_decode(dims_t, p, stride_h, stride_l=0, block_table=None, page_size=0, bps=0, low_bits=8):
    from budgeted_retention_amd import kvc
    N, L, Hkv, Hq, d = dims_t
    dims = kvc.make_dims(N, L, Hkv, Hq, d, stride_h)
    max_h = bps * page_size if block_table is not None else stride_h
    ws = torch.empty(max(1, kvc.kvc_decode_workspace_bytes(dims, max_h, stride_l)), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((N, L, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((N, L, Hq), dtype=torch.float32, device="cuda")
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    kvc.kvc_decode_attn(dims, c["q"], c["K"], c["V"], c["n_h"], stride_h, o, ws, lse,
                        None if block_table is None else block_table.cuda(), page_size, bps,
                        c.get("Kq"), c.get("Vq"), c.get("Ks"), c.get("Vs"), c.get("n_l"), stride_l, low_bits)
    torch.cuda.synchronize()
    return tl.f64(o), lse.cpu().numpy().astype(np.float64)


def _check_decode(g_o, g_lse, q, parts_per_row, dims_t):
    N, L, Hkv, Hq, d = dims_t
    G = Hq // Hkv
    for n in range(N):
        for l in range(L):
            for hq in range(Hq):
                r = (n * L + l) * Hkv + hq // G
                parts = parts_per_row[r]
                if sum(len(k) for k, _ in parts) == 0:
                    assert np.all(g_o[n, l, hq] == 0) and g_lse[n, l, hq] == -np.inf
                    continue
                o, lse = o_decode.decode_partitions(q[n, l, hq], parts)
                ob = numfmt.round_bf16(o)
                np.testing.assert_allclose(g_o[n, l, hq], ob, rtol=1e-2, atol=2e-2)   # the bar
                np.testing.assert_allclose(g_o[n, l, hq], o, rtol=8e-3, atol=1e-3)    # fp32 path
                assert g_lse[n, l, hq] == pytest.approx(lse, rel=1e-5, abs=1e-5)


@pytest.mark.parametrize("d,Hkv,Hq,stride", [(128, 2, 8, 700), (64, 1, 2, 300), (128, 4, 28, 513)])
def test_decode_bf16_pool(d, Hkv, Hq, stride):
    dims_t = (2, 2, Hkv, Hq, d)
    p = synth.decode_pools(*dims_t, stride, seed=d + stride)
    g_o, g_lse = _gpu_decode(dims_t, p, stride)
    K, V, n_h = tl.f64(p["K"]), tl.f64(p["V"]), p["n_h"].numpy()
    parts = [[(K[r, : n_h[r]], V[r, : n_h[r]])] for r in range(K.shape[0])]
    _check_decode(g_o, g_lse, tl.f64(p["q"]), parts, dims_t)


@pytest.mark.parametrize("d", [128, 64])
def test_decode_with_int8_partition(d):
    dims_t = (2, 3, 2, 8, d)
    p = synth.decode_pools(*dims_t, 400, stride_l=300, seed=3 + d)
    g_o, g_lse = _gpu_decode(dims_t, p, 400, stride_l=300)
    K, V, n_h = tl.f64(p["K"]), tl.f64(p["V"]), p["n_h"].numpy()
    n_l = p["n_l"].numpy()
    Kq, Vq = p["Kq"].numpy(), p["Vq"].numpy()
    Ks, Vs = p["Ks"].numpy().view(np.uint16), p["Vs"].numpy().view(np.uint16)
    parts = []
    for r in range(K.shape[0]):
        kl = o_quant.dequantize_rows(Kq[r, : n_l[r]], Ks[r, : n_l[r]])
        vl = o_quant.dequantize_rows(Vq[r, : n_l[r]], Vs[r, : n_l[r]])
        parts.append([(K[r, : n_h[r]], V[r, : n_h[r]]), (kl, vl)])
    _check_decode(g_o, g_lse, tl.f64(p["q"]), parts, dims_t)


@pytest.mark.parametrize("d", [128, 64])
def test_decode_with_int4_partition(d):
    dims_t = (2, 3, 2, 8, d)
    p = synth.decode_pools(*dims_t, 400, stride_l=300, seed=5 + d)
    rows = 2 * 3 * 2
    rng = np.random.default_rng(d)
    codes = rng.integers(-7, 8, (2, rows, 300, d))
    p["Kq"] = torch.from_numpy(o_quant.pack_nibbles(codes[0]).view(np.int8))
    p["Vq"] = torch.from_numpy(o_quant.pack_nibbles(codes[1]).view(np.int8))
    g_o, g_lse = _gpu_decode(dims_t, p, 400, stride_l=300, low_bits=4)
    K, V, n_h = tl.f64(p["K"]), tl.f64(p["V"]), p["n_h"].numpy()
    n_l = p["n_l"].numpy()
    Ks, Vs = p["Ks"].numpy().view(np.uint16), p["Vs"].numpy().view(np.uint16)
    parts = []
    for r in range(rows):
        kl = o_quant.dequantize_rows(codes[0, r, : n_l[r]], Ks[r, : n_l[r]])
        vl = o_quant.dequantize_rows(codes[1, r, : n_l[r]], Vs[r, : n_l[r]])
        parts.append([(K[r, : n_h[r]], V[r, : n_h[r]]), (kl, vl)])
    _check_decode(g_o, g_lse, tl.f64(p["q"]), parts, dims_t)


def test_decode_paged_layout():
    N, L, Hkv, Hq, d, ps = 3, 2, 2, 8, 128, 16
    T_store, bps = 1024, 25                       # 64 stored pages, 25 referenced per sequence
    dims_t = (N, L, Hkv, Hq, d)
    p = synth.decode_pools(*dims_t, T_store, seed=21)
    rows = N * L * Hkv
    p["n_h"] = torch.full((rows,), bps * ps - 7, dtype=torch.int32)     # ragged last page
    tbl = synth.page_table(N, T_store // ps, bps)
    g_o, g_lse = _gpu_decode(dims_t, p, T_store, block_table=tbl, page_size=ps, bps=bps)
    K, V = tl.f64(p["K"]), tl.f64(p["V"])
    parts = []
    for r in range(rows):
        n = r // (L * Hkv)
        t = np.arange(bps * ps - 7)
        slot = tbl[n].numpy()[t // ps] * ps + t % ps
        parts.append([(K[r, slot], V[r, slot])])
    _check_decode(g_o, g_lse, tl.f64(p["q"]), parts, dims_t)


@pytest.mark.parametrize("renumber_base,d,low_bits", [(-1, 128, 8), (0, 128, 8), (100, 64, 8),
                                                     (-1, 128, 4), (0, 64, 4)])
def test_tiered_compaction(renumber_base, d, low_bits):
    from budgeted_retention_amd import kvc
    N, L, Hkv, Hq, T, n_keep = 1, 2, 2, 8, 2000, 700
    rows = N * L * Hkv
    K, V, _ = synth.small_case(T, Hkv, Hq, d, 8, L, N, seed=40 + d)
    kept, n, act = synth.kept_and_actions(rows, T, n_keep)
    pos = np.tile(np.arange(T, dtype=np.int32) * 3 + 5, (rows, 1))      # non-trivial positions
    dims = kvc.make_dims(N, L, Hkv, Hq, d, T)
    cap = n_keep
    dev = "cuda"
    Ko = torch.zeros((rows, cap, d), dtype=torch.bfloat16, device=dev)
    Vo = torch.zeros_like(Ko)
    cb = d if low_bits == 8 else d // 2
    qmax = 127 if low_bits == 8 else 7
    Kq = torch.zeros((rows, cap, cb), dtype=torch.int8, device=dev)
    Vq = torch.zeros_like(Kq)
    Ks = torch.zeros((rows, cap), dtype=torch.int16, device=dev)
    Vs = torch.zeros_like(Ks)
    po = torch.full((rows, cap), -1, dtype=torch.int32, device=dev)
    pq = torch.full((rows, cap), -1, dtype=torch.int32, device=dev)
    nh = torch.zeros(rows, dtype=torch.int32, device=dev)
    nl = torch.zeros(rows, dtype=torch.int32, device=dev)
    out = kvc.CompactOut(cap, Ko, Vo, po, nh, torch.from_numpy(act).to(dev), Kq, Vq, Ks, Vs, pq, nl,
                         low_bits=low_bits)
    kvc.kvc_compact_rerotate(dims, K.to(dev), V.to(dev), torch.from_numpy(pos).to(dev),
                             torch.from_numpy(kept).to(dev), n_keep, torch.from_numpy(n).to(dev),
                             renumber_base, 1e4, out)
    torch.cuda.synchronize()
    Kb, Vb = tl.bits(K).reshape(rows, T, d), tl.bits(V).reshape(rows, T, d)
    unpack = (lambda x: x.astype(np.int8)) if low_bits == 8 else (lambda x: o_quant.unpack_nibbles(x.view(np.uint8), d))
    for r in range(rows):
        k = kept[r, : n[r]].astype(np.int64)
        a = act[r, : n[r]]
        oK, oV, op = o_compact.compact_row(Kb[r], Vb[r], pos[r], k, renumber_base, 1e4)
        H, Lw = np.flatnonzero(a == 2), np.flatnonzero(a == 1)
        assert nh[r].item() == H.size and nl[r].item() == Lw.size
        gK = tl.bits(Ko[r])[: H.size]
        np.testing.assert_array_equal(tl.bits(Vo[r])[: H.size], oV[H])
        np.testing.assert_array_equal(po[r].cpu().numpy()[: H.size], op[H])
        np.testing.assert_allclose(numfmt.bf16_bits_to_f64(gK), numfmt.bf16_bits_to_f64(oK[H]),
                                   rtol=1e-2, atol=2e-2)
        if renumber_base < 0:
            np.testing.assert_array_equal(gK, oK[H])
        # low tier: codes within +-1 and fp16 scales of the oracle's quantisation of
        # the same (re-rotated) bf16 key and the value
        if renumber_base < 0:
            ck, sk = o_quant.quantize_rows(numfmt.bf16_bits_to_f64(oK[Lw]), qmax)
            gck = unpack(Kq[r].cpu().numpy()[: Lw.size])
            assert np.abs(gck.astype(int) - ck.astype(int)).max() <= 1
            assert np.abs(gck).max() <= qmax
            np.testing.assert_array_equal(Ks[r].cpu().numpy().view(np.uint16)[: Lw.size], sk)
        cv, sv = o_quant.quantize_rows(numfmt.bf16_bits_to_f64(oV[Lw]), qmax)
        gcv = unpack(Vq[r].cpu().numpy()[: Lw.size])
        assert np.abs(gcv.astype(int) - cv.astype(int)).max() <= 1
        np.testing.assert_array_equal(Vs[r].cpu().numpy().view(np.uint16)[: Lw.size], sv)
        np.testing.assert_array_equal(pq[r].cpu().numpy()[: Lw.size], op[Lw])


@pytest.mark.parametrize("low_bits", [8, 4])
def test_tiered_compaction_zero_and_tiny_rows(low_bits):
    """PASK Appendix B.5 edge cases: an all-zero row gets zero codes and unit
    scale; a row whose largest magnitude is tiny gets the smallest positive
    fp16 scale (2^-24) and codes clipped to the range."""
    from budgeted_retention_amd import kvc
    rows, T, d = 2, 64, 128
    rng = np.random.default_rng(low_bits)
    K = rng.standard_normal((rows, T, d))
    V = rng.standard_normal((rows, T, d))
    K[:, 5], V[:, 5] = 0.0, 0.0                     # zero rows
    K[:, 9], V[:, 9] = 1e-9, -3e-9                  # far below 2^-24 * qmax
    Kb, Vb = numfmt.f64_to_bf16_bits(K), numfmt.f64_to_bf16_bits(V)
    kept = np.tile(np.arange(16, dtype=np.int32), (rows, 1))
    n = np.full(rows, 16, np.int32)
    act = np.ones((rows, 16), np.uint8)             # everything to the low tier
    dims = kvc.make_dims(1, 1, rows, rows, d, T)
    cb, qmax = (d, 127) if low_bits == 8 else (d // 2, 7)
    dev = "cuda"
    Ko = torch.zeros((rows, 16, d), dtype=torch.bfloat16, device=dev)
    Kq = torch.zeros((rows, 16, cb), dtype=torch.int8, device=dev)
    Vq = torch.zeros_like(Kq)
    Ks = torch.zeros((rows, 16), dtype=torch.int16, device=dev)
    Vs = torch.zeros_like(Ks)
    nh = torch.zeros(rows, dtype=torch.int32, device=dev)
    nl = torch.zeros(rows, dtype=torch.int32, device=dev)
    out = kvc.CompactOut(16, Ko, torch.zeros_like(Ko), None, nh, torch.from_numpy(act).to(dev), Kq, Vq, Ks, Vs,
                         None, nl, low_bits=low_bits)
    kvc.kvc_compact_rerotate(dims, torch.from_numpy(Kb.view(np.int16)).view(torch.bfloat16).to(dev),
                             torch.from_numpy(Vb.view(np.int16)).view(torch.bfloat16).to(dev), None,
                             torch.from_numpy(kept).to(dev), 16, torch.from_numpy(n).to(dev), -1, 1e4, out)
    torch.cuda.synchronize()
    unpack = (lambda x: x.astype(np.int8)) if low_bits == 8 else (lambda x: o_quant.unpack_nibbles(x.view(np.uint8), d))
    for r in range(rows):
        assert nl[r].item() == 16 and nh[r].item() == 0
        for X, q, sc in ((Kb, Kq, Ks), (Vb, Vq, Vs)):
            want_c, want_s = o_quant.quantize_rows(numfmt.bf16_bits_to_f64(X[r, :16]), qmax)
            got_c = unpack(q[r].cpu().numpy())
            got_s = sc[r].cpu().numpy().view(np.uint16)
            np.testing.assert_array_equal(got_s, want_s)
            assert np.abs(got_c.astype(int) - want_c.astype(int)).max() <= 1
            assert got_s[5] == 0x3C00 and not got_c[5].any()
            assert got_s[9] == 1 and np.abs(got_c[9]).max() <= qmax


def test_decode_full_session_shape_sampled_rows():
    """The decode launch bench.py times: 36 layers x 8 KV heads (G = 4, d 128),
    every row holding B = 2048 resident keys; the 4 query heads of sampled rows
    against the oracle."""
    dims_t = (1, 36, 8, 32, 128)
    B = 2048
    p = synth.decode_pools(*dims_t, B, seed=2048, device="cuda")
    p["n_h"].fill_(B)
    g_o, g_lse = _gpu_decode(dims_t, p, B)
    L, Hkv, G = 36, 8, 4
    for r in (0, 1, 143, L * Hkv - 1):
        l, h = r // Hkv, r % Hkv
        K, V = tl.f64(p["K"][r]), tl.f64(p["V"][r])
        for g in range(G):
            hq = h * G + g
            o, lse = o_decode.decode_partitions(tl.f64(p["q"][0, l, hq]), [(K, V)])
            np.testing.assert_allclose(g_o[0, l, hq], numfmt.round_bf16(o), rtol=1e-2, atol=2e-2)   # the bar
            np.testing.assert_allclose(g_o[0, l, hq], o, rtol=8e-3, atol=1e-3)                      # fp32 path
            assert g_lse[0, l, hq] == pytest.approx(lse, rel=1e-5, abs=1e-5)
