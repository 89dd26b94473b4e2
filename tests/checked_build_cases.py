"""The calls the bounds-checked build is run on: every kernel family once on
valid seeded inputs (score, select in its short-row and candidate forms,
compaction, decode, pooling, page lists), then compaction, decode and page
scores given caller data that the kernels clamp (a kept index past the cache,
counts above their buffers, a block-table entry outside the storage, a page
span past the cache). Imported by the test with the default library; run as a
script in a child process with KVC_LIBRARY naming libkvc_check.so, it saves
the same outputs and the check bits read after each group of calls."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)

from budgeted_retention_amd import synth  # noqa: E402
import kvc_testlib as tl  # noqa: E402


def valid_calls(kvc):
    """Every kernel family on valid inputs; returns host arrays."""
    out = {}
    w = synth.WORKLOADS["tiny"]
    inp = synth.make_compaction_inputs(w, "cpu")
    K, V, Q = inp.K.cuda(), inp.V.cuda(), inp.Q_obs.cuda()
    N, L, Hkv, Hq, d, T, B = w.n_seq, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim, w.n_tokens, w.budget
    rows = N * L * Hkv
    pol = kvc.Policy(w.n_sink, w.n_recent, B, 1, 1, 0, L, None,
                     torch.zeros((1, 1), dtype=torch.float32, device="cuda"))
    res = tl.gpu_path((N, L, Hkv, Hq, d, T), K, V, Q, w.window, pol, w.renumber_base, w.rope_base)
    for k, v in res.items():
        out["path_" + k] = np.asarray(v)
    # decode over the compacted cache
    dims_b = kvc.make_dims(N, L, Hkv, Hq, d, B)
    Ko = torch.from_numpy(res["K"].view(np.int16)).view(torch.bfloat16).reshape(rows, B, d).cuda()
    Vo = torch.from_numpy(res["V"].view(np.int16)).view(torch.bfloat16).reshape(rows, B, d).cuda()
    o = torch.empty((N, L, Hq, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(1, kvc.kvc_decode_workspace_bytes(dims_b, B, 0)), dtype=torch.uint8, device="cuda")
    kvc.kvc_decode_attn(dims_b, inp.q_dec.cuda(), Ko, Vo, torch.from_numpy(res["n_h"]).cuda(), B, o, ws)
    out["decode_o"] = tl.bits(o)
    # score pooling (max, kernel 7) over the path's scores
    dims = kvc.make_dims(N, L, Hkv, Hq, d, T)
    sc = torch.from_numpy(res["scores"]).cuda().reshape(N, L, Hkv, T)
    pooled = torch.empty_like(sc)
    kvc.kvc_pool_scores(dims, sc, 7, kvc.KVC_POOL_MAX, pooled)
    out["pooled"] = pooled.cpu().numpy()
    # select over long rows (the candidate kernel) and short unaligned rows
    rng = np.random.default_rng(5)
    for name, T2, B2 in (("long", 20000, 1024), ("short", 6001, 700)):
        s2 = torch.from_numpy(rng.gamma(0.5, 1.0, (1, 2, 2, T2)).astype(np.float32)).cuda()
        d2 = kvc.make_dims(1, 2, 2, 4, 64, T2)
        p2 = kvc.Policy(4, 64, B2, 1, 1, 0, 2, None, torch.zeros((1, 1), dtype=torch.float32, device="cuda"))
        kept = torch.full((4, B2), -1, dtype=torch.int32, device="cuda")
        nk = torch.zeros(4, dtype=torch.int32, device="cuda")
        kvc.kvc_select(d2, s2, p2, kept, B2, nk)
        out[f"select_{name}_kept"] = kept.cpu().numpy()
        out[f"select_{name}_n"] = nk.cpu().numpy()
    # page list -> token list (uniform pages of 16, a ragged last page)
    Tp, G = 1000, 16
    n_pages = (Tp + G - 1) // G
    pages = torch.from_numpy(np.stack([rng.permutation(n_pages)[:20] for _ in range(2)]).astype(np.int32)).cuda()
    n_listed = torch.tensor([20, 13], dtype=torch.int32, device="cuda")
    tokens = torch.full((2, 20 * G), -1, dtype=torch.int32, device="cuda")
    n_tok = torch.zeros(2, dtype=torch.int32, device="cuda")
    kvc.kvc_page_tokens(kvc.make_dims(2, 1, 1, 1, 64, Tp), G, n_pages, pages, n_listed, tokens, n_tok)
    out["page_tokens"] = tokens.cpu().numpy()
    out["page_n"] = n_tok.cpu().numpy()
    torch.cuda.synchronize()
    return out


def clamped_calls(kvc):
    """Caller data the kernels clamp: one kept list holds an index past the
    cache and a count above its stride; one decode count exceeds its pool; a
    block-table entry points outside the storage; a page span runs past the
    cache."""
    out = {}
    rng = np.random.default_rng(6)
    N, L, Hkv, Hq, d, T, ks = 1, 1, 2, 4, 64, 300, 40
    rows = N * L * Hkv
    K, V, _ = synth.small_case(T, Hkv, Hq, d, 4, L, N, seed=6)
    K, V = K.cuda(), V.cuda()
    dims = kvc.make_dims(N, L, Hkv, Hq, d, T)
    kept = np.stack([np.sort(rng.choice(T, ks, replace=False)) for _ in range(rows)]).astype(np.int32)
    kept[0, 7] = T + 5                  # past the cache: skipped
    n_kept = np.array([ks, ks + 3], np.int32)   # row 1: above the stride, read as ks
    Ko = torch.zeros((rows, ks, d), dtype=torch.bfloat16, device="cuda")
    Vo = torch.zeros_like(Ko)
    po = torch.full((rows, ks), -1, dtype=torch.int32, device="cuda")
    nh = torch.zeros(rows, dtype=torch.int32, device="cuda")
    kvc.kvc_compact_rerotate(dims, K, V, None, torch.from_numpy(kept).cuda(), ks, torch.from_numpy(n_kept).cuda(),
                             0, 1e4, kvc.CompactOut(ks, Ko, Vo, po, nh))
    out["cmp_K"], out["cmp_V"] = tl.bits(Ko), tl.bits(Vo)
    out["cmp_pos"], out["cmp_n"] = po.cpu().numpy(), nh.cpu().numpy()
    # decode with a row count above its pool: read as the pool size
    q = torch.from_numpy(rng.standard_normal((N, L, Hq, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    n_h = torch.tensor([ks, ks + 9], dtype=torch.int32, device="cuda")
    o = torch.empty((N, L, Hq, d), dtype=torch.bfloat16, device="cuda")
    dims_b = kvc.make_dims(N, L, Hkv, Hq, d, ks)
    ws = torch.empty(max(1, kvc.kvc_decode_workspace_bytes(dims_b, ks, 0)), dtype=torch.uint8, device="cuda")
    Kf = torch.from_numpy(out["cmp_K"].view(np.int16)).view(torch.bfloat16).reshape(rows, ks, d).cuda()
    Vf = torch.from_numpy(out["cmp_V"].view(np.int16)).view(torch.bfloat16).reshape(rows, ks, d).cuda()
    kvc.kvc_decode_attn(dims_b, q, Kf, Vf, n_h, ks, o, ws)
    out["dec_o"] = tl.bits(o)
    # paged decode whose block table points one used page outside the storage
    # (that page's tokens are skipped)
    ps, bps = 8, 5
    tbl = torch.tensor([[0, 2, 1, 4, 3]], dtype=torch.int32, device="cuda")
    tbl[0, 2] = -1
    n_p = torch.tensor([bps * ps - 3, bps * ps - 3], dtype=torch.int32, device="cuda")
    o2 = torch.empty_like(o)
    dims_p = kvc.make_dims(N, L, Hkv, Hq, d, ks)
    ws2 = torch.empty(max(1, kvc.kvc_decode_workspace_bytes(dims_p, bps * ps, 0)), dtype=torch.uint8, device="cuda")
    kvc.kvc_decode_attn(dims_p, q, Kf, Vf, n_p, ks, o2, ws2, block_table=tbl, page_size=ps, blocks_per_seq=bps)
    out["dec_paged_o"] = tl.bits(o2)
    # page scores over event pages, one span running past the cache (clamped)
    sc = torch.from_numpy(rng.gamma(0.5, 1.0, (N, L, Hkv, T)).astype(np.float32)).cuda()
    first = torch.tensor([[0, 16, 40, T - 10]], dtype=torch.int32, device="cuda")
    length = torch.tensor([[16, 16, 12, 16]], dtype=torch.int32, device="cuda")
    pscore = torch.empty((N, 4), dtype=torch.float32, device="cuda")
    kvc.kvc_page_scores(dims, sc, 16, 4, pscore, page_first=first, page_len=length)
    out["page_scores"] = pscore.cpu().numpy()
    torch.cuda.synchronize()
    return out


def main(path):
    from budgeted_retention_amd import _lib, kvc
    assert os.path.basename(_lib.LIB_PATH) == "libkvc_check.so", _lib.LIB_PATH
    _lib.load()
    print("checked build: valid calls", flush=True)
    kvc.kvc_check_read()                # nothing is pending in a new process; clears the words
    out = valid_calls(kvc)
    out["bits_valid"] = np.uint32(kvc.kvc_check_read())
    print("checked build: clamped calls", flush=True)
    out.update(clamped_calls(kvc))
    out["bits_clamped"] = np.uint32(kvc.kvc_check_read())
    out["bits_after_read"] = np.uint32(kvc.kvc_check_read())
    np.savez(path, **out)
    print("checked build: done", flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
