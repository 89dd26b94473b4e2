"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before enqueueing anything (these
calls return before any HIP runtime call, so no GPU is needed)."""
import ctypes
import glob
import os
import re

import pytest

from budgeted_retention_amd import _lib
from oracle import policy as o_policy

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(kvc_[a-z0-9_]+)\s*\(", text):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    declared = _declared_functions()
    assert {"kvc_score", "kvc_select", "kvc_compact_rerotate"} <= declared
    missing = [n for n in sorted(declared) if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding knows a prototype for each
    assert declared <= set(_lib.PROTOTYPES), declared - set(_lib.PROTOTYPES)


def test_version_and_helpers_match_oracle():
    lib = _lib.load()
    assert lib.kvc_version() >= 100
    for L, n in [(36, 3), (40, 3), (32, 3), (32, 4), (28, 1), (7, 5)]:
        for l in range(L):
            assert lib.kvc_layer_group(l, L, n) == o_policy.layer_group(l, L, n)
    assert lib.kvc_layer_group(5, 4, 2) == -1
    for k in [0, 1, 3, 7, 50]:
        assert lib.kvc_foresight_bonus(1e3, 0.35, k) == pytest.approx(
            o_policy.foresight_bonus(1e3, 0.35, k), rel=1e-14)


def _dims(**kw):
    d = dict(n_seq=1, n_layers=1, n_kv_heads=2, n_q_heads=8, head_dim=64, n_tokens=4096)
    d.update(kw)
    return _lib.KvcDims(d["n_seq"], d["n_layers"], d["n_kv_heads"], d["n_q_heads"],
                        d["head_dim"], 0, d["n_tokens"])


FAKE = 0x1000   # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), _lib.KVC_ERR_UNSUPPORTED),
    (dict(n_q_heads=7), _lib.KVC_ERR_ARG),
    (dict(n_tokens=0), _lib.KVC_ERR_ARG),
    (dict(n_seq=-1), _lib.KVC_ERR_ARG),
])
def test_score_rejects_bad_dims(kw, code):
    lib = _lib.load()
    d = _dims(**kw)
    st = lib.kvc_score(ctypes.byref(d), FAKE, FAKE, 16, FAKE, FAKE, 1 << 30, None)
    assert st == code
    assert lib.kvc_last_error().decode().startswith("kvc_score")


def test_score_rejects_window_workspace_and_nulls():
    lib = _lib.load()
    d = _dims()
    ws = lib.kvc_workspace_bytes(_lib.KVC_OP_SCORE, ctypes.byref(d), 16, 0)
    assert ws > 0
    assert lib.kvc_score(ctypes.byref(d), FAKE, FAKE, 0, FAKE, FAKE, ws, None) == _lib.KVC_ERR_ARG
    assert lib.kvc_score(ctypes.byref(d), FAKE, FAKE, 4097, FAKE, FAKE, ws, None) == _lib.KVC_ERR_ARG
    assert lib.kvc_score(ctypes.byref(d), FAKE, FAKE, 16, FAKE, FAKE, ws - 1, None) == _lib.KVC_ERR_WORKSPACE
    assert lib.kvc_score(ctypes.byref(d), FAKE, FAKE, 16, FAKE, None, ws, None) == _lib.KVC_ERR_WORKSPACE
    assert lib.kvc_score(ctypes.byref(d), None, FAKE, 16, FAKE, FAKE, ws, None) == _lib.KVC_ERR_ARG
    d2 = _dims(n_q_heads=64, n_kv_heads=2)     # G = 32, W*G = 512 > 256
    ws2 = lib.kvc_workspace_bytes(_lib.KVC_OP_SCORE, ctypes.byref(d2), 16, 0)
    assert lib.kvc_score(ctypes.byref(d2), FAKE, FAKE, 16, FAKE, FAKE, ws2, None) == _lib.KVC_ERR_UNSUPPORTED
    assert lib.kvc_workspace_bytes(99, ctypes.byref(d), 16, 0) == 0


def _policy(**kw):
    p = dict(n_sink=4, n_recent=64, budget=512, n_tags=1, n_groups=1, layer_base=0, n_layers_model=1)
    p.update(kw)
    return _lib.KvcPolicy(p["n_sink"], p["n_recent"], p["budget"], p["n_tags"], p["n_groups"],
                          p["layer_base"], p["n_layers_model"], 0, None, None, None)


@pytest.mark.parametrize("kw", [
    dict(budget=0), dict(n_sink=-1), dict(n_tags=0), dict(n_tags=300), dict(n_groups=0),
    dict(layer_base=1), dict(n_layers_model=0),
])
def test_select_rejects_bad_policy(kw):
    lib = _lib.load()
    d = _dims()
    p = _policy(**kw)
    assert lib.kvc_select(ctypes.byref(d), FAKE, ctypes.byref(p), FAKE, 512, FAKE, None, 0, None) == _lib.KVC_ERR_ARG


def test_select_rejects_small_kept_stride():
    lib = _lib.load()
    d = _dims()
    p = _policy()
    assert lib.kvc_select(ctypes.byref(d), FAKE, ctypes.byref(p), FAKE, 511, FAKE, None, 0, None) == _lib.KVC_ERR_ARG


def test_select_with_a_floor_table_needs_a_full_length_list():
    # PASK §3.5: floors take precedence over the budget, so a floor table can
    # make any token protected; the kept list must then hold all T entries.
    lib = _lib.load()
    d = _dims()
    p = _policy()
    p.tag_floor = FAKE
    assert lib.kvc_select(ctypes.byref(d), FAKE, ctypes.byref(p), FAKE, 512, FAKE, None, 0, None) == _lib.KVC_ERR_ARG
    assert lib.kvc_select(ctypes.byref(d), FAKE, ctypes.byref(p), FAKE, 4095, FAKE, None, 0, None) == _lib.KVC_ERR_ARG
    # T <= budget keeps every token: the usual min(budget, T) suffices
    d = _dims(n_tokens=300)
    p.budget = 300
    assert lib.kvc_select(ctypes.byref(d), FAKE, ctypes.byref(p), FAKE, 299, FAKE, None, 0, None) == _lib.KVC_ERR_ARG


def test_compact_rejects_bad_outputs():
    lib = _lib.load()
    d = _dims()
    out = _lib.KvcCompactOut()
    out.out_stride = 512
    st = lib.kvc_compact_rerotate(ctypes.byref(d), FAKE, FAKE, None, FAKE, 512, FAKE, 0, 1e4,
                                  ctypes.byref(out), None)
    assert st == _lib.KVC_ERR_ARG                                # K_out / V_out missing
    out.K_out = out.V_out = FAKE
    st = lib.kvc_compact_rerotate(ctypes.byref(d), FAKE, FAKE, None, FAKE, 512, FAKE, 0, 1.0,
                                  ctypes.byref(out), None)
    assert st == _lib.KVC_ERR_ARG                                # rope base must exceed 1
    out.action = FAKE
    st = lib.kvc_compact_rerotate(ctypes.byref(d), FAKE, FAKE, None, FAKE, 512, FAKE, -1, 1e4,
                                  ctypes.byref(out), None)
    assert st == _lib.KVC_ERR_ARG                                # int8 pools missing
    out.action = None
    out.out_stride = 0
    st = lib.kvc_compact_rerotate(ctypes.byref(d), FAKE, FAKE, None, FAKE, 512, FAKE, -1, 1e4,
                                  ctypes.byref(out), None)
    assert st == _lib.KVC_ERR_ARG


def test_decode_rejects_bad_arguments():
    lib = _lib.load()
    d = _dims()
    ws = lib.kvc_decode_workspace_bytes(ctypes.byref(d), 512, 0)
    assert ws > 0
    call = lambda **k: lib.kvc_decode_attn(
        ctypes.byref(k.get("dims", d)), FAKE, FAKE, FAKE, FAKE, k.get("stride_h", 512),
        k.get("bt", None), k.get("ps", 0), k.get("bps", 0), k.get("Kq"), k.get("Vq"), k.get("Ks"), k.get("Vs"),
        k.get("n_l", None), k.get("stride_l", 0), k.get("bits", 8), FAKE, None, FAKE, k.get("ws", ws), None)
    assert call(stride_h=0) == _lib.KVC_ERR_ARG
    assert call(ws=ws - 1) == _lib.KVC_ERR_WORKSPACE
    assert call(bt=FAKE, ps=0, bps=4) == _lib.KVC_ERR_ARG            # paged needs a page size
    assert call(n_l=FAKE, stride_l=64) == _lib.KVC_ERR_ARG            # int8 pools missing
    assert call(n_l=FAKE, stride_l=64, Kq=FAKE, Vq=FAKE, Ks=FAKE, Vs=FAKE, bits=2) == _lib.KVC_ERR_UNSUPPORTED
    big = _dims(n_q_heads=64, n_kv_heads=2)                             # G = 32 > 16
    assert call(dims=big, ws=1 << 40) == _lib.KVC_ERR_UNSUPPORTED


def test_compact_page_lists_reject_actions_and_negative_page():
    lib = _lib.load()
    d = _dims()
    out = _lib.KvcCompactOut()
    out.out_stride = 512
    out.K_out = out.V_out = FAKE
    out.kept_page = -1
    st = lib.kvc_compact_rerotate(ctypes.byref(d), FAKE, FAKE, None, FAKE, 32, FAKE, -1, 1e4,
                                  ctypes.byref(out), None)
    assert st == _lib.KVC_ERR_ARG
    out.kept_page = 16
    out.action = FAKE
    out.Kq = out.Vq = out.Ks = out.Vs = FAKE
    st = lib.kvc_compact_rerotate(ctypes.byref(d), FAKE, FAKE, None, FAKE, 32, FAKE, -1, 1e4,
                                  ctypes.byref(out), None)
    assert st == _lib.KVC_ERR_UNSUPPORTED                        # shared page lists are bf16 only
    out.action = None
    out.kept_page = 1 << 20
    st = lib.kvc_compact_rerotate(ctypes.byref(d), FAKE, FAKE, None, FAKE, 1 << 12, FAKE, -1, 1e4,
                                  ctypes.byref(out), None)
    assert st == _lib.KVC_ERR_ARG                                # listed tokens overflow int32


def test_page_scores_reject_bad_arguments():
    lib = _lib.load()
    d = _dims(n_tokens=1000)
    call = lambda ps=16, n=62, order=None, acc=None, n_cand=0, sc=FAKE, pf=None, pl=None: lib.kvc_page_scores(
        ctypes.byref(d), sc, ps, pf, pl, n, order, acc, n_cand, FAKE, None)
    assert call(sc=None) == _lib.KVC_ERR_ARG
    assert call(ps=0) == _lib.KVC_ERR_UNSUPPORTED
    assert call(ps=2048) == _lib.KVC_ERR_UNSUPPORTED
    assert call(n=63) == _lib.KVC_ERR_ARG                        # 63 * 16 > 1000 tokens
    assert call(order=FAKE) == _lib.KVC_ERR_ARG                  # order without accepted
    assert call(order=FAKE, acc=FAKE, n_cand=0) == _lib.KVC_ERR_ARG
    assert lib.kvc_last_error().decode().startswith("kvc_page_scores")
    assert call(pf=FAKE) == _lib.KVC_ERR_ARG                     # event pages need both arrays
    assert call(pl=FAKE) == _lib.KVC_ERR_ARG
    assert call(pf=FAKE, pl=FAKE, n=0) == _lib.KVC_ERR_ARG


def test_event_page_arguments_are_checked_before_any_launch():
    lib = _lib.load()
    d = _dims(n_tokens=1000)
    eff = lambda ps=16, pf=FAKE, pl=FAKE, n=70: lib.kvc_page_effect(
        ctypes.byref(d), 0, FAKE, FAKE, FAKE, 8, 992, ps, pf, pl, n, FAKE, None, FAKE, 1, None)
    assert eff(pl=None) == _lib.KVC_ERR_ARG
    assert eff(pf=None) == _lib.KVC_ERR_ARG
    assert eff(ps=65) == _lib.KVC_ERR_UNSUPPORTED                # an event page must fit a 64-key tile
    assert eff(ps=0) == _lib.KVC_ERR_UNSUPPORTED
    assert eff(n=0) == _lib.KVC_ERR_ARG
    assert eff(ps=24) == _lib.KVC_ERR_WORKSPACE                  # any length up to 64 passes the page checks
    assert eff(ps=24, pf=None, pl=None) == _lib.KVC_ERR_UNSUPPORTED  # uniform pages must divide 64
    ret = lambda ps=16: lib.kvc_page_retire(ctypes.byref(d), 0, FAKE, FAKE, FAKE, 8, 992, ps, FAKE, FAKE, 70,
                                            FAKE, 4, ctypes.c_float(0.1), FAKE, None, FAKE, 1, None)
    assert ret(ps=17) == _lib.KVC_ERR_UNSUPPORTED               # retire takes pages of up to 16 tokens
    tok = lambda ps=16, pf=FAKE, pl=FAKE, pages=FAKE, ls=8, os_=64: lib.kvc_page_tokens(
        ctypes.byref(d), ps, pf, pl, 70, pages, FAKE, ls, FAKE, FAKE, os_, None)
    assert tok(pl=None) == _lib.KVC_ERR_ARG
    assert tok(pages=None) == _lib.KVC_ERR_ARG
    assert tok(ps=0) == _lib.KVC_ERR_ARG
    assert tok(ls=0) == _lib.KVC_ERR_ARG
    assert tok(os_=0) == _lib.KVC_ERR_ARG
    assert lib.kvc_last_error().decode().startswith("kvc_page_tokens")
    sel = lambda ps=16, pf=FAKE, pl=FAKE, n=70, b=512, ks=64, kept=FAKE: lib.kvc_page_select(
        ctypes.byref(d), FAKE, ps, pf, pl, n, b, kept, ks, FAKE, None, None)
    assert sel(pl=None) == _lib.KVC_ERR_ARG
    assert sel(kept=None) == _lib.KVC_ERR_ARG
    assert sel(ps=4097) == _lib.KVC_ERR_UNSUPPORTED                 # lengths up to 4096 keep the sums in 32 bits
    assert sel(n=1 << 20) == _lib.KVC_ERR_UNSUPPORTED
    assert sel(n=0) == _lib.KVC_ERR_UNSUPPORTED
    assert sel(b=-1) == _lib.KVC_ERR_ARG
    assert sel(ks=0) == _lib.KVC_ERR_ARG
    assert sel(pf=None, pl=None, n=63) == _lib.KVC_ERR_ARG          # 63 uniform pages of 16 pass 1000 tokens
    assert lib.kvc_last_error().decode().startswith("kvc_page_select")


def test_compact_reference_store_rejects_bad_combinations():
    lib = _lib.load()
    d = _dims()
    out = _lib.KvcCompactOut()
    out.out_stride = 512
    out.K_out = out.V_out = FAKE
    call = lambda rb=0, base=1e4: lib.kvc_compact_rerotate(ctypes.byref(d), FAKE, FAKE, None, FAKE, 512, FAKE,
                                                           rb, base, ctypes.byref(out), None)
    out.K_ref_out = FAKE
    assert call() == _lib.KVC_ERR_ARG                            # p_ref_out missing
    out.p_ref_out = FAKE
    out.K_ref = FAKE
    assert call() == _lib.KVC_ERR_ARG                            # K_ref without p_ref
    out.p_ref = FAKE
    assert call(rb=-1, base=1.0) == _lib.KVC_ERR_ARG             # the check rotates: base must exceed 1
    out.kept_page = 16
    assert call() == _lib.KVC_ERR_UNSUPPORTED                    # plain per-row lists only
    out.kept_page = 0
    out.action = FAKE
    out.Kq = out.Vq = out.Ks = out.Vs = FAKE
    assert call() == _lib.KVC_ERR_UNSUPPORTED


def test_select_rejects_bad_tag_layout_and_decode_h2o_arguments():
    lib = _lib.load()
    d = _dims()
    p = _policy()
    p.tag_rows = 2
    assert lib.kvc_select(ctypes.byref(d), FAKE, ctypes.byref(p), FAKE, 512, FAKE, None, 0, None) == _lib.KVC_ERR_ARG
    ws = lib.kvc_decode_h2o_workspace_bytes(ctypes.byref(d), 512)
    assert ws > lib.kvc_decode_workspace_bytes(ctypes.byref(d), 512, 0)
    call = lambda **k: lib.kvc_decode_attn_h2o(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, k.get("stride", 512),
                                               k.get("acc", FAKE), FAKE, None, FAKE, k.get("ws", ws), None)
    assert call(acc=None) == _lib.KVC_ERR_ARG
    assert call(stride=0) == _lib.KVC_ERR_ARG
    assert call(ws=ws - 1) == _lib.KVC_ERR_WORKSPACE


def test_compact_carry_rejects_half_pairs_and_tiered_path():
    lib = _lib.load()
    d = _dims()
    out = _lib.KvcCompactOut()
    out.out_stride = 512
    out.K_out = out.V_out = FAKE
    call = lambda: lib.kvc_compact_rerotate(ctypes.byref(d), FAKE, FAKE, None, FAKE, 512, FAKE, -1, 1e4,
                                            ctypes.byref(out), None)
    out.score_in = FAKE
    assert call() == _lib.KVC_ERR_ARG                            # score_out missing
    out.score_out = FAKE
    out.tag_out = FAKE
    assert call() == _lib.KVC_ERR_ARG                            # tag_in missing
    out.tag_in = FAKE
    out.action = FAKE
    out.Kq = out.Vq = out.Ks = out.Vs = FAKE
    assert call() == _lib.KVC_ERR_UNSUPPORTED


def test_pool_rejects_bad_kernel_mode_and_alias():
    lib = _lib.load()
    d = _dims()
    other = FAKE + 64
    assert lib.kvc_pool_scores(ctypes.byref(d), FAKE, 4, 0, other, None) == _lib.KVC_ERR_ARG     # even kernel
    assert lib.kvc_pool_scores(ctypes.byref(d), FAKE, 257, 0, other, None) == _lib.KVC_ERR_ARG
    assert lib.kvc_pool_scores(ctypes.byref(d), FAKE, 7, 2, other, None) == _lib.KVC_ERR_ARG     # mode
    assert lib.kvc_pool_scores(ctypes.byref(d), FAKE, 7, 0, FAKE, None) == _lib.KVC_ERR_ARG      # alias
    assert lib.kvc_pool_scores(ctypes.byref(d), FAKE, 7, 0, None, None) == _lib.KVC_ERR_ARG
