"""Thin Python binding of libkvc.so with the C ABI's names.

Only argument marshalling happens here: torch tensors (device memory) are
checked for device, dtype and contiguity and turned into raw pointers, and
the call's status is turned into an exception. Every step of the path runs in
the HIP kernels behind the ABI; there is no fallback implementation.
"""
import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib

KvcDims = _lib.KvcDims
KVC_OP_SCORE = _lib.KVC_OP_SCORE
KVC_OP_SELECT = _lib.KVC_OP_SELECT
KVC_OK = _lib.KVC_OK
KVC_WARN_FLOOR_EXCESS = _lib.KVC_WARN_FLOOR_EXCESS
# kvc_compact_out.action codes (PASK {R, L, H}): release, int8 tier, bf16 tier
ACT_RELEASE, ACT_INT8, ACT_BF16 = 0, 1, 2
KvcError = _lib.KvcError


def make_dims(n_seq, n_layers, n_kv_heads, n_q_heads, head_dim, n_tokens):
    return KvcDims(n_seq, n_layers, n_kv_heads, n_q_heads, head_dim, 0, n_tokens)


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must live in GPU memory (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def kvc_version():
    return _lib.load().kvc_version()


def kvc_check_read(stream=None):
    """Bounds-checked builds: the kvc_check_read bits reported since the last
    read (0 when none), after synchronising the stream; raises KvcError
    (KVC_ERR_UNSUPPORTED) in other builds."""
    sites = ctypes.c_uint32(0)
    _lib.check(_lib.load().kvc_check_read(_stream(stream), ctypes.byref(sites)))
    return sites.value


def kvc_layer_group(layer, n_layers, n_groups):
    return _lib.load().kvc_layer_group(layer, n_layers, n_groups)


def kvc_foresight_bonus(sigma, lam, steps_ahead):
    return _lib.load().kvc_foresight_bonus(sigma, lam, steps_ahead)


def kvc_workspace_bytes(op, dims, W=0, B=0):
    lib = _lib.load()
    n = lib.kvc_workspace_bytes(op, ctypes.byref(dims), W, B)
    if n == 0 and lib.kvc_last_error():
        msg = lib.kvc_last_error().decode()
        if msg.startswith("kvc_workspace_bytes"):
            raise KvcError(_lib.KVC_ERR_ARG, msg)
    return n


def workspace(op, dims, W=0, B=0, device="cuda"):
    """Allocate (through torch) the workspace an operation needs."""
    n = kvc_workspace_bytes(op, dims, W, B)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def kvc_score(dims, K, Q_obs, W, scores, ws, stream=None):
    st = _lib.load().kvc_score(
        ctypes.byref(dims), _ptr(K, torch.bfloat16, "K"), _ptr(Q_obs, torch.bfloat16, "Q_obs"), W,
        _ptr(scores, torch.float32, "scores"), _ptr(ws, None, "ws"),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    return _lib.check(st)



def kvc_score_noalloc(dims, K, Q_obs, W, scores, stream=None):
    """kvc_score without a workspace: the library's static scratch array."""
    st = _lib.load().kvc_score_noalloc(
        ctypes.byref(dims), _ptr(K, torch.bfloat16, "K"), _ptr(Q_obs, torch.bfloat16, "Q_obs"), W,
        _ptr(scores, torch.float32, "scores"), _stream(stream))
    return _lib.check(st)


def kvc_score_options(single_read=False, wait_us=200000, diag_no_merge=False):
    return _lib.check(_lib.load().kvc_score_options(int(single_read), int(wait_us), int(diag_no_merge)))


def kvc_score_status(ws=None, stream=None):
    """Status of the last kvc_score call on `ws` (None: the last no-allocation call)."""
    return _lib.check(_lib.load().kvc_score_status(_ptr(ws, None, "ws"), _stream(stream)))


KVC_POOL_MAX, KVC_POOL_AVG = 0, 1


def kvc_pool_scores(dims, scores, kernel, mode, pooled, stream=None):
    st = _lib.load().kvc_pool_scores(ctypes.byref(dims), _ptr(scores, torch.float32, "scores"), kernel, mode,
                                     _ptr(pooled, torch.float32, "pooled"), _stream(stream))
    return _lib.check(st)

@dataclass
class Policy:
    n_sink: int
    n_recent: int
    budget: int
    n_tags: int = 1
    n_groups: int = 1
    layer_base: int = 0
    n_layers_model: int = 1
    tags: Optional[torch.Tensor] = None        # uint8 [N][T] (or [N][L][Hkv][T], tag_rows=1)
    tag_bonus: Optional[torch.Tensor] = None   # float32 [n_tags][n_groups]
    tag_floor: Optional[torch.Tensor] = None   # uint8 [n_tags][n_groups]
    tag_rows: int = 0                          # 1: tags are [N][L][Hkv][T], one per row

    def to_c(self):
        return _lib.KvcPolicy(
            self.n_sink, self.n_recent, self.budget, self.n_tags, self.n_groups, self.layer_base,
            self.n_layers_model, self.tag_rows, _ptr(self.tags, torch.uint8, "tags"),
            _ptr(self.tag_bonus, torch.float32, "tag_bonus"),
            _ptr(self.tag_floor, torch.uint8, "tag_floor"))


def kvc_select(dims, scores, policy: Policy, kept_idx, kept_stride, n_kept, ws=None, stream=None):
    """ws=None: a workspace of kvc_workspace_bytes(KVC_OP_SELECT) bytes is
    allocated here when the rows need one (long rows), else none is passed."""
    if ws is None:
        n = kvc_workspace_bytes(KVC_OP_SELECT, dims, 0, policy.budget)
        if n:
            ws = torch.empty(n, dtype=torch.uint8, device=scores.device)
    pol = policy.to_c()
    st = _lib.load().kvc_select(
        ctypes.byref(dims), _ptr(scores, torch.float32, "scores"), ctypes.byref(pol),
        _ptr(kept_idx, torch.int32, "kept_idx"), kept_stride, _ptr(n_kept, torch.int32, "n_kept"),
        _ptr(ws, None, "ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    return _lib.check(st)


@dataclass
class CompactOut:
    out_stride: int
    K_out: torch.Tensor
    V_out: torch.Tensor
    pos_out: Optional[torch.Tensor] = None
    n_h: Optional[torch.Tensor] = None
    action: Optional[torch.Tensor] = None      # uint8 [rows][kept_stride]
    Kq: Optional[torch.Tensor] = None
    Vq: Optional[torch.Tensor] = None
    Ks: Optional[torch.Tensor] = None          # fp16 scales stored as int16 bits
    Vs: Optional[torch.Tensor] = None
    pos_q: Optional[torch.Tensor] = None
    n_l: Optional[torch.Tensor] = None
    h_base: Optional[torch.Tensor] = None      # int32 [rows] first bf16 slot (append)
    l_base: Optional[torch.Tensor] = None      # int32 [rows] first int8 slot (append)
    kept_page: int = 0                         # > 0: kept lists are per-sequence page indices
    low_bits: int = 8                          # low tier codes: 8 (int8) or 4 (two nibbles per byte)
    K_ref: Optional[torch.Tensor] = None       # reference store of the current slots (bf16)
    p_ref: Optional[torch.Tensor] = None       # int32 positions of those references (< 0: none)
    K_ref_out: Optional[torch.Tensor] = None   # reference store of the kept slots
    p_ref_out: Optional[torch.Tensor] = None
    score_in: Optional[torch.Tensor] = None    # fp32 per-slot running score carried with the tokens
    score_out: Optional[torch.Tensor] = None
    tag_in: Optional[torch.Tensor] = None      # uint8 per-slot tag carried with the tokens
    tag_out: Optional[torch.Tensor] = None

    def to_c(self):
        return _lib.KvcCompactOut(
            _ptr(self.action, torch.uint8, "action"), self.out_stride, self.kept_page,
            _ptr(self.h_base, torch.int32, "h_base"), _ptr(self.l_base, torch.int32, "l_base"),
            _ptr(self.K_out, torch.bfloat16, "K_out"), _ptr(self.V_out, torch.bfloat16, "V_out"),
            _ptr(self.pos_out, torch.int32, "pos_out"), _ptr(self.n_h, torch.int32, "n_h"),
            _ptr(self.Kq, torch.int8, "Kq"), _ptr(self.Vq, torch.int8, "Vq"),
            _ptr(self.Ks, torch.int16, "Ks"), _ptr(self.Vs, torch.int16, "Vs"),
            _ptr(self.pos_q, torch.int32, "pos_q"), _ptr(self.n_l, torch.int32, "n_l"),
            _ptr(self.K_ref, torch.bfloat16, "K_ref"), _ptr(self.p_ref, torch.int32, "p_ref"),
            _ptr(self.K_ref_out, torch.bfloat16, "K_ref_out"), _ptr(self.p_ref_out, torch.int32, "p_ref_out"),
            _ptr(self.score_in, torch.float32, "score_in"), _ptr(self.score_out, torch.float32, "score_out"),
            _ptr(self.tag_in, torch.uint8, "tag_in"), _ptr(self.tag_out, torch.uint8, "tag_out"), self.low_bits)


def kvc_compact_rerotate(dims, K, V, pos_in, kept_idx, kept_stride, n_kept, renumber_base, rope_base,
                         out: CompactOut, stream=None):
    o = out.to_c()
    st = _lib.load().kvc_compact_rerotate(
        ctypes.byref(dims), _ptr(K, torch.bfloat16, "K"), _ptr(V, torch.bfloat16, "V"),
        _ptr(pos_in, torch.int32, "pos_in"), _ptr(kept_idx, torch.int32, "kept_idx"), kept_stride,
        _ptr(n_kept, torch.int32, "n_kept"), renumber_base, float(rope_base), ctypes.byref(o),
        _stream(stream))
    return _lib.check(st)


def kvc_decode_workspace_bytes(dims, max_h, stride_l=0):
    return _lib.load().kvc_decode_workspace_bytes(ctypes.byref(dims), max_h, stride_l)


def kvc_decode_attn(dims, q, K, V, n_h, stride_h, o, ws, lse=None, block_table=None, page_size=0,
                    blocks_per_seq=0, Kq=None, Vq=None, Ks=None, Vs=None, n_l=None, stride_l=0,
                    low_bits=8, stream=None):
    st = _lib.load().kvc_decode_attn(
        ctypes.byref(dims), _ptr(q, torch.bfloat16, "q"), _ptr(K, torch.bfloat16, "K"),
        _ptr(V, torch.bfloat16, "V"), _ptr(n_h, torch.int32, "n_h"), stride_h,
        _ptr(block_table, torch.int32, "block_table"), page_size, blocks_per_seq,
        _ptr(Kq, torch.int8, "Kq"), _ptr(Vq, torch.int8, "Vq"), _ptr(Ks, torch.int16, "Ks"),
        _ptr(Vs, torch.int16, "Vs"), _ptr(n_l, torch.int32, "n_l"), stride_l, low_bits,
        _ptr(o, torch.bfloat16, "o"), _ptr(lse, torch.float32, "lse"), _ptr(ws, None, "ws"),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    return _lib.check(st)


def kvc_decode_h2o_workspace_bytes(dims, stride_h):
    return _lib.load().kvc_decode_h2o_workspace_bytes(ctypes.byref(dims), stride_h)


def kvc_decode_attn_h2o(dims, q, K, V, n_h, stride_h, acc, o, ws, lse=None, stream=None):
    st = _lib.load().kvc_decode_attn_h2o(
        ctypes.byref(dims), _ptr(q, torch.bfloat16, "q"), _ptr(K, torch.bfloat16, "K"),
        _ptr(V, torch.bfloat16, "V"), _ptr(n_h, torch.int32, "n_h"), stride_h,
        _ptr(acc, torch.float32, "acc"), _ptr(o, torch.bfloat16, "o"), _ptr(lse, torch.float32, "lse"),
        _ptr(ws, None, "ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    return _lib.check(st)


def kvc_page_workspace_bytes(dims, W, q_first):
    return _lib.load().kvc_page_workspace_bytes(ctypes.byref(dims), W, q_first)


def page_workspace(dims, W, q_first, device="cuda"):
    return torch.empty(max(1, kvc_page_workspace_bytes(dims, W, q_first)), dtype=torch.uint8,
                       device=device)


def _pages(page_first, page_len):
    """Event pages: int32 [N][n_pages] first token and length, both or neither."""
    if (page_first is None) != (page_len is None):
        raise ValueError("page_first and page_len go together")
    return _ptr(page_first, torch.int32, "page_first"), _ptr(page_len, torch.int32, "page_len")


def kvc_page_effect(dims, layer, K, V, Q_win, W, q_first, page_size, n_pages, effect_rel, ws,
                    effect_abs=None, stream=None, page_first=None, page_len=None):
    pf, pl = _pages(page_first, page_len)
    st = _lib.load().kvc_page_effect(
        ctypes.byref(dims), layer, _ptr(K, torch.bfloat16, "K"), _ptr(V, torch.bfloat16, "V"),
        _ptr(Q_win, torch.bfloat16, "Q_win"), W, q_first, page_size, pf, pl, n_pages,
        _ptr(effect_rel, torch.float32, "effect_rel"), _ptr(effect_abs, torch.float32, "effect_abs"),
        _ptr(ws, None, "ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    return _lib.check(st)


def kvc_page_retire(dims, layer, K, V, Q_win, W, q_first, page_size, n_pages, order, tau_joint,
                    accepted, ws, joint_rel=None, stream=None, page_first=None, page_len=None):
    n_cand = order.shape[-1]
    pf, pl = _pages(page_first, page_len)
    st = _lib.load().kvc_page_retire(
        ctypes.byref(dims), layer, _ptr(K, torch.bfloat16, "K"), _ptr(V, torch.bfloat16, "V"),
        _ptr(Q_win, torch.bfloat16, "Q_win"), W, q_first, page_size, pf, pl, n_pages,
        _ptr(order, torch.int32, "order"), n_cand, float(tau_joint), _ptr(accepted, torch.uint8, "accepted"),
        _ptr(joint_rel, torch.float32, "joint_rel"), _ptr(ws, None, "ws"),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    return _lib.check(st)


def kvc_page_scores(dims, scores, page_size, n_pages, page_score, order=None, accepted=None, stream=None,
                    page_first=None, page_len=None):
    n_cand = 0 if order is None else order.shape[-1]
    pf, pl = _pages(page_first, page_len)
    st = _lib.load().kvc_page_scores(
        ctypes.byref(dims), _ptr(scores, torch.float32, "scores"), page_size, pf, pl, n_pages,
        _ptr(order, torch.int32, "order"), _ptr(accepted, torch.uint8, "accepted"), n_cand,
        _ptr(page_score, torch.float32, "page_score"), _stream(stream))
    return _lib.check(st)


def kvc_page_select(dims, page_score, page_size, n_pages, budget, kept, n_kept, n_tokens=None,
                    page_first=None, page_len=None, stream=None):
    pf, pl = _pages(page_first, page_len)
    st = _lib.load().kvc_page_select(
        ctypes.byref(dims), _ptr(page_score, torch.float32, "page_score"), page_size, pf, pl, n_pages,
        int(budget), _ptr(kept, torch.int32, "kept"), kept.shape[-1], _ptr(n_kept, torch.int32, "n_kept"),
        _ptr(n_tokens, torch.int32, "n_tokens"), _stream(stream))
    return _lib.check(st)


def kvc_page_tokens(dims, page_size, n_pages, pages, n_listed, tokens, n_tokens, page_first=None,
                    page_len=None, stream=None):
    pf, pl = _pages(page_first, page_len)
    st = _lib.load().kvc_page_tokens(
        ctypes.byref(dims), page_size, pf, pl, n_pages, _ptr(pages, torch.int32, "pages"),
        _ptr(n_listed, torch.int32, "n_listed"), pages.shape[-1], _ptr(tokens, torch.int32, "tokens"),
        _ptr(n_tokens, torch.int32, "n_tokens"), tokens.shape[-1], _stream(stream))
    return _lib.check(st)


# ---------------------------------------------------------------- host control (numpy in/out)

def _np_ptr(a, dtype):
    import numpy as np
    if a.dtype != dtype or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"expected a contiguous {dtype} array")
    return a.ctypes.data


def kvc_host_pask_costs(layers_per_group, n_kv_heads, head_dim, low_bits=8):
    import numpy as np
    lpg = np.ascontiguousarray(layers_per_group, dtype=np.int32)
    out = np.zeros((lpg.size, 3), dtype=np.float64)
    _lib.check(_lib.load().kvc_host_pask_costs(_np_ptr(lpg, np.int32), lpg.size, n_kv_heads, head_dim,
                                               low_bits, _np_ptr(out, np.float64)))
    return out


def kvc_host_pask_control(a0, amin, prio, critical, costs, budget_fraction, tags, reserve=0.0):
    """tags: uint8 [n_seq][n_tok]. Returns (actions uint8 [n_seq][n_tok][C], ledger [n_seq][n_tok+1])."""
    import numpy as np
    a0 = np.ascontiguousarray(a0, np.uint8)
    amin = np.ascontiguousarray(amin, np.uint8)
    prio = np.ascontiguousarray(prio, np.float32)
    crit = np.ascontiguousarray(critical, np.uint8)
    costs = np.ascontiguousarray(costs, np.float64)
    tags = np.ascontiguousarray(tags, np.uint8)
    n_seq, n_tok = tags.shape
    C = a0.shape[1]
    tbl = _lib.KvcPaskTable(a0.shape[0], C, _np_ptr(a0, np.uint8), _np_ptr(amin, np.uint8),
                            _np_ptr(prio, np.float32), _np_ptr(crit, np.uint8))
    acts = np.zeros((n_seq, n_tok, C), np.uint8)
    ledger = np.zeros((n_seq, n_tok + 1), np.float64)
    _lib.check(_lib.load().kvc_host_pask_control(
        ctypes.byref(tbl), _np_ptr(costs, np.float64), float(budget_fraction), float(reserve),
        _np_ptr(tags, np.uint8), n_seq, n_tok, _np_ptr(acts, np.uint8), _np_ptr(ledger, np.float64)))
    return acts, ledger


def kvc_host_pask_row_actions(actions, n_layers, n_kv_heads, recent):
    """actions: uint8 [n_seq][n_tok][n_groups]. Returns uint8 [n_seq][n_layers][n_kv_heads][n_tok]."""
    import numpy as np
    acts = np.ascontiguousarray(actions, np.uint8)
    n_seq, n_tok, C = acts.shape
    out = np.zeros((n_seq, n_layers, n_kv_heads, n_tok), np.uint8)
    _lib.check(_lib.load().kvc_host_pask_row_actions(_np_ptr(acts, np.uint8), n_seq, n_tok, C, n_layers,
                                                     n_kv_heads, int(recent), _np_ptr(out, np.uint8)))
    return out


def kvc_host_event_pages(event_len, G, start=0):
    """event_len: int event lengths of one sequence, in order from token
    `start`. Returns (first, length), int32 [n_pages] in token order."""
    import numpy as np
    ev = np.ascontiguousarray(event_len, np.int32)
    cap = max(1, int(ev.astype(np.int64).clip(min=0).sum()))     # a page holds at least one token
    first, length = np.zeros(cap, np.int32), np.zeros(cap, np.int32)
    n = ctypes.c_int32(0)
    _lib.check(_lib.load().kvc_host_event_pages(_np_ptr(ev, np.int32), ev.size, int(G), int(start),
                                                _np_ptr(first, np.int32), _np_ptr(length, np.int32), cap,
                                                ctypes.byref(n)))
    return first[: n.value].copy(), length[: n.value].copy()


def kvc_host_commit_candidates(R_minus, R_plus, tau_use, tau_dead, rho_use, rho_dead, max_scan=64):
    """Returns (state uint8 [n_pages], order int32 [max_scan] padded with -1, n_order)."""
    import numpy as np
    Rm = np.ascontiguousarray(R_minus, np.float32)
    Rp = np.ascontiguousarray(R_plus, np.float32)
    state = np.zeros(Rm.size, np.uint8)
    order = np.zeros(max_scan, np.int32)
    n = ctypes.c_int32(0)
    _lib.check(_lib.load().kvc_host_commit_candidates(
        _np_ptr(Rm, np.float32), _np_ptr(Rp, np.float32), Rm.size, tau_use, tau_dead, rho_use, rho_dead,
        max_scan, _np_ptr(state, np.uint8), _np_ptr(order, np.int32), ctypes.addressof(n)))
    return state, order, n.value


def kvc_host_commit_protect(R_minus, page_tokens, budget, eta, max_pages=16):
    """Returns (protect uint8 [n_pending], n_protected)."""
    import numpy as np
    Rm = np.ascontiguousarray(R_minus, np.float32)
    pt = np.ascontiguousarray(page_tokens, np.int32)
    out = np.zeros(max(Rm.size, 1), np.uint8)
    n = ctypes.c_int32(0)
    _lib.check(_lib.load().kvc_host_commit_protect(
        _np_ptr(Rm, np.float32), _np_ptr(pt, np.int32), Rm.size, budget, float(eta), max_pages,
        _np_ptr(out, np.uint8), ctypes.addressof(n)))
    return out[:Rm.size], n.value


def kvc_host_pace_renumber(m_next, shift, resident, limit, headroom, b_max):
    """Returns (renumber bool, new_shift)."""
    ren = ctypes.c_int32(0)
    sh = ctypes.c_int64(0)
    _lib.check(_lib.load().kvc_host_pace_renumber(m_next, shift, resident, limit, headroom, b_max,
                                                   ctypes.addressof(ren), ctypes.addressof(sh)))
    return bool(ren.value), sh.value
