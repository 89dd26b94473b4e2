"""ctypes loader for libkvc.so: struct layouts and function prototypes of
include/kvc.h. Loading fails loudly when the library has not been built."""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# KVC_LIBRARY selects another build of the same library (the AddressSanitizer
# build, libkvc_asan.so, for host-side checks; the bounds-checked build,
# libkvc_check.so); by default the in-tree libkvc.so.
LIB_PATH = os.environ.get("KVC_LIBRARY") or os.path.join(_PKG, "libkvc.so")

KVC_OK = 0
KVC_WARN_FLOOR_EXCESS = 1
KVC_ERR_ARG = -1
KVC_ERR_UNSUPPORTED = -2
KVC_ERR_WORKSPACE = -3
KVC_ERR_HIP = -4

# kvc_check_read bits (bounds-checked builds)
KVC_CHK_SCORE = 1 << 0
KVC_CHK_SELECT = 1 << 1
KVC_CHK_COMPACT = 1 << 2
KVC_CHK_DECODE = 1 << 3
KVC_CHK_POOL = 1 << 4
KVC_CHK_PAGE = 1 << 5
KVC_CHK_KEPT = 1 << 8
KVC_CHK_COUNT = 1 << 9
KVC_CHK_SPAN = 1 << 10
KVC_CHK_BLOCK = 1 << 11

KVC_OP_SCORE = 1
KVC_OP_SELECT = 2

c_void_p = ctypes.c_void_p
c_int32 = ctypes.c_int32
c_int64 = ctypes.c_int64
c_size_t = ctypes.c_size_t
c_double = ctypes.c_double


class KvcDims(ctypes.Structure):
    _fields_ = [
        ("n_seq", c_int32), ("n_layers", c_int32), ("n_kv_heads", c_int32),
        ("n_q_heads", c_int32), ("head_dim", c_int32), ("reserved", c_int32),
        ("n_tokens", c_int64),
    ]


class KvcPolicy(ctypes.Structure):
    _fields_ = [
        ("n_sink", c_int32), ("n_recent", c_int32), ("budget", c_int32),
        ("n_tags", c_int32), ("n_groups", c_int32), ("layer_base", c_int32),
        ("n_layers_model", c_int32), ("tag_rows", c_int32),
        ("tags", c_void_p), ("tag_bonus", c_void_p), ("tag_floor", c_void_p),
    ]


class KvcCompactOut(ctypes.Structure):
    _fields_ = [
        ("action", c_void_p), ("out_stride", c_int32), ("kept_page", c_int32),
        ("h_base", c_void_p), ("l_base", c_void_p),
        ("K_out", c_void_p), ("V_out", c_void_p), ("pos_out", c_void_p), ("n_h", c_void_p),
        ("Kq", c_void_p), ("Vq", c_void_p), ("Ks", c_void_p), ("Vs", c_void_p),
        ("pos_q", c_void_p), ("n_l", c_void_p),
        ("K_ref", c_void_p), ("p_ref", c_void_p), ("K_ref_out", c_void_p), ("p_ref_out", c_void_p),
        ("score_in", c_void_p), ("score_out", c_void_p), ("tag_in", c_void_p), ("tag_out", c_void_p),
        ("low_bits", c_int32),
    ]


class KvcPaskTable(ctypes.Structure):
    _fields_ = [("n_tags", c_int32), ("n_groups", c_int32), ("a0", c_void_p), ("amin", c_void_p),
                ("prio", c_void_p), ("critical", c_void_p)]


# name -> (restype, argtypes); mirrors include/kvc.h
PROTOTYPES = {
    "kvc_version": (ctypes.c_int, []),
    "kvc_last_error": (ctypes.c_char_p, []),
    "kvc_check_read": (ctypes.c_int, [c_void_p, c_void_p]),
    "kvc_workspace_bytes": (c_size_t, [ctypes.c_int, ctypes.POINTER(KvcDims), c_int32, c_int32]),
    "kvc_layer_group": (c_int32, [c_int32, c_int32, c_int32]),
    "kvc_foresight_bonus": (c_double, [c_double, c_double, c_double]),
    "kvc_score": (ctypes.c_int, [ctypes.POINTER(KvcDims), c_void_p, c_void_p, c_int32,
                                 c_void_p, c_void_p, c_size_t, c_void_p]),
    "kvc_score_noalloc": (ctypes.c_int, [ctypes.POINTER(KvcDims), c_void_p, c_void_p, c_int32, c_void_p, c_void_p]),
    "kvc_score_noalloc_max_bytes": (c_size_t, []),
    "kvc_score_options": (ctypes.c_int, [c_int32, ctypes.c_int64, c_int32]),
    "kvc_score_status": (ctypes.c_int, [c_void_p, c_void_p]),
    "kvc_pool_scores": (ctypes.c_int, [ctypes.POINTER(KvcDims), c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
    "kvc_select": (ctypes.c_int, [ctypes.POINTER(KvcDims), c_void_p, ctypes.POINTER(KvcPolicy),
                                  c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "kvc_compact_rerotate": (ctypes.c_int, [ctypes.POINTER(KvcDims), c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_int32, c_void_p, c_int32, c_double,
                                            ctypes.POINTER(KvcCompactOut), c_void_p]),
    "kvc_decode_workspace_bytes": (c_size_t, [ctypes.POINTER(KvcDims), c_int64, c_int64]),
    "kvc_decode_attn": (ctypes.c_int, [ctypes.POINTER(KvcDims), c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_int64, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_void_p, c_void_p,
                                       c_void_p, c_size_t, c_void_p]),
    "kvc_decode_h2o_workspace_bytes": (c_size_t, [ctypes.POINTER(KvcDims), c_int64]),
    "kvc_decode_attn_h2o": (ctypes.c_int, [ctypes.POINTER(KvcDims), c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_int64, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                           c_void_p]),
    "kvc_page_workspace_bytes": (c_size_t, [ctypes.POINTER(KvcDims), c_int32, c_int64]),
    "kvc_page_effect": (ctypes.c_int, [ctypes.POINTER(KvcDims), c_int32, c_void_p, c_void_p, c_void_p,
                                       c_int32, c_int64, c_int32, c_void_p, c_void_p, c_int32, c_void_p,
                                       c_void_p, c_void_p, c_size_t, c_void_p]),
    "kvc_page_retire": (ctypes.c_int, [ctypes.POINTER(KvcDims), c_int32, c_void_p, c_void_p, c_void_p,
                                       c_int32, c_int64, c_int32, c_void_p, c_void_p, c_int32, c_void_p,
                                       c_int32, ctypes.c_float, c_void_p, c_void_p, c_void_p, c_size_t,
                                       c_void_p]),
    "kvc_page_scores": (ctypes.c_int, [ctypes.POINTER(KvcDims), c_void_p, c_int32, c_void_p, c_void_p,
                                       c_int32, c_void_p, c_void_p, c_int32, c_void_p, c_void_p]),
    "kvc_page_tokens": (ctypes.c_int, [ctypes.POINTER(KvcDims), c_int32, c_void_p, c_void_p, c_int32,
                                       c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_void_p]),
    "kvc_page_select": (ctypes.c_int, [ctypes.POINTER(KvcDims), c_void_p, c_int32, c_void_p, c_void_p, c_int32,
                                       c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    "kvc_host_pask_row_actions": (ctypes.c_int, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                                 c_void_p]),
    "kvc_host_event_pages": (ctypes.c_int, [c_void_p, c_int32, c_int32, c_int64, c_void_p, c_void_p, c_int32,
                                            c_void_p]),
    "kvc_host_commit_protect": (ctypes.c_int, [c_void_p, c_void_p, c_int32, c_int32, c_double, c_int32,
                                               c_void_p, c_void_p]),
    "kvc_host_pace_renumber": (ctypes.c_int, [c_int64, c_int64, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                              c_void_p]),
    "kvc_host_pask_costs": (ctypes.c_int, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p]),
    "kvc_host_pask_control": (ctypes.c_int, [ctypes.POINTER(KvcPaskTable), c_void_p, c_double, c_double,
                                             c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
    "kvc_host_commit_candidates": (ctypes.c_int, [c_void_p, c_void_p, c_int32, ctypes.c_float,
                                                  ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                                  c_int32, c_void_p, c_void_p, c_void_p]),
}

_lib = None


def load():
    """Load libkvc.so once and attach the prototypes. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
            "(the HIP library is required; there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class KvcError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"kvc status {status}: {message}")
        self.status = status


def check(status, allow_warn=True):
    if status == KVC_OK or (allow_warn and status > 0):
        return status
    raise KvcError(status, load().kvc_last_error().decode())
