"""The no-allocation score entry point (kvc_score_noalloc, for callers that
cannot allocate device memory) against kvc_score with a workspace, through
the C ABI: two calls in a row, the second on a smaller input, each bit-equal
to kvc_score's output on the same input (the same kernels run on the same
data); a call whose scratch would exceed the static array is refused."""
import ctypes

import numpy as np
import pytest
import torch

from budgeted_retention_amd import _lib, synth

pytestmark = pytest.mark.gpu


def _inputs(L, Hkv, Hq, d, T, W, seed):
    K = synth.normal_bf16((1, L, Hkv, T, d), seed, "cuda")
    Q = synth.normal_bf16((1, L, Hq, W, d), seed + 1, "cuda")
    return K, Q


def _both(L, Hkv, Hq, d, T, W, seed):
    from budgeted_retention_amd import kvc
    dims = kvc.make_dims(1, L, Hkv, Hq, d, T)
    K, Q = _inputs(L, Hkv, Hq, d, T, W, seed)
    want = torch.empty((1, L, Hkv, T), dtype=torch.float32, device="cuda")
    ws = kvc.workspace(kvc.KVC_OP_SCORE, dims, W, 0, K.device)
    kvc.kvc_score(dims, K, Q, W, want, ws)
    got = torch.full_like(want, float("nan"))
    kvc.kvc_score_noalloc(dims, K, Q, W, got)
    torch.cuda.synchronize()
    return want.cpu().numpy(), got.cpu().numpy()


def test_noalloc_matches_kvc_score_twice_second_smaller():
    print("noalloc: first call 4 layers x 8 KV heads, T=33,000, W=32, G=4", flush=True)
    want, got = _both(4, 8, 32, 128, 33_000, 32, 501)
    assert np.array_equal(want.view(np.uint32), got.view(np.uint32))
    np.testing.assert_allclose(got.sum(-1), 128.0, rtol=1e-4)
    print("noalloc: second call 1 layer x 2 KV heads, T=5,000, W=16, G=4, d=64", flush=True)
    want, got = _both(1, 2, 8, 64, 5_000, 16, 777)
    assert np.array_equal(want.view(np.uint32), got.view(np.uint32))
    np.testing.assert_allclose(got.sum(-1), 64.0, rtol=1e-4)


def test_noalloc_refuses_calls_beyond_its_scratch():
    from budgeted_retention_amd import kvc
    lib = _lib.load()
    cap = lib.kvc_score_noalloc_max_bytes()
    dims = kvc.make_dims(64, 32, 8, 32, 128, 4096)              # 16,384 rows: beyond the array
    assert kvc.kvc_workspace_bytes(kvc.KVC_OP_SCORE, dims, 32, 0) > cap
    st = lib.kvc_score_noalloc(ctypes.byref(dims), 0x1000, 0x1000, 32, 0x1000, None)
    assert st == _lib.KVC_ERR_WORKSPACE
    assert b"static" in lib.kvc_last_error()
