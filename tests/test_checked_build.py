"""The bounds-checked build (libkvc_check.so, the kernels compiled with
-DKVC_CHECK). On the CPU: it exports the whole C ABI, and the default build
answers kvc_check_read with KVC_ERR_UNSUPPORTED. On the GPU: a child process
with the checked library runs every kernel family on valid inputs (no check
bit may be set) and then on caller data that the kernels clamp (exactly the
kept-index, count, block-table and page-span bits, no index bit); every
output equals the default build's bit for bit."""
import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest

from budgeted_retention_amd import _lib, build as _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "tests"))

import checked_build_cases as cases  # noqa: E402
from test_abi_host import _declared_functions  # noqa: E402

INDEX_BITS = (_lib.KVC_CHK_SCORE | _lib.KVC_CHK_SELECT | _lib.KVC_CHK_COMPACT | _lib.KVC_CHK_DECODE
              | _lib.KVC_CHK_POOL | _lib.KVC_CHK_PAGE)


def test_checked_library_exports_every_declared_function():
    assert os.path.exists(_build.CHECK_LIB_PATH), "libkvc_check.so is built with libkvc.so"
    lib = ctypes.CDLL(_build.CHECK_LIB_PATH)
    missing = [n for n in sorted(_declared_functions()) if not hasattr(lib, n)]
    assert not missing, missing


@pytest.mark.skipif(os.path.basename(_lib.LIB_PATH) == "libkvc_check.so", reason="the checked build itself")
def test_default_build_has_no_check_words():
    lib = _lib.load()
    sites = ctypes.c_uint32(123)
    assert lib.kvc_check_read(None, ctypes.byref(sites)) == _lib.KVC_ERR_UNSUPPORTED
    assert sites.value == 0
    assert lib.kvc_check_read(None, None) == _lib.KVC_ERR_ARG


@pytest.mark.gpu
@pytest.mark.timeout(300)
def test_checked_build_runs_clean_and_matches_the_default_build(tmp_path):
    from budgeted_retention_amd import kvc
    assert os.path.basename(_lib.LIB_PATH) == "libkvc.so"
    path = str(tmp_path / "checked.npz")
    env = dict(os.environ, KVC_LIBRARY=_build.CHECK_LIB_PATH)
    res = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "checked_build_cases.py"), path],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=240)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    got = dict(np.load(path))
    assert int(got.pop("bits_valid")) == 0
    clamped = int(got.pop("bits_clamped"))
    assert clamped & INDEX_BITS == 0, hex(clamped)
    assert clamped == _lib.KVC_CHK_KEPT | _lib.KVC_CHK_COUNT | _lib.KVC_CHK_BLOCK | _lib.KVC_CHK_SPAN, hex(clamped)
    assert int(got.pop("bits_after_read")) == 0
    want = cases.valid_calls(kvc)
    want.update(cases.clamped_calls(kvc))
    assert got.keys() == want.keys()
    for k in want:
        np.testing.assert_array_equal(got[k], want[k], err_msg=k)
    # the clamped compaction skipped the entry past the cache (its slot kept
    # its old contents) and read row 1's list to its stride
    assert list(want["cmp_n"]) == [40, 40]
    assert want["cmp_pos"][0, 7] == -1 and (want["cmp_pos"][1] >= 0).all()
