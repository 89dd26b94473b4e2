"""Builds libkvc.so (the HIP kernels and the C ABI) in-tree for gfx950.

Every source under csrc/ (HIP kernels and host C++) is compiled with hipcc for gfx950 and linked
into budgeted_retention_amd/libkvc.so. Packed-FP32 instructions are disabled
for all device code.
"""
import concurrent.futures
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libkvc.so")

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: cannot build libkvc.so")
    return exe


# Per-source extra flags. The score and page-effect kernels consume every MFMA
# result on the VALU; keeping the accumulators in VGPRs (instead of AGPRs)
# saves one v_accvgpr_read per logit.
EXTRA_FLAGS = {
    "score.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "page_effect.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


# AddressSanitizer on the host code only (device code is never instrumented):
# the argument checks, workspace sizing and host control routines run under it.
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
ASAN_LIB_PATH = os.path.join(PKG, "libkvc_asan.so")

# Bounds-checked kernels: every index wrapped in KVC_IDX is checked against its
# range and caller data the kernels clamp is noted (kvc_check_read reports both).
CHECK_FLAGS = ["-DKVC_CHECK"]
CHECK_LIB_PATH = os.path.join(PKG, "libkvc_check.so")


def _compile(src, obj, verbose, extra=()):
    cmd = [_hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose=False, jobs=8, asan=False, check=False):
    """Compile every csrc/*.hip and link libkvc.so; returns the library path.
    asan=True builds libkvc_asan.so instead, the host code under AddressSanitizer
    (load it with the sanitizer runtime preloaded; see asan_runtime());
    check=True builds libkvc_check.so, the kernels with their bounds checks."""
    if asan and check:
        raise ValueError("one variant per build")
    bdir = BUILD_DIR + ("_asan" if asan else "_check" if check else "")
    out = ASAN_LIB_PATH if asan else CHECK_LIB_PATH if check else LIB_PATH
    extra = ASAN_FLAGS if asan else CHECK_FLAGS if check else []
    os.makedirs(bdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = [os.path.join(bdir, os.path.splitext(os.path.basename(s))[0] + ".o") for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], verbose, extra), zip(srcs, objs)))
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    _write_build_info()
    return out


BUILD_INFO = os.path.join(PKG, "build_info.json")


def _write_build_info():
    """The commit the library was built from (for run records on machines
    that get the tree without its history)."""
    import json
    info = {"git": None, "dirty": None}
    try:
        info["git"] = subprocess.run(["git", "rev-parse", "--short=12", "HEAD"], cwd=ROOT, capture_output=True,
                                     text=True, timeout=10).stdout.strip() or None
        st = subprocess.run(["git", "status", "--porcelain", "--untracked-files=no"], cwd=ROOT,
                            capture_output=True, text=True, timeout=10).stdout
        info["dirty"] = bool(st.strip()) if info["git"] else None
    except Exception:
        pass
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f)


def asan_runtime():
    """The AddressSanitizer runtime of hipcc's compiler, to preload into Python."""
    res = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime of hipcc's compiler was not found")
    return path


if __name__ == "__main__":
    import sys
    if "--asan" in sys.argv:
        print(build(verbose=True, asan=True))
        print(asan_runtime())
    elif "--check" in sys.argv:
        print(build(verbose=True, check=True))
    else:
        print(build(verbose=True))
