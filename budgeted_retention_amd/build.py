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


def _compile(src, obj, verbose):
    cmd = [_hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose=False, jobs=8):
    """Compile every csrc/*.hip and link libkvc.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = [os.path.join(BUILD_DIR, os.path.splitext(os.path.basename(s))[0] + ".o") for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], verbose), zip(srcs, objs)))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
