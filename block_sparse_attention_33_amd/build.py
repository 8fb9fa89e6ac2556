"""Build libmsa.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m block_sparse_attention_33_amd.build      # or __graft_entry__.build()

Every HIP source is compiled to an object under _build/, then linked into
block_sparse_attention_33_amd/libmsa.so.  Compiles every time it is called.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmsa.so")
ARCH = os.environ.get("MSA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["index_branch.hip", "invert.hip", "main_branch.hip", "decode.hip", "backward.hip", "probe.hip", "msa_api.cpp",
           "device_state.cpp"]

COMMON = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]

# MFMA accumulators in VGPRs for the forward kernels (their softmax reads
# every accumulator with VALU instructions; in AGPRs each value would first
# be copied out).  The backward keeps its long-lived dK / dV accumulators in
# AGPRs instead, which leaves the VGPRs to the K / V operands (measured 7 %
# faster on MI355X).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
PER_FILE = {"backward.hip": []}


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libmsa.so)")
    return exe


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [_hipcc(), *lang, *COMMON, *PER_FILE.get(src, VGPR_FORM), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
