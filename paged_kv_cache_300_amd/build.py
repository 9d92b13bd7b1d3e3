"""Build ``libpagedkv.so`` (the C ABI and its gfx950 kernels) in-tree with hipcc.

Usage: ``python -m paged_kv_cache_300_amd.build`` or ``build()`` from Python.  Every call recompiles.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libpagedkv.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["abi.cpp", "slot_store.hip", "qknorm_rope_store.hip", "attn_generic.hip", "attn_decode.hip",
           "attn_prefill.hip", "attn_prefill_w32.hip"]
# Per-source flags.  The 32x32 prefill keeps MFMA results in VGPRs (its exponentials read the scores directly);
# the query operand and the rest of its 512 registers go to AGPRs.
EXTRA_FLAGS = {"attn_prefill_w32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-function",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
    # Packed fp32 arithmetic stays off: the kernels are written for plain fp32 VALU ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _compile(hipcc, src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc, *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj, res.stderr


def build(verbose=False):
    """Compile every source for gfx950 and link ``libpagedkv.so`` next to this file; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(hipcc, s), SOURCES))
    objs = [r[0] for r in results]
    if verbose:
        for _, err in results:
            filtered = [ln for ln in err.splitlines() if "packed-fp32-ops" not in ln]
            if filtered:
                print("\n".join(filtered), file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
