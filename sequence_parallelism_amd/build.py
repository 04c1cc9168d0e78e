"""Build the HIP library (libusp.so) in-tree for gfx950 with hipcc.

Usage: python -m sequence_parallelism_amd.build
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libusp.so")
SOURCES = ["usp_abi.hip", "permute.hip", "merge.hip", "attn_fwd.hip", "attn_bwd.hip",
           "attn_bwd_dq.hip", "schedule.hip"]

# gfx950 only; packed-FP32 VALU instructions disabled.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"),
]


# Per-file additions.  attn_bwd.hip: MFMA results in VGPRs (its only AGPRs are the
# dK^T / dV^T accumulators, pinned there by inline assembly), so the softmax reads
# the score accumulators without AGPR-to-VGPR copies.
EXTRA_FLAGS = {
    "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose=False):
    """Compile every source into an object (with its own extra flags), then link
    libusp.so.  Always recompiles."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()

    def compile_one(name):
        obj = os.path.join(objdir, name + ".o")
        cmd = [cc] + HIPCC_FLAGS + ["-c"] + EXTRA_FLAGS.get(name, []) + [os.path.join(CSRC, name), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {name}:\n" + res.stdout + res.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
