"""Build libdsa.so (all HIP kernels + the C ABI) in-tree for gfx950.

    python dsa_lightning_indexer_amd/build.py      (or __graft_entry__.build())
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libdsa.so")
BUILD = os.path.join(HERE, "_build")
ARCH = os.environ.get("DSA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["select.hip", "select_few.hip", "indexer.hip", "sparse_attn.hip", "overlap.hip", "distill.hip", "similarity.hip",
           "gather_probe.hip", "pattern_search.cpp", "api.cpp", "noalloc.hip"]
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Werror", "-Wno-unused-function",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-file extra flags.  The indexer's inputs and MFMA results are finite: with
# NaNs ruled out, fmaxf(x, 0) (the ReLU) is one v_max_f32 instead of a
# NaN-quieting v_max plus the max.
# MFMA results stay in VGPRs (the VALU epilogue reads them directly instead of
# copying them out of AGPRs).
EXTRA = {"indexer.hip": ["-fno-honor-nans"], "sparse_attn.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "distill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    return obj, msg


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, msg in results:
        if msg and verbose:
            print(msg, file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
