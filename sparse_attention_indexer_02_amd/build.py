"""Build the HIP library libsparse_indexer.so for gfx950, in-tree.

    python -m sparse_attention_indexer_02_amd.build
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsparse_indexer.so")
SOURCES = ["api.hip", "score.hip", "topk.hip", "witness.hip", "block_select.hip", "dosa.hip",
           "prior.hip", "consume.hip", "prefill_fused.hip"]
ARCH = os.environ.get("SI_OFFLOAD_ARCH", "gfx950")

COMMON = ["hipcc", f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          # never emit packed fp32 arithmetic
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas"]
# The block-sparse dot is defined as separately rounded products and adds.
EXTRA = {"block_select.hip": ["-ffp-contract=off"]}


def _compile(src, verbose):
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = COMMON + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, sources=None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in (sources or SOURCES) if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print("built", LIB)
