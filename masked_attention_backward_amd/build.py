"""Build ``libmaskattn.so`` (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m masked_attention_backward_amd.build [-v]``.  Object files go to
``masked_attention_backward_amd/_build/``; the shared library to
``masked_attention_backward_amd/libmaskattn.so``.
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
LIB = os.path.join(PKG, "libmaskattn.so")
INCLUDE = os.path.join(ROOT, "include")

# (source, object name, preprocessor definitions).  attn_bwd_variant.hip is compiled once
# per dK/dV + dQ kernel variant the dispatch uses (dtype x mask kind x waves), so the large
# unrolled kernels build in parallel.
SOURCES = [("capi.hip", "capi", []), ("attn_bwd.hip", "attn_bwd", []), ("attn_fwd.hip", "attn_fwd", []),
           ("mask_tables.hip", "mask_tables", [])]
for _dt, _dtn in ((0, "f16"), (1, "bf16")):
    for _nw in (2, 4):
        SOURCES.append(("attn_bwd_variant.hip", f"bwd_{_dtn}_window_nw{_nw}",
                        [f"-DMA_VARIANT_DTYPE={_dt}", "-DMA_VARIANT_MASK=0", f"-DMA_VARIANT_NW={_nw}"]))
    for _nw in (1, 2, 3, 4):
        SOURCES.append(("attn_bwd_variant.hip", f"bwd_{_dtn}_block_nw{_nw}",
                        [f"-DMA_VARIANT_DTYPE={_dt}", "-DMA_VARIANT_MASK=1", f"-DMA_VARIANT_NW={_nw}"]))

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Packed fp32 VALU ops stay disabled: plain scalar fp32 code only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
    "-Wno-unused-result",
]


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libmaskattn.so")
    return exe


def _compile(entry, verbose):
    src, name, defs = entry
    obj = os.path.join(BUILD, name + ".o")
    cmd = [_hipcc(), *FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
