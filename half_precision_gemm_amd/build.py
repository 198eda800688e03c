"""Build libhgemm.so (the C-ABI library with its gfx950 kernels) in-tree.

    python half_precision_gemm_amd/build.py          # or __graft_entry__.build()

hipcc cross-compiles for gfx950 without a GPU.  Packed-fp32 VALU ops are
disabled for all device code (-packed-fp32-ops feature off).
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libhgemm.so")
SOURCES = [os.path.join(CSRC, "hg_api.cpp"), os.path.join(CSRC, "hg_kernels.hip"),
           os.path.join(CSRC, "hg_fast.hip"), os.path.join(CSRC, "hg_ring.hip"),
           os.path.join(CSRC, "hg_trsm.hip"), os.path.join(CSRC, "hg_xform.hip"),
           os.path.join(CSRC, "hg_noalloc.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(extra=(), out=LIB, verbose=False):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + list(extra) + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libhgemm.so")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
