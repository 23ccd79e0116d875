"""Build libgdn.so (the gfx950 HIP library) in-tree with hipcc.

Usage: python -m gated_deltanet_chunkwise_amd.build   (or build() from Python)
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = [os.path.join(CSRC, "gdn_api.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("gdn_common.h", "gdn_kernels.h", "gdn_kda.h", "gdn_decode.h", "gdn_bwd.h")] + [
    os.path.join(INCLUDE, "gdn.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # Keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs (gfx950 allows either): no AGPR<->VGPR
    # copies around the VALU work on accumulators (state decay, conversions).
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE,
    "-I", CSRC,
]


def build(out=LIB, extra=(), verbose=False):
    """Compile every HIP source into `out`.  Always recompiles."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *extra, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, err))
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def is_stale(lib=LIB):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(extra=sys.argv[1:], verbose=True))
