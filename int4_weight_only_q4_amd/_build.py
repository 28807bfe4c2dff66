"""Builds libq4.so (the HIP kernels and C ABI) in-tree for gfx950 with hipcc.

Each ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in parallel,
skipped when the object is newer than its source and the headers), then linked
into ``libq4.so`` beside this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libq4.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
    # packed FP32 instructions stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every rounding as written in the source (hot loops use explicit fmaf / dot2):
    # fused and unfused paths must produce identical bits
    "-ffp-contract=off",
    "-Wno-unused-result",
]
# Per-source additions. The matvec matrix-core kernels take their MFMA results
# in ordinary VGPRs, which the scaling FMAs read directly (the accumulation-
# register form costs a v_accvgpr_read per value).
EXTRA_FLAGS = {
    "q4_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _headers_mtime() -> float:
    hs = glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(INCLUDE, "*.h"))
    return max(os.path.getmtime(h) for h in hs)


def _compile(src: str, force: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    if (not force and os.path.exists(obj)
            and os.path.getmtime(obj) > max(os.path.getmtime(src), _headers_mtime())):
        return obj
    cmd = [HIPCC] + FLAGS + EXTRA_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    os.replace(obj + ".tmp", obj)
    return obj


def build(force: bool = True, jobs: int = 8) -> str:
    """Compile every HIP source and link libq4.so. Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, force), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=False))
