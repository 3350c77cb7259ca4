"""Build the HIP library ``libglass_amd.so`` in-tree for gfx950.

Each ``csrc/*.hip`` file is compiled with hipcc (in parallel) and the objects
are linked into one shared library next to this file.  Packed-FP32 VALU
instructions are disabled for all device code.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libglass_amd.so")
ARCH = os.environ.get("GLASS_AMD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-I" + INCLUDE, "-I" + CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, build_dir: str, extra) -> str:
    obj = os.path.join(build_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose: bool = True, out: str = LIB, defines=()) -> str:
    """Compile every source and link ``out`` (default: the in-tree library).
    ``defines``: extra ``NAME=VALUE`` preprocessor definitions (build options
    such as GLASS_AMD_RING_DEPTH)."""
    extra = ["-D" + d for d in defines]
    build_dir = BUILD if not defines else BUILD + "_" + "_".join(
        d.replace("=", "") for d in defines)
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), srcs))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out, file=sys.stderr)
    return out


# The debug build whose kernels first fill their LDS with NaN words (run the
# GPU parity tests against it with GLASS_AMD_LIBRARY pointing at it).
LIB_LDS_NAN = os.path.join(PKG, "libglass_amd_ldsnan.so")


if __name__ == "__main__":
    if "--lds-nan-fill" in sys.argv[1:]:
        build(out=LIB_LDS_NAN, defines=("GLASS_AMD_LDS_NAN_FILL=1",))
    else:
        build()
