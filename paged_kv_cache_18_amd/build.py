"""Build libpa.so (gfx950) in-tree with hipcc.

``python -m paged_kv_cache_18_amd.build`` compiles every source under
``csrc/`` to an object in ``_build/`` (in parallel) and links
``paged_kv_cache_18_amd/libpa.so``.  It always recompiles: it is the
"does it build" check as well as the build.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # the packed fp32 instructions stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # matrix-core accumulators in ordinary VGPRs: the softmax rescale touches
    # them with vector ALU ops, which AGPRs would force to copy back and forth
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def sources():
    out = [os.path.join(CSRC, "pa_host.cpp"), os.path.join(CSRC, "pa_capi.cpp")]
    kdir = os.path.join(CSRC, "kernels")
    out += sorted(os.path.join(kdir, f) for f in os.listdir(kdir) if f.endswith(".hip"))
    return out


def hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: ROCm is required to build libpa")
    return h


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the fp32 feature flag above; that note is expected
    msgs = [ln for ln in (r.stderr or "").splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    return obj, "\n".join(m for m in msgs if m.strip())


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for obj, msgs in results:
        if msgs and verbose:
            print(msgs, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
