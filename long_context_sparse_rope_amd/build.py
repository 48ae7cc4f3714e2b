"""Build liblcsr.so (gfx950) in-tree with hipcc.

Every source under csrc/ is compiled to an object in _build/ and linked into
_lib/liblcsr.so.  HIP code is compiled with packed-fp32 instructions turned
off (-packed-fp32-ops).
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "liblcsr.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
HIP_FLAGS = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops"]
# Per-source extras.  The attention kernels take LLVM's memory-clause
# scheduling strategy (AMDGPU backend): it groups the LDS fragment reads of
# the consumer waves and measured about 1% less attention time per 1M-token
# step than the default strategy (same registers, same results).
EXTRA_FLAGS = {"attn.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]}


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = ([HIPCC] + COMMON + HIP_FLAGS + EXTRA_FLAGS.get(src, []) +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    if src.endswith(".cpp"):
        cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, r


def build(verbose=False, jobs=None):
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(8, len(srcs))
    objs = []
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for src, obj, r in ex.map(_compile, srcs):
            msgs = (r.stdout + r.stderr).strip()
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
            if verbose and msgs:
                print(f"[{src}]\n{msgs}", file=sys.stderr)
            objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
