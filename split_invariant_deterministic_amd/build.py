"""Builds libinv.so, the C-ABI library of hand-written gfx950 kernels.

    python -m split_invariant_deterministic_amd.build      (from the repo root)

Every source under csrc/ is compiled by hipcc for gfx950 into _build/ and
linked in-tree as split_invariant_deterministic_amd/libinv.so, which is what
the ctypes binding loads. Flags that fix numerics:

* -ffp-contract=off: a*b+c stays a rounded multiply and a rounded add unless
  the source asks for a fused multiply-add, so every kernel variant rounds
  the same way;
* -Xclang -target-feature -Xclang -packed-fp32-ops: no packed fp32 vector
  instructions are generated (host passes warn that they do not know the
  feature; that is harmless).
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libinv.so")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I" + os.path.join(ROOT, "include"),
]


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = ["hipcc"] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in p.stderr.splitlines() if noise not in l)
    return src, obj, p.returncode, err


def build(verbose=True, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(8, len(srcs))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, srcs))
    objs = []
    for src, obj, rc, err in results:
        if err.strip() and verbose:
            print(f"[{src}]\n{err}", file=sys.stderr)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src}")
        objs.append(obj)
    tmp = LIB + ".tmp"
    # -z defs: an unresolved symbol (say a kernel stub the compiler failed to
    # emit) fails the build here instead of the first dlopen on a GPU host
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp] + objs
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n" + p.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
