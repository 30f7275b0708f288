"""Build libvc.so (HIP for gfx950) in place with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libvc.so")
SOURCES = ["vc_core.cpp", "quant.hip", "select.hip", "draft.hip", "verify.hip", "accept.hip", "prefetch.cpp", "sched.cpp"]
ARCH = os.environ.get("VC_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    # IEEE fp32 division and sqrt (the quantiser must round exactly like the spec)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed-fp32 VALU instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs (no AGPR copies around MFMA)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]
# The attention kernels never see NaN in valid inputs: without NaN semantics
# their max reductions need no operand canonicalisation (2-3 % faster verify).
# The quantiser, the selector and argmax keep IEEE NaN behaviour.
FILE_FLAGS = {"draft.hip": ["-fno-honor-nans"], "verify.hip": ["-fno-honor-nans"]}


def _quiet(text: str) -> str:
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l)


def build(verbose: bool = True) -> str:
    """Compile every source to an object (in parallel), then link libvc.so."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    tmpdir = tempfile.mkdtemp(prefix="vc_build_")
    objs = [os.path.join(tmpdir, s + ".o") for s in SOURCES]

    def compile_one(i):
        src = SOURCES[i]
        cmd = ["hipcc", *FLAGS, *FILE_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", objs[i]]
        r = subprocess.run(cmd, capture_output=True, text=True)
        return cmd, r
    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        results = list(ex.map(compile_one, range(len(SOURCES))))
    for cmd, r in results:
        if verbose:
            print(" ".join(cmd), flush=True)
        out = _quiet(r.stdout + r.stderr)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed ({r.returncode}):\n{out}")
        if out.strip() and verbose:
            print(out, flush=True)
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-ldl"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc link failed ({r.returncode}):\n{_quiet(r.stdout + r.stderr)}")
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    os.rmdir(tmpdir)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
