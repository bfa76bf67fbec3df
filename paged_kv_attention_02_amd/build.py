"""Build libpka.so (HIP, gfx950) in-tree with hipcc.

    python -m paged_kv_attention_02_amd.build

The library is written next to this file; the Python binding loads it from
there.  Every HIP source is compiled for gfx950 only, with packed fp32 ops
disabled (-packed-fp32-ops).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpka.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: no copies between the AGPR and
    # VGPR files around the softmax (gfx950 reads both as MFMA operands)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
]


# Sources compiled on their own with extra flags, then linked in: the extend
# kernels for 192-wide keys take the max-ILP scheduling strategy (faster at
# those widths, slower for others, so not for the whole library).
EXTRA_FLAGS = {
    "extend_dk192.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def sources():
    return sorted(f for f in glob.glob(os.path.join(CSRC, "*.hip")) if os.path.basename(f) not in EXTRA_FLAGS)


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libpka.so (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    objs = []
    try:
        for name, extra in EXTRA_FLAGS.items():
            obj = "%s.%s.o" % (tmp, name)
            flags = [f for f in HIPCC_FLAGS if f != "-shared"]
            _run([hipcc(), *flags, *extra, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, name), "-o", obj],
                 verbose)
            objs.append(obj)
        # objects first: the driver marks every source after them as HIP
        _run([hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *objs, *sources(), "-o", tmp], verbose)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    os.replace(tmp, LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libpka.so")


if __name__ == "__main__":
    print(build(verbose=True))
