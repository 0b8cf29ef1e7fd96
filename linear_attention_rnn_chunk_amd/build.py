"""Build the C-ABI library libgdn_mi355x.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn_mi355x.so")
SOURCES = ["gdn_api.cpp", "gdn_kernels.hip", "gdn_decode.hip", "gdn_noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         # packed fp32 ALU forms are kept out of every code object
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # matrix-core results in ordinary VGPRs: the recurrence scales and converts its
         # accumulators with vector ALU ops, which cannot address AGPRs directly
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


# measurement build: the scan records per-phase step timestamps (gdn_debug_stamps)
STAMPS_LIB = os.path.join(HERE, "libgdn_mi355x_stamps.so")


def build(verbose: bool = False, stamps: bool = False) -> str:
    """Compile every HIP/C++ source into LIB (atomic replace), or with ``stamps`` the
    measurement build into STAMPS_LIB.  Returns its path."""
    lib = STAMPS_LIB if stamps else LIB
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = ([HIPCC] + FLAGS + (["-DGDN_SCAN_STAMPS"] if stamps else []) + [os.path.join(CSRC, s) for s in SOURCES]
           + ["-o", tmp])
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, out))
    if verbose and out:
        print(out, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, stamps="--stamps" in sys.argv[1:]))
