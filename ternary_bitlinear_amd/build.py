"""Build the HIP library libbitlinear.so in-tree for gfx950 (hipcc, no GPU needed)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbitlinear.so")
SOURCES = ["abi.hip", "pack.hip", "quant.hip", "forward.hip", "base3.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: no multiply-add fusion anywhere (the quantisers' rounding
#   decisions depend on each fp32 operation rounding on its own).
# -Xclang -target-feature -Xclang -packed-fp32-ops: no packed fp32 VALU ops.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    if verbose and (r.stdout or r.stderr):
        sys.stderr.write(r.stdout + r.stderr)
    # A kernel the host pass rejects silently leaves its launch stub undefined;
    # a shared library links anyway and only fails at load time.  Refuse it.
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    stubs = [l for l in nm.stdout.splitlines() if "__device_stub__" in l]
    if nm.returncode == 0 and stubs:
        os.remove(tmp)
        raise RuntimeError("undefined kernel stubs in the built library:\n" + "\n".join(stubs[:10]))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
