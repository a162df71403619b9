"""Build the HIP library libbitlinear.so in-tree for gfx950 (hipcc, no GPU needed).

Each source compiles to an object of its own (in parallel); the objects are
linked into one shared library.  Every kernel is launched from the source that
defines it, so no device code crosses objects.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbitlinear.so")
# chip-limit probes for the bench (a plain read, an int8 matrix-instruction
# loop); a library of their own, not part of the BitLinear ABI
PROBES_LIB = os.path.join(PKG, "libbitlinear_probes.so")
OBJ_DIR = os.path.join(PKG, "_build")
SOURCES = ["abi.hip", "pack.hip", "quant.hip", "forward.hip", "base3.hip", "noalloc.hip"]
PROBE_SOURCES = ["probes.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: no multiply-add fusion anywhere (the quantisers' rounding
#   decisions depend on each fp32 operation rounding on its own).
# -Xclang -target-feature -Xclang -packed-fp32-ops: no packed fp32 VALU ops.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd[-3:])}")
    if verbose and (r.stdout or r.stderr):
        sys.stderr.write(r.stdout + r.stderr)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = [s for s in SOURCES + PROBE_SOURCES if os.path.exists(os.path.join(CSRC, s))]
    objs = {s: os.path.join(OBJ_DIR, s.replace(".hip", ".o")) for s in srcs}
    cmds = [[HIPCC, *FLAGS, "-c", "-o", objs[s], os.path.join(CSRC, s)] for s in srcs]
    with ThreadPoolExecutor(max_workers=jobs or min(len(cmds), os.cpu_count() or 1)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    probe_objs = [objs[s] for s in PROBE_SOURCES if s in objs]
    if probe_objs:
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", PROBES_LIB, *probe_objs],
             verbose)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
          *[objs[s] for s in SOURCES if s in objs]], verbose)
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
