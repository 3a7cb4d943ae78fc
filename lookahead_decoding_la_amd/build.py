"""Build the HIP library liblaamd.so for gfx950 (in-tree).

    python -m lookahead_decoding_la_amd.build

Every HIP source in csrc/ is compiled with hipcc to an object file, then
linked into lookahead_decoding_la_amd/liblaamd.so.  Packed-fp32 instructions
are turned off for all device code.  The attention source selects its MFMAs
with VGPR accumulators: its softmax rescales the accumulators with vector
ALU operations, which cannot read AGPRs, and with AGPR accumulators the
compiler copies all of them between the two register files in every chunk.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblaamd.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include")]

# extra flags per source file
FILE_FLAGS = {"la_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip"))


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(OBJ, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        # the host pass does not know the device-only feature flag
        lines = [l for l in out.splitlines()
                 if "packed-fp32-ops" not in l or "error" in l]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed: " + ", ".join(failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
