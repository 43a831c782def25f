"""Build libple.so (the C-ABI library) from csrc/*.hip with hipcc for gfx950.

Each source compiles to an object in parallel, then one shared library is
linked next to this file, where the Python binding loads it.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libple.so")
HIPCC = "/opt/rocm/bin/hipcc"

SOURCES = ["ple_api.hip", "ple_hash.hip", "ple_gather.hip", "ple_proj.hip", "ple_fuse.hip", "ple_decode.hip"]

COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-I", os.path.join(ROOT, "include"),
          # packed fp32 instructions stay off (compiler-generated v_pk_*_f32)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
PER_FILE = {
    # the dequant sums two fp32 products; they must not contract to an FMA
    "ple_gather.hip": ["-ffp-contract=off"],
}


def compile_commands():
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        cmds.append([HIPCC, *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    return cmds


def link_command():
    objs = [os.path.join(OBJ, s.replace(".hip", ".o")) for s in SOURCES]
    return [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB]


def build(verbose: bool = False):
    os.makedirs(OBJ, exist_ok=True)
    procs = [(c, subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
             for c in compile_commands()]
    errors = []
    for c, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass warns that it does not know -packed-fp32-ops: harmless
        text = "\n".join(ln for ln in text.splitlines() if "packed-fp32-ops" not in ln)
        if p.returncode != 0:
            errors.append(" ".join(c) + "\n" + text)
        elif verbose and text.strip():
            print(text)
    if errors:
        raise RuntimeError("libple build failed:\n" + "\n".join(errors))
    p = subprocess.run(link_command(), stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if p.returncode != 0:
        raise RuntimeError("libple link failed:\n" + p.stdout.decode(errors="replace"))
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
