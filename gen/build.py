"""Build the two table-generator libraries (CPU: gcc; GPU: hipcc for gfx950)."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))

HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def commands():
    host = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-fopenmp", "-ffp-contract=off",
            os.path.join(HERE, "csrc", "tablegen_host.c"),
            "-o", os.path.join(HERE, "libplegen_host.so")]
    hip = ["/opt/rocm/bin/hipcc", *HIPCC_FLAGS, os.path.join(HERE, "csrc", "tablegen.hip"),
           "-o", os.path.join(HERE, "libplegen_hip.so")]
    return [host, hip]


def build():
    procs = [subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT) for c in commands()]
    for c, p in zip(commands(), procs):
        out, _ = p.communicate()
        if p.returncode != 0:
            raise RuntimeError("build failed: " + " ".join(c) + "\n" + out.decode(errors="replace"))


if __name__ == "__main__":
    build()
