"""Build the CPU oracle (plain C, gcc, OpenMP for the projection loop only)."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def command():
    return ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-fopenmp", "-ffp-contract=off",
            os.path.join(HERE, "ple_oracle.c"), "-lm", "-o", os.path.join(HERE, "libple_oracle.so")]


def build():
    p = subprocess.run(command(), stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if p.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + p.stdout.decode(errors="replace"))


if __name__ == "__main__":
    build()
