"""Build the CPU oracle (plain C, gcc, OpenMP for the projection loop only).

build() makes libple_oracle.so, the library the tests load. build(sanitize=True)
also makes the sanitizer artifacts the CPU tests run:
  - libple_oracle_ubsan.so: the same library with UndefinedBehaviorSanitizer
    (every report fatal); the pin suite runs against it in a subprocess with
    PLE_ORACLE_LIB pointing to it;
  - sanitize_check: an executable of the oracle and sanitize_check.c with
    AddressSanitizer and UndefinedBehaviorSanitizer linked in statically,
    which calls every oracle function on edge cases.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ple_oracle.c")
LIB = os.path.join(HERE, "libple_oracle.so")
UBSAN_LIB = os.path.join(HERE, "libple_oracle_ubsan.so")
CHECK_EXE = os.path.join(HERE, "sanitize_check")

_COMMON = ["-std=c11", "-fopenmp", "-ffp-contract=off"]
_SAN = ["-g", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]


def command():
    return ["gcc", "-O2", "-fPIC", "-shared", *_COMMON, SRC, "-lm", "-o", LIB]


def sanitize_commands():
    ubsan = ["gcc", "-O1", "-fPIC", "-shared", *_COMMON, *_SAN, "-fsanitize=undefined", SRC, "-lm",
             "-o", UBSAN_LIB]
    check = ["gcc", "-O1", *_COMMON, *_SAN, "-fsanitize=address,undefined", "-static-libasan",
             "-static-libubsan", SRC, os.path.join(HERE, "sanitize_check.c"), "-lm", "-o", CHECK_EXE]
    return [ubsan, check]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if p.returncode != 0:
        raise RuntimeError("oracle build failed: " + " ".join(cmd) + "\n" + p.stdout.decode(errors="replace"))


def build(sanitize: bool = False):
    _run(command())
    if sanitize:
        for cmd in sanitize_commands():
            _run(cmd)


if __name__ == "__main__":
    import sys
    build(sanitize="--sanitize" in sys.argv)
