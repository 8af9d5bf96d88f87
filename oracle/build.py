"""Build the CPU oracle (TEST INFRASTRUCTURE ONLY) into oracle/liboracle.so.

Plain scalar C, -O2, no fast-math, FP contraction off, default x86-64 ISA, so
every float operation is one IEEE operation in the order the source writes it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qk_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(extra_flags=(), lib=LIB):
    """Compile the oracle into `lib` (the in-tree liboracle.so by default; the
    sanitizer test builds an instrumented copy elsewhere)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-Werror", *extra_flags,
           "-o", lib + ".tmp", SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(sys.argv[1:]))
