"""Build the fp64 oracle (test infrastructure) into oracle/liboracle.so with gcc.

Plain C11, -O2, no fast-math and no FMA contraction, OpenMP over
(sequence, head). Run as ``python oracle/build.py``; ``__graft_entry__.build()``
calls :func:`build` too.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
FLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
         "-fno-fast-math", "-Wall", "-Wextra", "-Werror"]


def build(out: str = LIB, extra=()) -> str:
    src = os.path.join(HERE, "oracle.c")
    tmp = out + ".tmp"
    cmd = ["gcc", *FLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
