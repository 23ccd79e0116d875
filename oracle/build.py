"""Compile the fp64 CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain gcc, IEEE fp64 (no fast-math, no -march), so results do not depend on
the host it is built on.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(src=SRC, out=LIB, extra=(), werror=True):
    """Compile `src` into the shared library `out`; raise on failure."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           *(["-Werror"] if werror else []), *extra, "-o", tmp, src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(extra=sys.argv[1:]))
