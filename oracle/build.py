"""Build the oracle's shared library (test infrastructure only).

    python oracle/build.py            # writes oracle/librmm_oracle.so

Plain gcc, -O2 -ffp-contract=off: every multiply and add rounds on its own,
as written in rmm_oracle.c.  No BLAS, no OpenMP, no threads.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rmm_oracle.c")
LIB = os.path.join(HERE, "librmm_oracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]


def build(src=SRC, out=LIB, extra=()):
    """Compile `src` into the shared library `out`; returns `out`."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)
