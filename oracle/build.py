"""Build the C oracle into ``oracle/liboracle.so`` (test infrastructure only).

Plain gcc, fp64, OpenMP over chains, no fast-math.  Nothing here is shared
with the HIP library.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "la2_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def compile_oracle(src=SRC, out=LIB, extra_flags=()):
    """Compile ``src`` to the shared library ``out`` and return its path."""
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(compile_oracle(), file=sys.stderr)
