"""Compile the C oracle into ``oracle/liboracle.so``.

TEST INFRASTRUCTURE: the oracle is the checker for the HIP path, not part of it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "fused_ar_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

# Strict IEEE evaluation: no contraction of a*b+c into an FMA, no reassociation, SSE arithmetic.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-msse2", "-mfpmath=sse", "-Wall", "-Wextra", "-Werror"]


def build(source=SOURCE, output=LIBRARY, extra_flags=()):
    """Compile ``source`` to the shared library ``output`` with gcc; return ``output``."""
    tmp = output + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build())
