"""Build the CPU oracle shared library (test infrastructure only).

gcc -O2 -ffp-contract=off: GCC's default in GNU C mode contracts a*b+c into
fused multiply-adds, which would change the rounding of the fixed order; the
oracle writes every fused multiply-add it wants as fmaf().  No -ffast-math:
it links FTZ/DAZ start-up code and reorders sums.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared",
          "-fvisibility=hidden", "-Wall", "-Wextra", "-Wno-unused-parameter", "-pthread"]


def build(src=SRC, out=LIB, extra_flags=(), quiet=False):
    """Compile `src` into the shared library `out`; returns `out`."""
    cmd = ["gcc", *CFLAGS, *extra_flags, src, "-o", out + ".tmp", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    if res.stderr and not quiet:
        sys.stderr.write(res.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
