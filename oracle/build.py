"""Compile the CPU oracle (test infrastructure only) into oracle/libsdm_oracle.so.

Plain gcc, no FMA contraction, no fast-math: each fp32 operation in
sdm_oracle.c is one IEEE-754 binary32 operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sdm_oracle.c")
LIB = os.path.join(HERE, "libsdm_oracle.so")

CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fno-builtin-expf",
          "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(force: bool = True, extra_flags=(), out: str = LIB) -> str:
    """Build the oracle library (at `out`, by default oracle/libsdm_oracle.so);
    returns its path."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(SRC):
        return out
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(force=True, extra_flags=sys.argv[1:]))
