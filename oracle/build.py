"""Builds the C oracle (test infrastructure) with gcc: plain -O2, no FMA
contraction, no fast-math, so each float operation in the source is one
IEEE-754 binary32 operation."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sq_oracle.c")
LIB_PATH = os.path.join(HERE, "libsq_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build() -> str:
    tmp = LIB_PATH + ".tmp"
    subprocess.run(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
