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


# The same source under AddressSanitizer and UndefinedBehaviorSanitizer (with
# float-to-integer conversions out of range), every report fatal: the tests
# run the oracle's pins against this build as well (host code only).
SANITIZE = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined,float-cast-overflow",
            "-fno-sanitize-recover=all"]


def build() -> str:
    tmp = LIB_PATH + ".tmp"
    subprocess.run(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build_sanitized(path: str) -> str:
    flags = [f for f in CFLAGS if f != "-O2"] + SANITIZE
    subprocess.run(["gcc", *flags, SRC, "-o", path, "-lm"], check=True)
    return path


if __name__ == "__main__":
    print(build())
