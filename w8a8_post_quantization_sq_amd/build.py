"""Builds libsq.so (the HIP library behind include/sq.h) and libsq_probe.so (the
benchmark's measured ceilings, include/sq_probe.h) in-tree for gfx950.

Flags:
  --offload-arch=gfx950                  CDNA4 / MI355X only
  -O3 -ffp-contract=off                  no FMA contraction of the float sequences
                                         that decide int8 codes (there are none
                                         to contract today; this keeps it so)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                         no packed fp32 instructions
  -mllvm -amdgpu-mfma-vgpr-form=1        matrix-core accumulators in arch VGPRs: the
                                         product's working set fits the 256 VGPRs
                                         without accumulator copies in its loop
  -fvisibility=hidden                    only the extern "C" sq_* symbols export
The compiler's default IEEE-correct float division and sqrt are kept (no
fast-math).
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libsq.so")

PROBE_PATH = os.path.join(HERE, "libsq_probe.so")
PROBE_SOURCES = ["probe.hip"]

SOURCES = ["sq_api.cpp", "k_calib.hip", "k_fold.hip", "k_quant.hip", "k_gemm.hip", "k_pack.hip",
           "k_rot.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def _compile(sources, out: str, verbose: bool) -> str:
    srcs = []
    for s in sources:
        p = os.path.join(CSRC, s)
        # .cpp sources are host code; .hip sources carry the kernels
        srcs += (["-x", "hip", p, "-x", "none"] if s.endswith(".hip") else [p])
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Builds libsq.so (the layer) and libsq_probe.so (the benchmark's
    measured ceilings); returns the path of libsq.so."""
    _compile(PROBE_SOURCES, PROBE_PATH, verbose)
    return _compile(SOURCES, LIB_PATH, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
