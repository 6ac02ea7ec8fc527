"""Compile liblora4.so for gfx950 with hipcc (in-tree, next to this file).

    python -m lora_fine_tuning_amd.build
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "liblora4.so")
SOURCES = [os.path.join(HERE, "csrc", "lora4.hip")]   # includes every csrc/*.hpp
# measured roofline denominators (MFMA rate, HBM read bandwidth), beside the library
PROBE_LIB = os.path.join(HERE, "libpeakprobe.so")
PROBE_SOURCES = [os.path.join(HERE, "csrc", "peak_probe.hip")]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division: the NF4 encoder divides by the block absmax
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-ffp-contract=off",
    "-fvisibility=hidden",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(sources, out, verbose):
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           *sources, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed")
    os.replace(out + ".tmp", out)


def build(verbose=False):
    """Compile the library and the peak probe; returns the library's path.
    Always recompiles."""
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    _compile(SOURCES, LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
