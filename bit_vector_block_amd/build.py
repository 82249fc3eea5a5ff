"""Build libsift.so in-tree with hipcc for gfx950 (always recompiles)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["sift_api.hip", "decode_kernels.hip", "prepare_kernels.hip", "prefill_kernels.hip", "encode_kernels.hip"]
OUT = os.path.join(HERE, "libsift.so")
# the MFMA throughput probe bench.py measures the attention kernel against (not the prefill path)
PROBE_SOURCES = ["mfma_probe.hip"]
PROBE_OUT = os.path.join(HERE, "libsift_probe.so")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # packed fp32 VALU ops stay off for every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(sources, out, verbose):
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in sources], "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False) -> str:
    _compile(SOURCES, OUT, verbose)
    _compile(PROBE_SOURCES, PROBE_OUT, verbose)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
