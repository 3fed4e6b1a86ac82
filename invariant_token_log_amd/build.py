"""Compile the HIP sources into the in-tree shared library for gfx950.

    python -m invariant_token_log_amd.build

Arithmetic is pinned by the flags: no fast-math, no floating-point
contraction (every fused multiply-add in the kernels is an explicit fmaf),
packed-fp32 instruction selection disabled.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libinvariant_logp.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.hip", "logp_kernels.hip", "linear_logp.hip", "linear_bwd.hip"]
# bandwidth probes that bench.py times next to the kernels (not part of the
# library's C ABI)
PROBE_PATH = os.path.join(HERE, "libitl_ceiling.so")
PROBE_SOURCES = ["ceiling.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(sources, out, verbose):
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    # hipcc hands the packed-fp32 feature flag to the host pass too, whose x86
    # backend reports that it does not know it; that line is expected and
    # dropped, anything else the compiler says is shown.
    rest = [ln for ln in res.stderr.splitlines()
            if "-packed-fp32-ops' is not a recognized feature" not in ln]
    if verbose and rest:
        sys.stderr.write("\n".join(rest) + "\n")
    os.replace(tmp, out)
    return out


def build(verbose=False):
    """Compile every HIP source into LIB_PATH, and the bandwidth probes into
    PROBE_PATH (always recompiles)."""
    _compile(SOURCES, LIB_PATH, verbose)
    _compile(PROBE_SOURCES, PROBE_PATH, verbose)
    return LIB_PATH


def asm(out_dir, verbose=False):
    """Write the gfx950 assembly of every source (for reading the code the
    compiler produced: reductions, conversions, absence of contraction)."""
    os.makedirs(out_dir, exist_ok=True)
    for s in SOURCES + PROBE_SOURCES:
        out = os.path.join(out_dir, s.replace(".hip", ".s"))
        cmd = [hipcc(), *[f for f in FLAGS if f not in ("-shared", "-fPIC")],
               "--cuda-device-only", "-S", "-I", INCLUDE, "-I", CSRC,
               os.path.join(CSRC, s), "-o", out]
        subprocess.run(cmd, check=True)
        if verbose:
            print(out)


if __name__ == "__main__":
    print(build(verbose=True))
