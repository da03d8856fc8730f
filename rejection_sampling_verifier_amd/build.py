"""Build libspecverify.so (HIP kernels + C ABI) for gfx950 in the package directory.

Run ``python -m rejection_sampling_verifier_amd.build``.  hipcc cross-compiles
for gfx950 without a GPU present.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libspecverify.so")
# The compiler's per-kernel resource report (registers, spills, scratch, LDS,
# occupancy) of the last build, written next to the library.
RESOURCES = os.path.join(PKG, "libspecverify.resources.txt")
SOURCES = [os.path.join(PKG, "csrc", "spec_verify.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    # Every floating-point contraction in the kernels is written out
    # explicitly (fmaf); the compiler must not add others.
    "-ffp-contract=off",
    # No packed fp32 instructions (v_pk_*_f32) in generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
    "-I" + os.path.join(PKG, "csrc"),
    "-Rpass-analysis=kernel-resource-usage",
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    with open(RESOURCES, "w") as f:
        f.write(res.stderr)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
