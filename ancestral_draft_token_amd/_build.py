"""Build the HIP library in-tree for gfx950 (MI355X).

``hipcc`` cross-compiles without a GPU. The library is one shared object
built from ``csrc/dspark.hip`` (the sampler and verification) and
``csrc/window_attn.hip`` (the drafter's windowed block attention),
``ancestral_draft_token_amd/libdspark.so``, exporting the C ABI declared in
``include/dspark.h``.
"""

from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "dspark.hip")
SOURCES = [SRC, os.path.join(PKG, "csrc", "window_attn.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdspark.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # the bit-for-bit logits/T recompute needs every float op rounded on its own
    "-ffp-contract=off",
    # no packed-FP32 instructions: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the library's only atomics (a workgroup's arrival, a failure record) run
    # on one thread; the backend's combining of atomics across a wave would
    # make each wait at once for its result, and so for every load issued
    # before it (the W stream of the resident kernels' setup)
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build_library(out: str = LIB, extra_flags=()) -> str:
    """Compile the sources under ``csrc/`` into ``out`` (always recompiles)."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, f"-I{INCLUDE}", "-o", tmp, *SOURCES]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library())
