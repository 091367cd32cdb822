"""Build libsbl.so (all HIP kernels + the C ABI) in-tree for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsbl.so")
# SBL_SANITIZE=1: the host code (argument checks, launch set-up, caches) is
# built with AddressSanitizer and UndefinedBehaviorSanitizer into
# libsbl_san.so, which the binding then loads; device code is unchanged.
# Run Python with the clang ASan runtime preloaded (see SANITIZE_RUNTIME).
SANITIZE = os.environ.get("SBL_SANITIZE") == "1"
LIB_SAN = os.path.join(HERE, "libsbl_san.so")
SANITIZE_RUNTIME = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # every float operation is its own IEEE operation: no contraction into FMA
    "-ffp-contract=off",
    # keep the compiler from emitting packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, sanitize: bool = SANITIZE) -> str:
    out = LIB_SAN if sanitize else LIB
    san = []
    if sanitize:
        san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    cmd = [HIPCC, *FLAGS, *san, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *sources(), "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature: drop that warning
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
