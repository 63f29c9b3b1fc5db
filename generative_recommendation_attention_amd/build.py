"""Builds libhstu.so (the HIP library behind include/hstu.h) for gfx950.

    python -m generative_recommendation_attention_amd.build

Every source is compiled by hipcc into one shared library next to this file.
Packed fp32 VALU instructions are disabled for device code
(-target-feature -packed-fp32-ops); the host pass warns that it does not know
the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libhstu.so")
SOURCES = ["api.cpp", "schedule.hip", "attn_fwd.hip", "attn_bwd.hip", "layer.hip", "noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def command(output: str = LIBRARY, extra=()) -> list:
    return ([hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]
            + list(extra) + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", output])


def build(output: str = LIBRARY, verbose: bool = False) -> str:
    tmp = output + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    build(verbose=True)
    print(LIBRARY)
    sys.exit(0)
