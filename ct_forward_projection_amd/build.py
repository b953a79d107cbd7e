"""Build libdrr.so in-tree with hipcc for gfx950.

Flags: -O3; hardware float atomics for the backward scatter
(-munsafe-fp-atomics); packed-FP32 instruction selection switched off for the
device code (-Xclang -target-feature -Xclang -packed-fp32-ops; the host pass
warns that it does not know the feature, which is harmless).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libdrr.so")
SOURCES = [os.path.join(CSRC, "drr_kernels.hip"), os.path.join(CSRC, "drr_pose.hip"),
           os.path.join(CSRC, "drr_siddon.hip"), os.path.join(CSRC, "drr_camera.hip"),
           os.path.join(CSRC, "drr_noise.hip"), os.path.join(CSRC, "drr_brick.hip"),
           os.path.join(CSRC, "drr_abi.hip")]
HEADERS = [os.path.join(CSRC, "drr_device.hpp"), os.path.join(CSRC, "drr_internal.hpp"),
           os.path.join(CSRC, "drr_sample.hpp"), os.path.join(CSRC, "drr_stage.hpp"),
           os.path.join(CSRC, "drr_window.hpp"), os.path.join(CSRC, "drr_brick.hpp"),
           os.path.join(os.path.dirname(HERE), "include", "drr.h")]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
         "-munsafe-fp-atomics", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall"]


def build(verbose: bool = False) -> str:
    tmp = LIBRARY + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def is_stale() -> bool:
    if not os.path.exists(LIBRARY):
        return True
    t = os.path.getmtime(LIBRARY)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
