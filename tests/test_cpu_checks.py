"""CPU-side checks of the library's host code (no GPU):

* brick index replay: the brick-owned backward's index arithmetic
  (csrc/drr_brick.hpp) compiled for the host with AddressSanitizer and
  UndefinedBehaviorSanitizer and replayed on pinhole cameras against a direct
  scatter (tests/cpu_checks/brick_replay.cpp);
* ABI host validation under ASan/UBSan: the whole library built with the
  sanitizers on its host code, driven by tests/cpu_checks/abi_check.cpp through
  every entry point's invalid and empty calls;
* Siddon brick replay: the brick-owned Siddon backward's walk
  (csrc/drr_siddon.hpp) compiled for the host with the sanitizers, each ray's
  pieces from the bricks against the whole walk, bit for bit
  (tests/cpu_checks/siddon_replay.hip).

Builds go to a temporary directory named by a hash of their inputs, so a
repeated run reuses them.
"""
import hashlib
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHECKS = os.path.join(ROOT, "tests", "cpu_checks")
CSRC = os.path.join(ROOT, "ct_forward_projection_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_INCLUDE = "/opt/rocm/include"


def _build_dir(inputs, tag):
    h = hashlib.sha256(tag.encode())
    for p in sorted(inputs):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + f.read())
    d = os.path.join(tempfile.gettempdir(), f"drr_cpu_checks_{tag}_{h.hexdigest()[:16]}")
    os.makedirs(d, exist_ok=True)
    return d


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    return r.returncode, out


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_brick_index_replay_under_sanitizers():
    src = os.path.join(CHECKS, "brick_replay.cpp")
    d = _build_dir([src] + _sources(), "brick")
    exe = os.path.join(d, "brick_replay")
    if not os.path.exists(exe):
        rc, out = _run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", "-I" + ROCM_INCLUDE,
                        "-D__HIP_PLATFORM_AMD__", src, "-o", exe + ".tmp"])
        assert rc == 0, out
        os.replace(exe + ".tmp", exe)
    rc, out = _run([exe], timeout=300)
    print(out)
    assert rc == 0, out
    assert "all brick index checks passed" in out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_siddon_brick_walk_replay_under_sanitizers():
    """Host build of the Siddon brick walk (no device code): every ray's pieces
    from the brick walks equal the whole walk's, every brick entry is in range,
    and every brick with a piece of a ray finds its pixel among its candidates."""
    src = os.path.join(CHECKS, "siddon_replay.hip")
    d = _build_dir([src] + _sources(), "siddon")
    exe = os.path.join(d, "siddon_replay")
    if not os.path.exists(exe):
        rc, out = _run([HIPCC, "-x", "hip", "--cuda-host-only", "-std=c++17", "-O1", "-g",
                        "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-sanitize-recover=undefined",
                        "-o", exe + ".tmp", src])
        assert rc == 0, out
        os.replace(exe + ".tmp", exe)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    rc, out = _run([exe], timeout=300, env=env)
    print(out)
    assert rc == 0, out
    assert "all Siddon brick checks passed" in out


@pytest.mark.slow
@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_host_validation_under_sanitizers():
    """The library's host code with ASan/UBSan (device code built as usual,
    never launched: every call here fails validation or is empty)."""
    drv = os.path.join(CHECKS, "abi_check.cpp")
    header = os.path.join(ROOT, "include", "drr.h")
    d = _build_dir([drv, header] + _sources(), "abi")
    lib = os.path.join(d, "libdrr_asan.so")
    exe = os.path.join(d, "abi_check")
    hip_sources = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".hip")]
    if not os.path.exists(lib):
        rc, out = _run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fPIC",
                        "-shared", "-munsafe-fp-atomics",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-sanitize-recover=undefined",
                        "-o", lib + ".tmp", *hip_sources])
        assert rc == 0, out
        os.replace(lib + ".tmp", lib)
    if not os.path.exists(exe):
        rc, out = _run([HIPCC, "-std=c++17", "-O1", "-g",
                        "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined",
                        "-o", exe + ".tmp", drv, "-L" + d, "-ldrr_asan", "-Wl,-rpath," + d])
        assert rc == 0, out
        os.replace(exe + ".tmp", exe)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    rc, out = _run([exe], timeout=300, env=env)
    print(out)
    assert rc == 0, out
    assert "all ABI host checks passed" in out
