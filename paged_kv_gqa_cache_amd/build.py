"""Build libpagedkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_gqa_cache_amd.build [--host-sanitizers]

Compiles every ``csrc/*.hip`` into ``paged_kv_gqa_cache_amd/libpagedkv.so``
(with --host-sanitizers: ``libpagedkv_hostsan.so``, the host code built with
AddressSanitizer and UndefinedBehaviorSanitizer, for the CPU tests).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libpagedkv.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from emitting packed fp32 math on gfx950
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs: no accumulator copies between
    # the AGPR and VGPR files in the tile loops (measured: chunked prefill
    # 317 -> 291 us, decode unchanged)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


# Host-side sanitizer build (a CPU test target): AddressSanitizer and
# UndefinedBehaviorSanitizer on the host code only (argument validation,
# descriptors, launch set-up); the device code is compiled as usual.
HOSTSAN_LIB = os.path.join(HERE, "libpagedkv_hostsan.so")
HOSTSAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = True, host_sanitizers: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = HOSTSAN_LIB if host_sanitizers else LIB
    tmp = out + ".tmp"
    extra = HOSTSAN_FLAGS if host_sanitizers else []
    cmd = [hipcc, *HIPCC_FLAGS, *extra, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(host_sanitizers="--host-sanitizers" in sys.argv[1:])
    sys.exit(0)
