"""Build libnvfp4.so (HIP, gfx950) in-tree with hipcc.

    python -m nvfp4_bit_quantization_amd.build

Every HIP source is compiled for gfx950 only, with fp contraction off (every
fused multiply-add in the kernels is written out explicitly) and with the
packed-fp32 instructions disabled.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libnvfp4.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["quantize.hip", "kv.hip", "gemm.hip", "attn.hip", "capi.cpp", "profile.cpp"]
HEADERS = ["device.hpp", "launch.hpp"]

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    f"-I{os.path.join(ROOT, 'include')}",
]

# Options for one source on top of COMMON.  The W4A4 GEMM runs one wave a
# SIMD (occupancy is fixed by its registers), so the machine scheduler's
# max-ILP strategy costs nothing in waves and interleaves the fp16
# expansion with the MFMAs better (7040 x 3072 x 3072: 105.2-105.5 against
# 108.9-109.2 us a call; no spills in any kernel of the file).
EXTRA = {"gemm.hip": ["-mllvm", "--amdgpu-sched-strategy=max-ilp"]}


def source_hash() -> str:
    """sha256 (first 16 hex digits) of every source, header and build flag the
    library is made from; compiled into the library (nvfp4_build_hash) so
    that a library older than its sources is refused at load time."""
    h = hashlib.sha256()
    for f in SOURCES + HEADERS:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    with open(os.path.join(ROOT, "include", "nvfp4.h"), "rb") as fh:
        h.update(fh.read())
    h.update(" ".join(c for c in COMMON if not c.startswith("-I")).encode())  # no paths
    for f in sorted(EXTRA):
        h.update(("\0" + f + " " + " ".join(EXTRA[f])).encode())
    return h.hexdigest()[:16]


def _compile(src: str, digest: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), f'-DNVFP4_BUILD_HASH="{digest}"', "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l
                    and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    digest = source_hash()
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda src: _compile(src, digest), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    """True if the library is missing or was built from other sources (by
    content, not file times, which a copy of the tree may not keep)."""
    if not os.path.exists(LIB):
        return True
    import ctypes

    try:
        fn = ctypes.CDLL(LIB).nvfp4_build_hash
    except (OSError, AttributeError):
        return True
    fn.restype = ctypes.c_char_p
    return fn().decode() != source_hash()


if __name__ == "__main__":
    print(build(verbose=True))
