"""Shared test utilities: independent formulations used to pin the oracle.

Nothing here is imported by the oracle or by the GPU library.
"""
from __future__ import annotations

import os
import subprocess
import tempfile

import numpy as np
import torch

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def dense_f32_patterns(low_bits=(0x000, 0x001, 0xFFF), signs=(0, 1), max_exp=255) -> np.ndarray:
    """Every float32 whose low 12 mantissa bits are in ``low_bits``.

    The high 11 mantissa bits and the exponent run over all values, so the
    set holds every rounding midpoint of any format with <= 10 mantissa bits
    together with its neighbours one ulp either side.
    """
    hi = np.arange(0, 1 << 19, dtype=np.uint32)  # 8 exponent + 11 mantissa bits
    hi = hi[(hi >> 11) < max_exp]  # drop inf/NaN exponents unless asked
    out = []
    for s in signs:
        for lb in low_bits:
            out.append((np.uint32(s) << np.uint32(31)) | (hi << np.uint32(12)) | np.uint32(lb))
    return np.concatenate(out).view(np.float32)


def e2m1_by_thresholds(y: np.ndarray) -> np.ndarray:
    """E2M1 code from the rounding midpoints of the grid {0,.5,1,1.5,2,3,4,6}.

    Hand-derived: a midpoint between an even and an odd code goes to the even
    code, so the comparison is <= where the lower neighbour is even and <
    where it is odd.  Independent of the oracle's nearest-by-distance search.
    """
    a = np.abs(y.astype(np.float64))
    k = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5)
         + (a >= 3.5) + (a > 5.0)).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << 3
    return sign | k


def torch_e4m3_encode(t: np.ndarray) -> np.ndarray:
    """torch's float32 -> float8_e4m3fn cast (nearest-even), as code bytes."""
    return torch.from_numpy(np.ascontiguousarray(t, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def torch_e4m3_value(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float32).numpy()


def torch_bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_signed_values(nibbles: np.ndarray) -> np.ndarray:
    """Signed value of E2M1 nibbles from the bit layout (1 sign, 2 exp bias 1, 1 mantissa)."""
    k = (nibbles & 7).astype(np.int64)
    e = k >> 1
    m = k & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int32)))
    return np.where(nibbles & 8, -mag, mag)


def unpack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[R, C/2] bytes -> [R, C] nibbles (even column in the low nibble)."""
    lo = codes & 0xF
    hi = codes >> 4
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


_rocm_lib = None


def rocm_host_converters():
    """ctypes handle on ROCm's host-side OCP E2M1/E4M3 converters (header
    library amd_hip_ocp_host.hpp), built here with amdclang++ in host-only
    mode, or None if that is not possible."""
    global _rocm_lib
    if _rocm_lib is not None:
        return _rocm_lib
    import ctypes

    src = r'''
#include <cstdint>
#include <hip/amd_detail/amd_hip_ocp_host.hpp>
extern "C" void rocm_e2m1(const float* x, long n, uint8_t* out) {
  for (long i = 0; i < n; ++i) out[i] = (uint8_t)fcbx::from_float<float, fcbx::Encoding::E2M1, true>(x[i], 0);
}
extern "C" void rocm_e4m3(const float* x, long n, uint8_t* out) {
  for (long i = 0; i < n; ++i) out[i] = (uint8_t)fcbx::from_float<float, fcbx::Encoding::E4M3, true>(x[i], 0);
}
'''
    d = tempfile.mkdtemp(prefix="ocp_host_")
    cpp = os.path.join(d, "ocp.cpp")
    so = os.path.join(d, "ocp.so")
    with open(cpp, "w") as f:
        f.write(src)
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    r = subprocess.run([clang, "-O2", "-std=c++17", "-shared", "-fPIC", "-x", "hip",
                        "--cuda-host-only", f"-I{ROCM}/include", "-o", so, cpp],
                       capture_output=True)
    if r.returncode != 0:
        return None
    L = ctypes.CDLL(so)
    for fn in (L.rocm_e2m1, L.rocm_e4m3):
        fn.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p]
        fn.restype = None
    _rocm_lib = L
    return L


def rocm_encode(fn_name: str, x: np.ndarray) -> np.ndarray:
    L = rocm_host_converters()
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    getattr(L, fn_name)(x.ctypes.data, x.size, out.ctypes.data)
    return out


def kmean_fp64_exact(K: np.ndarray) -> bool:
    """True if, for every channel (column) of K, a sum of its values in double
    is exact in any order: each nonzero value is an odd multiple of 2^k for
    some k >= k_min, so every partial sum is an integer multiple of 2^k_min
    no larger in magnitude than sum |v|; below 2^53 * 2^k_min such a multiple
    is a double.  (The kernels' key-mean sums are exact, and so equal the
    oracle's exact mean, on such inputs.)"""
    K = np.ascontiguousarray(K, np.float32)
    u = K.view(np.uint32)
    be = ((u >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int32)
    M = (u & np.uint32(0x7FFFFF)).astype(np.int32)
    M |= np.where(be > 0, np.int32(0x800000), np.int32(0))  # value = +-M * 2^(max(be, 1) - 150)
    low = M & -M                                           # lowest set bit of M (a power of two)
    lexp = (low.astype(np.float32).view(np.int32) >> 23) - 127
    k = np.where(M != 0, lexp + np.maximum(be, 1) - 150, np.int32(1 << 20))
    kmin = k.min(axis=0).astype(np.int64)
    s = np.abs(K).sum(axis=0, dtype=np.float64) * (1.0 + 1e-9)
    return bool(np.all(s < np.ldexp(1.0, np.minimum(53 + kmin, 1000))))
