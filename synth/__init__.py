"""Seeded synthetic inputs for the NVFP4 data path.

This module holds random-number generation only: no step of the
quantization method lives here.  Both the CPU oracle's tests and the GPU
path's tests and benchmark draw their inputs from it, so the two sides see
the same bytes.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used counter-style: output i of stream
``key`` is ``mix(key + (i + 1) * GOLDEN)``.  Uniforms take the top 53 bits;
normals come from the Box-Muller transform (cosine branch only), so every
element is a pure function of (key, index) and any sub-range can be drawn
on its own.

The workload shapes follow the LongLive-2.0 pages (880 tokens per latent
frame, 8 frames per chunk, 24 heads of width 128, model width 3072); the
value distributions (unit normals with sparse x20 / x30 outliers, a
per-channel key bias, N(0, 0.02^2) weights) are the stated synthetic recipe.
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Stream ids: one sub-stream per operand so operands never share draws.
STREAM_VALUES = 1
STREAM_OUTLIER_MASK = 2
STREAM_CHANNEL_BIAS = 3
STREAM_BM_U2 = 4


def _mix(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def stream_key(seed: int, operand: int, stream: int) -> np.uint64:
    """Derive a 64-bit stream key from (seed, operand id, stream id)."""
    base = np.array([(seed * 1_000_003 + operand * 7919 + stream) & 0xFFFFFFFFFFFFFFFF],
                    dtype=np.uint64)
    return _mix(base)[0]


def raw_u64(key: np.uint64, start: int, n: int) -> np.ndarray:
    idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(np.uint64(key) + idx * GOLDEN)


def uniform(key: np.uint64, start: int, n: int) -> np.ndarray:
    """Uniform doubles in [0, 1) with 53 random bits."""
    return (raw_u64(key, start, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(seed: int, operand: int, n: int, start: int = 0) -> np.ndarray:
    """N(0, 1) doubles by Box-Muller (cos branch)."""
    u1 = 1.0 - uniform(stream_key(seed, operand, STREAM_VALUES), start, n)  # (0, 1]
    u2 = uniform(stream_key(seed, operand, STREAM_BM_U2), start, n)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def outlier_mask(seed: int, operand: int, n: int, p: float, start: int = 0) -> np.ndarray:
    """Independent Bernoulli(p) draw per element."""
    return uniform(stream_key(seed, operand, STREAM_OUTLIER_MASK), start, n) < p


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits.

    Input-side rounding only: the generator hands bf16 tensors to both
    sides, so this is part of producing the input, not of the method.
    """
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b16: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Workload recipes
# ---------------------------------------------------------------------------

def activations(seed: int, operand: int, rows: int, cols: int, p_out: float, out_scale: float) -> np.ndarray:
    """float32 [rows, cols]: N(0,1) with a Bernoulli(p_out) subset scaled by out_scale."""
    n = rows * cols
    x = normal(seed, operand, n)
    m = outlier_mask(seed, operand, n, p_out)
    x[m] *= out_scale
    return x.astype(np.float32).reshape(rows, cols)


def weights(seed: int, operand: int, rows: int, cols: int, std: float = 0.02) -> np.ndarray:
    """float32 [rows, cols] ~ N(0, std^2)."""
    return (normal(seed, operand, rows * cols) * std).astype(np.float32).reshape(rows, cols)


def kv_chunk(seed: int, chunk: int, tokens: int, heads: int, head_dim: int, token_start: int = 0,
             threads: int = 1):
    """One KV chunk as bf16 bit arrays [tokens, heads, head_dim].

    K = N(0,1) + bias[c], bias ~ N(0, 4) drawn once per channel c of the head
    dimension and shared by all heads and chunks (channel outliers).
    V = N(0,1).  ``token_start`` lets a caller draw a sub-range of tokens
    (the same values the full chunk would hold there).  ``threads`` > 1 draws
    token ranges on that many threads (numpy releases the GIL in its array
    loops); every element is a function of its index, so the result is the
    same.
    """
    if threads > 1 and tokens >= 2 * threads:
        from concurrent.futures import ThreadPoolExecutor

        cuts = [tokens * i // threads for i in range(threads + 1)]
        with ThreadPoolExecutor(threads) as ex:
            parts = list(ex.map(lambda i: kv_chunk(seed, chunk, cuts[i + 1] - cuts[i], heads,
                                                   head_dim, token_start + cuts[i]),
                                range(threads)))
        return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))
    hd = heads * head_dim
    bias = normal(seed, 999, head_dim) * 2.0
    start = token_start * hd
    n = tokens * hd
    k = normal(seed, 2 * chunk + 10, n, start).reshape(tokens, heads, head_dim) + bias[None, None, :]
    v = normal(seed, 2 * chunk + 11, n, start).reshape(tokens, heads, head_dim)
    return to_bf16_bits(k.astype(np.float32)), to_bf16_bits(v.astype(np.float32))


def host_threads() -> int:
    """Worker threads for host-side generation and the oracle: the CPUs this
    process may run on, at most 16."""
    import os

    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# Shapes of the LongLive-2.0 5B model as used by the workloads.
TOKENS_PER_FRAME = 880
FRAMES_PER_CHUNK = 8
HEADS = 24
HEAD_DIM = 128
D_MODEL = 3072
D_FFN = 14336
CHUNK_TOKENS = TOKENS_PER_FRAME * FRAMES_PER_CHUNK  # 7040
