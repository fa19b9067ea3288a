"""Pins of the oracle's LoRA branch (lora_ref).

The branch is (alpha / r) XA B^T with XA = bf16(fp32(x A^T)).  Pinned by:
  * an exact integer case against numpy's integer matmul of the same chain;
  * the pages' composition W = Dequant(Q(W_0)) + (alpha / r) B A: the branch
    equals (alpha / r) x (B A)^T up to the bf16 rounding of XA (a swapped or
    transposed factor fails this);
  * XA itself against fp64 x A^T, within one bf16 rounding.
"""
import numpy as np
import pytest


def test_exact_integer_chain(orc):
    rng = np.random.default_rng(41)
    x = rng.integers(-2, 3, (20, 64)).astype(np.float32)
    a = rng.integers(-1, 2, (16, 64)).astype(np.float32)
    b = rng.integers(-4, 5, (24, 16)).astype(np.float32)
    y, s, xa = orc.lora_ref(x, a, b, 0.125)
    xa_int = x.astype(np.int64) @ a.astype(np.int64).T
    assert np.all(np.abs(xa_int) <= 128)  # |x a| <= 2 * 64: integers exact in bf16
    assert np.array_equal(xa.astype(np.int64), xa_int)
    assert np.array_equal(y, 0.125 * (xa_int @ b.astype(np.int64).T))
    assert np.array_equal(s, 0.125 * (np.abs(xa_int) @ np.abs(b.astype(np.int64)).T))


def test_matches_weight_update_form(orc):
    rng = np.random.default_rng(42)
    M, K, N, r = 40, 256, 48, 32
    x = rng.standard_normal((M, K)).astype(np.float32)
    a = (rng.standard_normal((r, K)) * 0.05).astype(np.float32)
    b = (rng.standard_normal((N, r)) * 0.05).astype(np.float32)
    scale = 16.0 / r
    y, s, xa = orc.lora_ref(x, a, b, scale)
    dW = scale * (b.astype(np.float64) @ a.astype(np.float64))  # (alpha / r) B A, [N, K]
    ref = x.astype(np.float64) @ dW.T
    assert np.all(np.abs(y - ref) <= 2.0 ** -8 * s + 1e-12)


def test_xa_is_one_rounding_from_exact(orc):
    rng = np.random.default_rng(43)
    x = rng.standard_normal((33, 512)).astype(np.float32)
    a = rng.standard_normal((16, 512)).astype(np.float32)
    _, _, xa = orc.lora_ref(x, a, np.ones((8, 16), np.float32), 1.0)
    exact = x.astype(np.float64) @ a.astype(np.float64).T
    assert np.all(np.abs(xa - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-30)


def test_shape_errors(orc):
    with pytest.raises(ValueError):
        orc.lora_ref(np.ones((2, 32), np.float32), np.ones((16, 16), np.float32),
                     np.ones((4, 16), np.float32), 1.0)
