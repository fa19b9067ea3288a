"""Pins of the oracle's W4A4 GEMM reference (CPU only)."""
import numpy as np

import synth
from helpers import e2m1_signed_values, torch_e4m3_value, unpack_nibbles


def test_exact_integer_case(orc):
    # all block scales 1.0 (E4M3 0x38) and s_dec = 1: every product is a
    # multiple of 1/4, so 4*y is an integer matmul of 2*V values
    rng = np.random.default_rng(1)
    M, N, K = 48, 32, 160
    a = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    w = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa = np.full((M, K // 16), 0x38, np.uint8)
    sw = np.full((N // 16, K // 16), 0x38, np.uint8)
    y, s = orc.gemm_ref(a, sa, 1.0, w, sw, 1.0)
    ai = (2 * e2m1_signed_values(unpack_nibbles(a))).astype(np.int64)
    wi = (2 * e2m1_signed_values(unpack_nibbles(w))).astype(np.int64)
    assert np.array_equal(y * 4, (ai @ wi.T).astype(np.float64))
    assert np.array_equal(s * 4, (np.abs(ai) @ np.abs(wi).T).astype(np.float64))


def test_matches_float64_matmul_of_dequantized(orc):
    A = synth.activations(1001, 5, 64, 512, 0.01, 20.0)
    W = synth.activations(1001, 6, 96, 512, 0.01, 20.0)
    ca, sa, da = orc.quantize(A)
    cw, sw, dw = orc.quantize(W, layout=orc.LAYOUT_2D)
    y, s = orc.gemm_ref(ca, sa, da, cw, sw, dw)
    Ah = e2m1_signed_values(unpack_nibbles(ca)) * np.repeat(torch_e4m3_value(sa), 16, axis=1)
    Wh = e2m1_signed_values(unpack_nibbles(cw)) * np.repeat(np.repeat(torch_e4m3_value(sw), 16, 0), 16, 1)
    ref = (Ah @ Wh.T) * (np.float64(da) * np.float64(dw))
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert np.all(s + 1e-9 >= np.abs(y))


def test_rows_subset(orc):
    A = synth.activations(1001, 7, 40, 64, 0.01, 20.0)
    W = synth.weights(1001, 8, 32, 64)
    ca, sa, da = orc.quantize(A)
    cw, sw, dw = orc.quantize(W, layout=orc.LAYOUT_2D)
    y, _ = orc.gemm_ref(ca, sa, da, cw, sw, dw)
    rows = np.array([39, 0, 17])
    y2, _ = orc.gemm_ref(ca, sa, da, cw, sw, dw, rows=rows)
    assert np.array_equal(y2, y[rows])
