"""Pins of the oracle's NVFP4 quantizer with the Four-Over-Six search (CPU only).

What fixes the oracle here (none of it re-types the oracle's formulas):
  * exact round trip of values already on the E2M1 x E4M3 grid;
  * brute-force optimality: every code is the nearest E2M1 value to x / S
    for its block scale, and the kept candidate has the lower true (fp64)
    squared error wherever the two candidates are not within rounding of a
    tie -- the pages' rule "evaluate 6 and 4, keep the lower-error encoding";
  * the standard (target 6) block scale is torch's nearest-even E4M3 cast
    of amax * s_enc / 6, up to the rounding of that product;
  * invariants: sign symmetry, power-of-two scaling, 2-D on identical rows
    equals 1-D, 2-D of W^T is the transpose of 2-D of W (the reason the
    pages give for 2-D weight scaling), zero tensor;
  * exhaustive small blocks over a value set that produces ties.
"""
import numpy as np
import pytest

import synth
from helpers import e2m1_signed_values, torch_e4m3_encode, torch_e4m3_value, unpack_nibbles

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def cfg1_tensor(seed=1001, rows=4096, cols=128):
    return synth.activations(seed, 0, rows, cols, 0.01, 20.0)


def block_scales_f64(scales, s_dec):
    return torch_e4m3_value(scales).astype(np.float64) * np.float64(s_dec)


def check_nearest_codes(x, codes, S_elem, rel=2e-6):
    """Each element's code is (up to rounding of x * r) the nearest grid point to x/S."""
    nib = unpack_nibbles(codes)
    v = e2m1_signed_values(nib)
    xd = x.astype(np.float64)
    err = np.abs(xd - v * S_elem)
    mag = np.abs(xd)[..., None]
    cand = np.abs(mag - GRID[None, None, :] * S_elem[..., None])
    best = cand.min(axis=-1)
    assert np.all(err <= best + rel * 6 * S_elem + 1e-300)
    # sign bit follows the input's sign
    assert np.array_equal((nib >> 3).astype(bool), np.signbit(x))


def test_round_trip_on_grid(orc):
    rng = np.random.default_rng(5)
    R, Cc = 64, 256
    nb = Cc // 16
    sig_codes = rng.integers(0x08, 0x7F, size=(R, nb)).astype(np.uint8)  # normal E4M3
    sig_codes[0, 0] = 0x7E  # one block at 448 -> tensor amax 6 * 448 = 2688, s_dec = 1
    sig = torch_e4m3_value(sig_codes).astype(np.float32)
    k = rng.integers(0, 8, size=(R, Cc)).astype(np.uint8)
    k.reshape(R, nb, 16)[:, :, 3] = 7  # every block reaches 6 * sigma
    sgn = rng.integers(0, 2, size=(R, Cc)).astype(np.uint8)
    nib = k | (sgn << 3)
    x = (e2m1_signed_values(nib) * np.repeat(sig, 16, axis=1)).astype(np.float32)
    codes, scales, s_dec = orc.quantize(x)
    assert s_dec == 1.0
    assert np.array_equal(scales, sig_codes)
    assert np.array_equal(unpack_nibbles(codes), nib)
    xh = orc.dequantize(codes, scales, s_dec)
    assert np.array_equal(xh.view(np.uint32), x.view(np.uint32))


def test_codes_nearest_and_choice_lower_true_error(orc):
    x = cfg1_tensor()
    codes, scales, s_dec, e6, e4 = orc.quantize(x, return_errors=True)
    S = np.repeat(block_scales_f64(scales, s_dec), 16, axis=1)
    check_nearest_codes(x, codes, S)

    # true fp64 SSE of both candidates, built from torch's E4M3 and the grid
    amax_t = np.abs(x).max()
    s_enc, _ = orc.tensor_scales(amax_t)
    xb = x.reshape(x.shape[0], -1, 16).astype(np.float64)
    amax_b = np.abs(xb).max(axis=-1)
    sse = []
    for c in (6.0, 4.0):
        ideal = (np.float32(amax_b / c) * np.float32(s_enc)).astype(np.float32)
        sc = torch_e4m3_encode(ideal)
        Sc = torch_e4m3_value(sc).astype(np.float64) * np.float64(s_dec)
        y = xb / np.where(Sc > 0, Sc, np.inf)[..., None]
        q = GRID[np.abs(np.abs(y)[..., None] - GRID).argmin(axis=-1)]
        sse.append(((xb - np.sign(xb) * q * Sc[..., None]) ** 2).sum(axis=-1))
    sse6, sse4 = sse
    chose4 = (e4 < e6)
    clear = np.abs(sse4 - sse6) > 1e-4 * np.maximum(sse4, sse6) + 1e-30
    assert clear.mean() > 0.9
    assert np.array_equal(chose4[clear], (sse4 < sse6)[clear])
    assert 0.05 < chose4.mean() < 0.95  # both targets are actually used


def test_standard_scale_is_nearest_e4m3(orc):
    x = cfg1_tensor(seed=1002)
    codes, scales, s_dec = orc.quantize(x, search=orc.SEARCH_6)
    s_enc, _ = orc.tensor_scales(np.abs(x).max())
    amax_b = np.abs(x.reshape(x.shape[0], -1, 16)).max(axis=-1).astype(np.float64)
    exact = amax_b / 6.0 * np.float64(s_enc)
    lo = torch_e4m3_encode((exact * (1 - 1e-6)).astype(np.float32))
    hi = torch_e4m3_encode((exact * (1 + 1e-6)).astype(np.float32))
    assert np.all((scales == lo) | (scales == hi))
    assert np.mean(lo == hi) > 0.99


def test_4o6_total_error_not_worse_than_6(orc):
    x = cfg1_tensor(seed=1003)
    c46, s46, d46 = orc.quantize(x, search=orc.SEARCH_4O6)
    c6, s6, d6 = orc.quantize(x, search=orc.SEARCH_6)
    e46 = ((orc.dequantize(c46, s46, d46).astype(np.float64) - x) ** 2).sum()
    e6 = ((orc.dequantize(c6, s6, d6).astype(np.float64) - x) ** 2).sum()
    assert e46 < e6


def test_sign_symmetry(orc):
    x = cfg1_tensor(seed=1004, rows=512)
    c1, s1, d1 = orc.quantize(x)
    c2, s2, d2 = orc.quantize(-x)
    assert d1 == d2 and np.array_equal(s1, s2)
    assert np.array_equal(c2, c1 ^ 0x88)


@pytest.mark.parametrize("k", [-8, -3, 5, 12])
def test_power_of_two_scaling(orc, k):
    x = cfg1_tensor(seed=1005, rows=512)
    c1, s1, d1 = orc.quantize(x)
    c2, s2, d2 = orc.quantize(np.ldexp(x, k).astype(np.float32))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert d2 == np.float32(np.ldexp(np.float64(d1), k))


def test_zero_tensor(orc):
    x = np.zeros((32, 64), np.float32)
    c, s, d = orc.quantize(x)
    assert d == 1.0 and not c.any() and not s.any()
    c, s, d = orc.quantize(-x)
    assert np.all(c == 0x88) and not s.any()


def test_amax_in_equals_computed(orc):
    x = cfg1_tensor(seed=1006, rows=256)
    a = orc.quantize(x)
    b = orc.quantize(x, amax=float(np.abs(x).max()))
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


def test_exhaustive_small_blocks(orc):
    # Blocks [a, b, c, 0, ..., 0] over a value set rich in E2M1 midpoints at
    # the scales both candidates produce; tensor scale pinned to s_enc = 1.
    vals = np.array([0.0, 0.25, 0.75, 1.0, 1.25, 1.75, 2.5, 3.0, 3.5, 4.0, 4.5, 5.0, 6.0,
                     -0.5, -1.5, -5.0], np.float32) * np.float32(8.0)
    a, b, c = np.meshgrid(vals, vals, vals, indexing="ij")
    x = np.zeros((a.size, 16), np.float32)
    x[:, 0], x[:, 1], x[:, 2] = a.ravel(), b.ravel(), c.ravel()
    codes, scales, s_dec, e6, e4 = orc.quantize(x, amax=2688.0, return_errors=True)
    assert s_dec == 1.0
    S = np.repeat(block_scales_f64(scales, s_dec), 16, axis=1)
    check_nearest_codes(x, codes, S)
    # the kept encoding's true squared error is the smaller candidate error
    e6, e4 = e6.ravel().astype(np.float64), e4.ravel().astype(np.float64)
    xh = orc.dequantize(codes, scales, s_dec).astype(np.float64)
    sse_kept = ((xh - x) ** 2).sum(axis=1)
    assert np.allclose(sse_kept, np.minimum(e6, e4), rtol=1e-6, atol=0)
    assert np.all(e4[e4 < e6] < e6[e4 < e6])
    assert 0 < (e4 < e6).sum() < len(e6)


def test_2d_identical_rows_equals_1d(orc):
    rng = np.random.default_rng(9)
    row = (rng.standard_normal((40, 64)) * 3).astype(np.float32)
    x2 = np.repeat(row[:, None, :], 16, axis=1).reshape(40 * 16, 64)
    c1, s1, d1 = orc.quantize(row)
    c2, s2, d2 = orc.quantize(x2, layout=orc.LAYOUT_2D)
    assert d1 == d2
    assert np.array_equal(s2, s1)
    assert np.array_equal(c2.reshape(40, 16, 32), np.repeat(c1[:, None, :], 16, axis=1))


def test_2d_transpose(orc):
    W = synth.weights(1003, 1, 256, 512)
    cW, sW, dW, e6, e4 = orc.quantize(W, layout=orc.LAYOUT_2D, return_errors=True)
    cT, sT, dT = orc.quantize(np.ascontiguousarray(W.T), layout=orc.LAYOUT_2D)
    assert dW == dT
    same = sT.T == sW
    # a block can only differ when its two candidate errors are within the
    # rounding of the differently ordered error sums
    near_tie = np.abs(e4 - e6) <= 1e-5 * np.maximum(e4, e6)
    assert np.all(same | near_tie)
    nW = unpack_nibbles(cW)
    nT = unpack_nibbles(cT)
    ok = np.repeat(np.repeat(same, 16, axis=0), 16, axis=1)
    assert np.array_equal(nT.T[ok], nW[ok])


def test_2d_codes_nearest(orc):
    W = synth.weights(1003, 2, 512, 256)
    c, s, d = orc.quantize(W, layout=orc.LAYOUT_2D)
    S = np.repeat(np.repeat(block_scales_f64(s, d), 16, axis=0), 16, axis=1)
    check_nearest_codes(W, c, S)


def test_shape_errors(orc):
    with pytest.raises(ValueError):
        orc.quantize(np.zeros((4, 24), np.float32))
    with pytest.raises(ValueError):
        orc.quantize(np.zeros((8, 32), np.float32), layout=orc.LAYOUT_2D)


# Blocks whose two candidates tie exactly, with distinct block scales
# (tensor scale pinned to s_enc = s_dec = 1 by amax = 2688).  Derived by hand:
#   [6, 1.25, 0...]: target 6 gives scale 1.0 (E4M3 0x38), codes 6 -> 0x7,
#     1.25 -> 1.0 (the midpoint of 1 and 1.5 goes to the even code 0x2),
#     error (1/4)^2; target 4 gives scale 1.5 (0x3C), 6 -> 4 * 1.5 (0x6),
#     1.25 * RN(1/1.5) = 0.8333 -> 1.0 * 1.5 (0x2), error (1/4)^2 as well.
#   [6, -3, 1.5, 0...]: both candidates reproduce every value (error 0).
# The rule keeps target 6 on a tie, so both blocks take scale 0x38.
TIE_BLOCKS = [
    ([6.0, 1.25], 0.0625, [0x27] + [0] * 7),
    ([6.0, -3.0, 1.5], 0.0, [0xD7, 0x03] + [0] * 6),
]


def tie_block(vals):
    x = np.zeros((1, 16), np.float32)
    x[0, :len(vals)] = vals
    return x


@pytest.mark.parametrize("vals,err,codes", TIE_BLOCKS, ids=["tie_nonzero", "tie_zero"])
def test_four_over_six_tie_keeps_six(orc, vals, err, codes):
    x = tie_block(vals)
    c, s, d, e6, e4 = orc.quantize(x, amax=2688.0, return_errors=True)
    assert d == 1.0
    assert e6[0, 0] == e4[0, 0] == np.float32(err)
    assert s[0, 0] == 0x38, hex(s[0, 0])
    assert list(c[0]) == codes
    # 2-D: sixteen identical rows tie the same way (tree sums of equal row errors)
    c2, s2, _ = orc.quantize(np.repeat(x, 16, axis=0), layout=orc.LAYOUT_2D, amax=2688.0)
    assert s2[0, 0] == 0x38 and all(list(r) == codes for r in c2)
