"""Pins of the oracle's random Hadamard transform (rht16).

The transform is y = (1/4) H16 diag(s) x per 1x16 block (H16 Sylvester,
H[i][j] = (-1)^popcount(i & j)), computed by the fp32 butterfly.  Pinned by:
  * the matrix definition, exactly, on integer data (no rounding anywhere);
  * the fp64 matrix product on random data, within the butterfly's fp32
    error bound;
  * the inverse: x = diag(s) * rht16(y, no signs) exactly on integer data;
  * Parseval, and the invariance of A W^T when both operands are
    transformed along K.
"""
import numpy as np

H16 = np.array([[(-1.0) ** bin(i & j).count("1") for j in range(16)] for i in range(16)])


def rht_def(x, signs):
    """fp64 matrix definition, per 16-column block."""
    s = np.array([-1.0 if (signs >> j) & 1 else 1.0 for j in range(16)])
    R, C = x.shape
    xb = x.astype(np.float64).reshape(R, C // 16, 16) * s
    return (0.25 * np.einsum("ij,rbj->rbi", H16, xb)).reshape(R, C)


def test_hadamard_matrix_is_orthogonal():
    assert np.array_equal(H16 @ H16.T, 16 * np.eye(16))


def test_matches_definition_exactly_on_integers(orc):
    rng = np.random.default_rng(31)
    x = rng.integers(-1000, 1000, (64, 128)).astype(np.float32)
    for signs in (0, 0xFFFF, 0x5A3C, int(rng.integers(0, 1 << 16))):
        assert np.array_equal(orc.rht16(x, signs).astype(np.float64), rht_def(x, signs))


def test_within_butterfly_error_bound(orc):
    rng = np.random.default_rng(32)
    x = (rng.standard_normal((128, 256)) * np.exp2(rng.integers(-20, 20, (128, 256)))).astype(np.float32)
    signs = 0xB7E1
    y = orc.rht16(x, signs).astype(np.float64)
    ref = rht_def(x, signs)
    # 4 rounded additions along every path, each |error| <= 2^-24 |partial|,
    # partials bounded by the block's sum of |x|; the final * 0.25 is exact
    bound = 4 * 2.0 ** -24 * 0.25 * np.repeat(np.abs(x.astype(np.float64)).reshape(128, 16, 16).sum(2), 16, axis=1)
    assert np.all(np.abs(y - ref) <= bound + 1e-300)


def test_inverse_recovers_input(orc):
    rng = np.random.default_rng(33)
    x = (rng.integers(-4096, 4096, (32, 64)) * 4).astype(np.float32)
    signs = 0x93C5
    y = orc.rht16(x, signs)
    back = orc.rht16(y, 0)  # (1/4) H (1/4) H S x = S x
    s = np.tile(np.array([-1.0 if (signs >> j) & 1 else 1.0 for j in range(16)], np.float32), 4)
    assert np.array_equal(back * s, x)


def test_parseval_and_product_invariance(orc):
    rng = np.random.default_rng(34)
    a = rng.standard_normal((48, 512)).astype(np.float32)
    w = rng.standard_normal((40, 512)).astype(np.float32)
    signs = 0x2D4B
    ya, yw = orc.rht16(a, signs), orc.rht16(w, signs)
    assert np.allclose((ya.astype(np.float64) ** 2).sum(1), (a.astype(np.float64) ** 2).sum(1), rtol=1e-5)
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    got = ya.astype(np.float64) @ yw.astype(np.float64).T
    assert np.allclose(got, ref, rtol=0, atol=1e-4 * np.abs(ref).max())
