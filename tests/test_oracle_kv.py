"""Pins of the oracle's KV-cache path: K-smoothing, chunk storage, the
multi-shot effective set and the gather (CPU only)."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(v) for v in line.split()])
    return rows


def small_chunk(seed=2002, T=200, H=3, d=32):
    k, v = synth.kv_chunk(seed, 0, T, H, d)
    K = synth.bf16_bits_to_f32(k).reshape(T, H * d)
    V = synth.bf16_bits_to_f32(v).reshape(T, H * d)
    return K, V


def test_storage_formula_golden(orc):
    (T, H, d, bf16_bytes, nvfp4_bytes, rn, rd), = read_golden("kv_storage.txt")
    assert bf16_bytes == 4 * T * H * d
    # bytes actually produced by the oracle for one chunk: codes + scales of K and V
    K, V = small_chunk(T=64, H=H, d=d)
    ch = orc.kv_encode_chunk(K, V)
    per_token = sum(ch[k].nbytes for k in ("kc", "ks", "vc", "vs")) // 64
    assert per_token * T == nvfp4_bytes
    assert nvfp4_bytes * 8 == 9 * T * H * d
    assert bf16_bytes * rd == nvfp4_bytes * rn  # 32/9 = 3.56, the pages' "about 3.6x"
    assert round(bf16_bytes / nvfp4_bytes, 1) == 3.6


def mean_rn64_rn32(col):
    """(float)RN64(S / T) with S the exact sum, by Python's exact rationals:
    Fraction(float) is exact, int / int true division (Fraction.__float__)
    is correctly rounded to double, numpy's float32 cast rounds to nearest."""
    s = sum((Fraction(float(v)) for v in col), Fraction(0))
    return np.float32(float(s / len(col)))


def test_kv_mean_exact(orc):
    K, _ = small_chunk(T=300)
    mu = orc.kv_mean(K)
    for ch in range(K.shape[1]):
        exact = math.fsum(float(v) for v in K[:, ch]) / K.shape[0]
        # mu is the double quotient rounded to float: within one float ulp of exact
        assert abs(float(mu[ch]) - exact) <= np.spacing(np.float32(abs(exact)))
        assert mu[ch] == mean_rn64_rn32(K[:, ch])


def test_kv_mean_wide_binades_equals_rational(orc):
    """Values over 200 binades, subnormals and cancellations: the naive double
    sum is inexact there, the oracle's mean is still the exact one."""
    rng = np.random.default_rng(4)
    T = 257
    K = (rng.standard_normal((T, 8)) * np.exp2(rng.integers(-100, 100, (T, 8)))).astype(np.float32)
    K[::7, 1] = np.float32(2.0 ** -149) * rng.integers(1, 50, K[::7, 1].shape)  # subnormals
    K[:, 2] = np.where(np.arange(T) % 2 == 0, np.float32(3e38), np.float32(-3e38))
    K[5, 2] = np.float32(1e-30)  # a tiny survivor of a huge cancellation
    K[:, 3] = 0.0
    K[:, 4] = np.float32(-1.5e-7)
    mu = orc.kv_mean(K)
    for ch in range(8):
        assert mu[ch] == mean_rn64_rn32(K[:, ch]), ch
    assert mu[3] == 0.0 and mu[4] == np.float32(-1.5e-7)
    # 129 values +3e38 (even tokens), 127 values -3e38 and one 1e-30 (token 5):
    # 2 * 3e38 + 1e-30 over 257 tokens is what is left
    big, tiny = Fraction(float(np.float32(3e38))), Fraction(float(np.float32(1e-30)))
    assert mu[2] == np.float32(float((2 * big + tiny) / T))


def test_kv_mean_order_free(orc):
    """Permuting the tokens leaves every mean bit-identical, on data where
    sequential double sums in the two orders differ."""
    rng = np.random.default_rng(5)
    T = 301
    K = (rng.standard_normal((T, 16)) * np.exp2(rng.integers(-60, 60, (T, 16)))).astype(np.float32)
    perm = rng.permutation(T)
    mu, mu_p = orc.kv_mean(K), orc.kv_mean(np.ascontiguousarray(K[perm]))
    assert np.array_equal(mu.view(np.uint32), mu_p.view(np.uint32))
    seq = lambda col: sum(float(v) for v in col)
    assert any(seq(K[:, c]) != seq(K[perm, c]) for c in range(16))


def test_kv_mean_closed_forms(orc):
    # constant channel: the mean is the value; +-a pairs: zero; 1, 1, 2: 4/3
    K = np.zeros((6, 4), np.float32)
    K[:, 0] = np.float32(0.3)
    K[:, 1] = [5.0, -5.0, 2.5, -2.5, 1e-3, -1e-3]
    K[:3, 2] = [1.0, 1.0, 2.0]
    K[3:, 2] = [1.0, 1.0, 2.0]
    K[:, 3] = [2.0 ** 60, 1.0, -(2.0 ** 60), 2.0, 0.0, 0.0]  # naive left-to-right: (0 + 2) / 6
    mu = orc.kv_mean(K)
    assert mu[0] == np.float32(0.3)
    assert mu[1] == 0.0
    assert mu[2] == np.float32(4.0 / 3.0)
    assert mu[3] == np.float32(0.5)


def test_kv_mean_rounds_to_double_then_float(orc):
    """The double rounding of the reading: S / T = 1 + 2^-24 + 2^-60/3 rounds
    to the double 1 + 2^-24, an exact float midpoint, which rounds to the even
    float 1.0 (one direct rounding to float would give 1 + 2^-23)."""
    vals = np.array([2.0 + 2.0 ** -22, 1.0 - 2.0 ** -24, 2.0 ** -60], np.float32)
    assert (Fraction(float(vals[0])) + Fraction(float(vals[1])) + Fraction(float(vals[2]))
            == Fraction(3) + Fraction(3, 2 ** 24) + Fraction(1, 2 ** 60))
    mu = orc.kv_mean(vals.reshape(3, 1))
    assert mu[0] == np.float32(1.0)


def test_fp64_exactness_domain_checker():
    """The test-side check that a key chunk lies where a double sum in any
    order is exact (every partial sum a multiple of the smallest ulp, below
    2^53 of them)."""
    from helpers import kmean_fp64_exact

    ok = np.array([[1.0, 3.0], [2.0 ** -20, -7.5]], np.float32)
    assert kmean_fp64_exact(ok)
    bad = np.array([[2.0 ** 40, 1.0], [2.0 ** -30, 1.0]], np.float32)  # 70 bits in channel 0
    assert kmean_fp64_exact(np.array([[2.0 ** 20], [2.0 ** -30]], np.float32))  # 50 bits
    assert not kmean_fp64_exact(bad)
    # the 64 s ring's first chunk is inside
    k, _ = synth.kv_chunk(1005, 0, 7040, 24, 128)
    assert kmean_fp64_exact(synth.bf16_bits_to_f32(k).reshape(7040, -1))


def test_smoothed_keys_have_zero_mean_and_amax_shortcut(orc):
    K, V = small_chunk(T=512)
    mu = orc.kv_mean(K)
    Ks = (K - mu[None, :]).astype(np.float32)
    assert np.all(np.abs(Ks.astype(np.float64).mean(axis=0)) <= 1e-6 * np.abs(K).max())
    # amax of RN(K - mu) elementwise equals the per-channel max/min shortcut
    kmax, kmin = K.max(axis=0), K.min(axis=0)
    short = np.maximum((kmax - mu).astype(np.float32), (mu - kmin).astype(np.float32)).max()
    assert np.abs(Ks).max() == short


def test_chunk_roundtrip_error_bound(orc):
    K, V = small_chunk(T=256)
    ch = orc.kv_encode_chunk(K, V)
    Kh = synth.bf16_bits_to_f32(orc.kv_dequant_tokens(ch, 0, 256, key=True))
    Vh = synth.bf16_bits_to_f32(orc.kv_dequant_tokens(ch, 0, 256, key=False))
    # NVFP4 relative step is at most 1/2 of the block max scale (grid gap 2 near 6)
    for X, Xh in ((K, Kh), (V, Vh)):
        xb = X.reshape(256, -1, 16)
        err = np.abs(Xh - X).reshape(256, -1, 16).max(axis=-1)
        bound = np.abs(xb - (K.mean(axis=0).reshape(1, -1, 16) if X is K else 0)).max(axis=-1) / 6 * 1.01 + 0.02
        assert np.all(err <= bound * 1.0 + 1e-3)
    # keys: smoothing helps -- error of K with the per-channel bias removed is
    # far below quantizing the raw keys
    raw = orc.quantize(K)
    e_raw = np.abs(orc.dequantize(*raw) - K).mean()
    assert np.abs(Kh - K).mean() < 0.8 * e_raw


def test_dequant_tokens_matches_dequantize(orc):
    K, V = small_chunk(T=64)
    ch = orc.kv_encode_chunk(K, V)
    xv = orc.dequantize(ch["vc"], ch["vs"], ch["sdv"])
    assert np.array_equal(orc.kv_dequant_tokens(ch, 0, 64, key=False), orc.bf16_rne(xv))
    xk = orc.dequantize(ch["kc"], ch["ks"], ch["sdk"])
    assert np.array_equal(orc.kv_dequant_tokens(ch, 10, 20, key=True),
                          orc.bf16_rne((xk + ch["mu"][None, :])[10:30]))


def test_effective_set_golden_64s(orc):
    Tc, W, sink = 7040, 4, 3 * 880
    cuts = [0, 10, 20, 30]
    rows = read_golden("effective_set_64s.txt")
    total = 0
    for t, n in rows:
        shot = max(c for c in cuts if c <= t)
        got = orc.effective_tokens(t, Tc, W, sink, shot * Tc, sink, want_list=False)
        assert got == n, (t, got, n)
        total += got
    assert total == 1188000


@pytest.mark.parametrize("Tc,W,g,s,shot,t", [
    (100, 3, 30, 20, 0, 7), (100, 3, 30, 20, 2, 7), (100, 1, 100, 100, 5, 9),
    (64, 2, 0, 0, 3, 6), (50, 5, 10, 40, 1, 3), (8, 2, 8, 8, 6, 6), (8, 2, 8, 8, 6, 7)])
def test_effective_set_vs_interval_union(orc, Tc, W, g, s, shot, t):
    toks = orc.effective_tokens(t, Tc, W, g, shot * Tc, s)
    assert np.all(np.diff(toks) > 0)
    hi = t * Tc
    ivs = [(0, min(g, hi)), (shot * Tc, min(shot * Tc + s, hi)), (max(0, t - W) * Tc, hi)]
    ivs = sorted((a, b) for a, b in ivs if b > a)
    merged = []
    for a, b in ivs:
        if merged and a <= merged[-1][1]:
            merged[-1] = (merged[-1][0], max(b, merged[-1][1]))
        else:
            merged.append((a, b))
    expect = np.concatenate([np.arange(a, b) for a, b in merged]) if merged else np.zeros(0, np.int64)
    assert np.array_equal(toks, expect)


def test_gather_oracle_composes_chunks(orc):
    Tc, H, d, W = 48, 2, 32, 2
    g = s = 16
    chunks = {}
    for c in range(5):
        k, v = synth.kv_chunk(77, c, Tc, H, d)
        chunks[c] = orc.kv_encode_chunk(synth.bf16_bits_to_f32(k).reshape(Tc, H * d),
                                        synth.bf16_bits_to_f32(v).reshape(Tc, H * d))
    toks, Kg, Vg = orc.gather_window(chunks, 5, Tc, W, g, 2 * Tc, s)
    assert len(toks) == g + s + W * Tc
    assert np.array_equal(Kg[:g], orc.kv_dequant_tokens(chunks[0], 0, g, key=True))
    assert np.array_equal(Vg[g:g + s], orc.kv_dequant_tokens(chunks[2], 0, s, key=False))
    assert np.array_equal(Kg[-Tc:], orc.kv_dequant_tokens(chunks[4], 0, Tc, key=True))


def test_threaded_chunk_driver_equals_c_routine(orc):
    """The oracle's row-range driver (statistics over the chunk, then row
    ranges encoded on threads) gives the C routine's bytes, and a token
    subset gives those rows of it."""
    K, V = small_chunk(seed=2003, T=300, H=2, d=64)
    a = orc.kv_encode_chunk(K, V)
    b = orc.kv_encode_chunk(K, V, threads=5)
    for name in ("kc", "ks", "vc", "vs", "mu"):
        assert np.array_equal(a[name], b[name]), name
    assert a["sdk"] == b["sdk"] and a["sdv"] == b["sdv"]
    rows = np.array([299, 0, 17, 150])
    c = orc.kv_encode_chunk(K, V, rows=rows, threads=3)
    for name in ("kc", "ks", "vc", "vs"):
        assert np.array_equal(a[name][rows], c[name]), name
    assert np.array_equal(orc.kv_dequant_rows(a, key=True, threads=4),
                          orc.kv_dequant_tokens(a, 0, 300, key=True))
