"""Pins of the oracle's KV-cache path: K-smoothing, chunk storage, the
multi-shot effective set and the gather (CPU only)."""
import math
import os

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


def test_kv_mean_exact(orc):
    K, _ = small_chunk(T=300)
    mu = orc.kv_mean(K)
    for ch in range(K.shape[1]):
        exact = math.fsum(float(v) for v in K[:, ch]) / K.shape[0]
        # mu is the double quotient rounded to float: within one float ulp of exact
        assert abs(float(mu[ch]) - exact) <= np.spacing(np.float32(abs(exact)))


def test_kv_mean_tile_order_matters_only_in_rounding(orc):
    # values spread over 60 binades: the fixed tile order is what makes the
    # result reproducible; it still lies within a few ulps of the exact mean
    rng = np.random.default_rng(4)
    K = (rng.standard_normal((257, 8)) * np.exp2(rng.integers(-30, 30, (257, 8)))).astype(np.float32)
    mu = orc.kv_mean(K)
    for ch in range(8):
        exact = math.fsum(float(v) for v in K[:, ch]) / 257
        assert abs(float(mu[ch]) - exact) <= 1e-6 * np.abs(K[:, ch]).max()


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
