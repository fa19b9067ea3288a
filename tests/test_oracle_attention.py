"""Pins of the oracle's attention (attention_ref) against mathematics.

Brute force in pure Python on tiny inputs (distinct heads, so a wrong head or
operand index fails), closed forms (identical keys and scale 0 give the mean
of the values; a dominant key gives its value), invariances (key order, a
shift of every key along a fixed vector), the log-sum-exp merge of two key
sets, and the empty set.
"""
import math

import numpy as np
import pytest

import oracle as orc


def rnd(seed, *shape, s=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * s).astype(np.float32)


def brute(q, k, v, scale):
    nq, H, d = q.shape
    nk = k.shape[0]
    o = np.zeros((nq, H, d))
    lse = np.zeros((nq, H))
    for i in range(nq):
        for h in range(H):
            s = [scale * sum(float(q[i, h, e]) * float(k[j, h, e]) for e in range(d))
                 for j in range(nk)]
            w = [math.exp(x) for x in s]
            tot = sum(w)
            lse[i, h] = math.log(tot)
            for e in range(d):
                o[i, h, e] = sum(w[j] * float(v[j, h, e]) for j in range(nk)) / tot
    return o, lse


def test_brute_force_tiny():
    q, k, v = rnd(1, 3, 2, 5), rnd(2, 7, 2, 5), rnd(3, 7, 2, 5)
    o, ao, lse = orc.attention_ref(q, k, v, 0.7)
    ob, lb = brute(q, k, v, 0.7)
    assert np.allclose(o, ob, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, lb, rtol=1e-12, atol=1e-13)
    assert np.all(ao >= np.abs(o) - 1e-15)


def test_rows_pick_queries():
    q, k, v = rnd(4, 6, 2, 8), rnd(5, 9, 2, 8), rnd(6, 9, 2, 8)
    o, _, lse = orc.attention_ref(q, k, v, 0.3)
    rows = np.array([5, 0, 3])
    o2, _, lse2 = orc.attention_ref(q, k, v, 0.3, rows=rows)
    assert np.array_equal(o2, o[rows]) and np.array_equal(lse2, lse[rows])


def test_identical_keys_and_zero_scale_give_the_mean():
    q, v = rnd(7, 4, 3, 16), rnd(8, 10, 3, 16)
    k = np.repeat(rnd(9, 1, 3, 16), 10, axis=0)
    mean = v.astype(np.float64).mean(axis=0)
    o, _, lse = orc.attention_ref(q, k, v, 0.25)
    assert np.allclose(o, mean[None], rtol=1e-13, atol=1e-14)
    o0, _, lse0 = orc.attention_ref(q, rnd(10, 10, 3, 16), v, 0.0)
    assert np.allclose(o0, mean[None], rtol=1e-13, atol=1e-14)
    assert np.allclose(lse0, math.log(10.0), rtol=1e-14)


def test_dominant_key_selects_its_value():
    q = np.zeros((1, 1, 4), np.float32)
    q[0, 0, 0] = 1.0
    k = rnd(11, 6, 1, 4, s=0.1)
    k[4, 0, 0] = 80.0  # score gap > 70: the other weights are below e^-70
    v = rnd(12, 6, 1, 4)
    o, _, _ = orc.attention_ref(q, k, v, 1.0)
    # weight 1 for key 4, at most 5e-34 in total for the rest: below half an
    # ulp of the sums, so the result is v[4] exactly
    assert np.array_equal(o[0, 0], v[4, 0].astype(np.float64))


def test_key_order_and_shift_invariance():
    q, v = rnd(13, 5, 2, 8), rnd(15, 12, 2, 8)
    k = np.round(rnd(14, 12, 2, 8) * 1024) / 1024  # on a 2^-10 grid: k + 0.5 is exact
    o, _, lse = orc.attention_ref(q, k, v, 0.5)
    perm = np.random.default_rng(16).permutation(12)
    o2, _, lse2 = orc.attention_ref(q, k[perm], v[perm], 0.5)
    assert np.allclose(o2, o, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse2, lse, rtol=1e-12, atol=1e-13)
    # every key moved by u: each query's scores move by scale * q.u together
    u = np.zeros((1, 2, 8), np.float32)
    u[0, :, 3] = 0.5
    o3, _, lse3 = orc.attention_ref(q, k + u, v, 0.5)
    assert np.allclose(o3, o, rtol=1e-12, atol=1e-13)
    shift = 0.5 * 0.5 * q[:, :, 3].astype(np.float64)
    assert np.allclose(lse3, lse + shift, rtol=1e-12, atol=1e-13)


def test_log_sum_exp_merge_of_two_key_sets():
    q, k, v = rnd(17, 4, 2, 8), rnd(18, 11, 2, 8), rnd(19, 11, 2, 8)
    o, _, lse = orc.attention_ref(q, k, v, 0.4)
    oa, _, la = orc.attention_ref(q, k[:6], v[:6], 0.4)
    ob, _, lb = orc.attention_ref(q, k[6:], v[6:], 0.4)
    mx = np.maximum(la, lb)
    wa, wb = np.exp(la - mx), np.exp(lb - mx)
    merged = (wa[..., None] * oa + wb[..., None] * ob) / (wa + wb)[..., None]
    assert np.allclose(merged, o, rtol=1e-12, atol=1e-13)
    assert np.allclose(mx + np.log(wa + wb), lse, rtol=1e-12, atol=1e-13)


def test_empty_key_set():
    q = rnd(20, 3, 2, 8)
    k = np.zeros((0, 2, 8), np.float32)
    o, ao, lse = orc.attention_ref(q, k, k, 0.5)
    assert np.all(o == 0) and np.all(ao == 0) and np.all(np.isneginf(lse))


def test_shape_mismatch_rejected():
    with pytest.raises(ValueError):
        orc.attention_ref(rnd(21, 2, 2, 8), rnd(22, 3, 2, 8), rnd(23, 3, 1, 8), 1.0)
