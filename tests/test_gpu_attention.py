"""GPU parity: attention over K_eff(t) read packed from the ring (the
dequantization fused in), against the oracle's double-precision attention
over the oracle's own gather of the same chunks.

Bar, per output element (q, head, e):
  |o - o_ref| <= 2^-8 (A + |o_ref|) + 2^-16 scale |q| max_j |k_j| A
with A = sum_j w_j |v_j| / sum_j w_j (the oracle's abs-weighted value).  The
GPU rounds the softmax weights to bf16 (each within 2^-9 of its own value;
the normaliser sums the same rounded weights, so numerator and denominator
move together: at most 2^-9 A), rounds o to bf16 (2^-9 |o|), and forms the
scores in fp32 from exact bf16 products: a 128-term fp32 sum is off by at
most 128 * 2^-24 sum_e |q_e k_e| <= 2^-17 |q| |k_j|, which moves each weight
by at most that much relative (x2 with the normaliser); the fp32 sums over
the tiles add ~2^-15 relative at the sizes here.  The bound takes twice the
two bf16 terms.  lse = m + ln(sum of the rounded weights): within 2^-9 of
the exact log-sum-exp from the rounding, plus the score term; the bound is
|lse - lse_ref| <= 2^-16 scale |q| max|k| + 2^-8 + 2^-14 |lse_ref|.
With key splits each split's weights are rounded relative to its own
maximum (the same 2^-9 per weight), and the merge scales a split's fp32
numerator and normaliser by the same factor 2^(m_s - M): a few 2^-24
relative more, inside the same bound.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_quantization_amd as m

    m.lib()
    return m


def bf16_gpu(bits, shape):
    return torch.from_numpy(bits.view(np.int16).reshape(shape)).view(torch.bfloat16).cuda()


def f32_of_bits(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def queries(seed, n, H, d):
    _, qb = synth.kv_chunk(seed, 0, n, H, d)  # N(0, 1) values rounded to bf16
    return qb.reshape(n, H, d), f32_of_bits(qb).reshape(n, H, d)


def check(nv, orc, ring, chunks, cfg, t, shot, qbits, qf, rows=None, scale=None,
          key_splits=(0,)):
    """Each split count in `key_splits` (0 = the library's choice) against
    one oracle result."""
    Tc, H, d = cfg.chunk_tokens, cfg.heads, cfg.head_dim
    g_tok = cfg.sink_frames_global * cfg.tokens_per_frame
    s_tok = cfg.sink_frames_shot * cfg.tokens_per_frame
    scale = d ** -0.5 if scale is None else scale
    nq = qf.shape[0]
    q = bf16_gpu(qbits, (nq, H, d))
    runs = []
    for ks in key_splits:
        lse = torch.empty((nq, H), dtype=torch.float32, device="cuda")
        runs.append((ks, ring.attention(t, q, scale, lse=lse, key_splits=ks), lse))
    _, Kr, Vr = orc.gather_window(chunks, t, Tc, cfg.window_chunks, g_tok, shot * Tc, s_tok)
    k = f32_of_bits(Kr).reshape(-1, H, d)
    v = f32_of_bits(Vr).reshape(-1, H, d)
    o_ref, a_ref, lse_ref = orc.attention_ref(qf, k, v, scale, rows=rows)
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else torch.from_numpy(np.asarray(rows)).cuda()
    for ks, o, lse in runs:
        og = o[sel].float().cpu().numpy().astype(np.float64)
        lg = lse[sel].cpu().numpy().astype(np.float64)
        if k.shape[0] == 0:
            assert np.all(og == 0) and np.all(np.isneginf(lg)), f"step {t} splits {ks}: empty set"
            continue
        qsel = qf if rows is None else qf[rows]
        qn = np.linalg.norm(qsel.astype(np.float64), axis=2)                  # [n, H]
        kmax = np.linalg.norm(k.astype(np.float64), axis=2).max(axis=0)        # [H]
        sc = 2.0 ** -16 * scale * qn * kmax[None, :]
        tol = 2.0 ** -8 * (a_ref + np.abs(o_ref)) + sc[..., None] * a_ref
        err = np.abs(og - o_ref)
        worst = np.unravel_index(np.argmax(err - tol), err.shape)
        assert np.all(err <= tol), \
            f"step {t} splits {ks}: o off at {worst}: {err[worst]} > {tol[worst]}"
        ltol = sc + 2.0 ** -8 + 2.0 ** -14 * np.abs(lse_ref)
        assert np.all(np.abs(lg - lse_ref) <= ltol), f"step {t} splits {ks}: lse off"


def small_cfg(nv, **kw):
    base = dict(tokens_per_frame=16, frames_per_chunk=4, heads=2, head_dim=128,
                sink_frames_global=1, sink_frames_shot=2, window_chunks=2)
    base.update(kw)
    return nv.KVConfig(**base)


def drive(nv, orc, cfg, cuts, steps, seed, at_step):
    ring = nv.KVRing(cfg)
    Tc, H, d = cfg.chunk_tokens, cfg.heads, cfg.head_dim
    chunks, shot = {}, 0
    for t in range(steps):
        if t in cuts:
            shot = t
            ring.begin_shot(t)
        at_step(ring, chunks, t, shot)
        kb, vb = synth.kv_chunk(seed, t, Tc, H, d)
        ring.store_chunk(t, bf16_gpu(kb, (Tc, H, d)), bf16_gpu(vb, (Tc, H, d)))
        chunks[t] = orc.kv_encode_chunk(f32_of_bits(kb).reshape(Tc, H * d),
                                        f32_of_bits(vb).reshape(Tc, H * d), search=cfg.search)


def test_attention_every_step_small_ring(nv, orc):
    """Tc = 64, 2 heads, W = 2, a 16-token global sink and a 32-token shot
    sink, shot cuts at 0 and 4: empty set, sink-only, partial 64-key tiles,
    up to four segments; 100 queries (a ragged query tile).  One split, and
    3 and 8 key splits (splits without tiles at the early steps)."""
    cfg = small_cfg(nv)
    qbits, qf = queries(3001, 100, cfg.heads, cfg.head_dim)

    def at(ring, chunks, t, shot):
        print("case: attention small ring step", t, flush=True)
        check(nv, orc, ring, chunks, cfg, t, shot, qbits, qf, key_splits=(1, 3, 8))

    drive(nv, orc, cfg, {0, 4}, 8, 3002, at)


@pytest.mark.parametrize("nq", [1, 129, 300])
def test_attention_query_counts(nv, orc, nq):
    cfg = small_cfg(nv, tokens_per_frame=40, window_chunks=3)  # Tc = 160: 2.5 tiles a chunk
    qbits, qf = queries(3003 + nq, nq, cfg.heads, cfg.head_dim)

    def at(ring, chunks, t, shot):
        if t == 5:
            print("case: attention nq", nq, flush=True)
            check(nv, orc, ring, chunks, cfg, t, shot, qbits, qf, key_splits=(1, 2, 5))

    drive(nv, orc, cfg, {0, 3}, 6, 3004, at)


@pytest.mark.parametrize("scale", [0.0, 0.01, 0.3])
def test_attention_softmax_scales(nv, orc, scale):
    """Scale 0 (uniform weights: the mean of the values), a flat and a
    sharp softmax, at a step with all four segments."""
    cfg = small_cfg(nv)
    qbits, qf = queries(3007, 70, cfg.heads, cfg.head_dim)

    def at(ring, chunks, t, shot):
        if t == 7:  # global sink, shot sink (chunk 4, below the window), chunks 5 and 6
            print("case: attention scale", scale, flush=True)
            check(nv, orc, ring, chunks, cfg, t, shot, qbits, qf, scale=scale, key_splits=(1, 4))

    drive(nv, orc, cfg, {0, 4}, 8, 3008, at)


def test_attention_64s_ring_step_15_sampled(nv, orc):
    """The 64 s ring (7040 tokens x 24 heads x 128 a chunk, W = 4, 3-frame
    sinks, shots at 0 and 10) at step 15: 7040 queries over the 33,440-token
    set (2640 + 2640 sink tokens and 4 window chunks), the launch the bench
    times (the library's split choice), and one split; 12 sampled queries
    (first and last included) x 24 heads against the oracle."""
    print("case: attention 64 s ring step 15", flush=True)
    cfg = nv.KVConfig()
    Tc, H, d = cfg.chunk_tokens, cfg.heads, cfg.head_dim
    # chunks 1..9 leave the set before step 15: they reuse chunk 0's values
    need = [0, 10, 11, 12, 13, 14]

    def make(t):
        kb, vb = synth.kv_chunk(3005, t, Tc, H, d)
        enc = orc.kv_encode_chunk(f32_of_bits(kb).reshape(Tc, H * d),
                                  f32_of_bits(vb).reshape(Tc, H * d))
        return kb, vb, enc

    with ThreadPoolExecutor(max_workers=6) as ex:
        made = dict(zip(need, ex.map(make, need)))
    chunks = {t: made[t][2] for t in need}
    ring = nv.KVRing(cfg)
    for t in range(15):
        if t % 10 == 0:
            ring.begin_shot(t)
        kb, vb, _ = made.get(t, made[0])
        ring.store_chunk(t, bf16_gpu(kb, (Tc, H, d)), bf16_gpu(vb, (Tc, H, d)))
    assert ring.effective_tokens(15) == 33440
    qbits, qf = queries(3006, Tc, H, d)
    rows = np.unique(np.concatenate([[0, 127, 128, Tc - 1],
                                     np.random.default_rng(7).integers(0, Tc, 8)]))
    print("case: attention 64 s ring step 15 plan", ring.attention_plan(15, Tc), flush=True)
    check(nv, orc, ring, chunks, cfg, 15, 10, qbits, qf, rows=rows, key_splits=(0, 1))


@pytest.mark.parametrize("key_splits", [1, 3, 8])
def test_attention_identical_values_reproduced(nv, orc, key_splits):
    """Every token of every chunk carries the same value row: the softmax
    weights, whatever they are, then average identical rows, and o must be
    that row exactly (bf16).  The kernel divides the bf16-rounded weights'
    value product by the sum of the same rounded weights, so o is an exact
    weighted mean up to fp32 summation; a normaliser of unrounded weights
    would scale o by up to 1 +- 2^-9 and move it off the row.  (A -0 value
    comes back as +0: the sums start from +0.)"""
    cfg = small_cfg(nv)
    Tc, H, d = cfg.chunk_tokens, cfg.heads, cfg.head_dim
    qbits, _ = queries(3011, 200, H, d)
    _, vrow = synth.kv_chunk(3012, 0, 1, H, d)
    vb = np.ascontiguousarray(np.broadcast_to(vrow, (Tc, H, d)))
    ring = nv.KVRing(cfg)
    vhat = None
    for t in range(6):
        if t in (0, 4):
            ring.begin_shot(t)
        kb, _ = synth.kv_chunk(3013, t, Tc, H, d)
        ring.store_chunk(t, bf16_gpu(kb, (Tc, H, d)), bf16_gpu(vb, (Tc, H, d)))
        if vhat is None:
            enc = orc.kv_encode_chunk(f32_of_bits(kb).reshape(Tc, H * d),
                                      f32_of_bits(vb).reshape(Tc, H * d))
            vhat = orc.kv_dequant_tokens(enc, 0, 1, key=False).reshape(H, d)
    print("case: attention identical values, splits", key_splits, flush=True)
    q = bf16_gpu(qbits, (200, H, d))
    for scale in (d ** -0.5, 0.7):
        o = ring.attention(6, q, scale, key_splits=key_splits)
        torch.cuda.synchronize()
        of = o.float().cpu().numpy()
        assert np.array_equal(of, np.broadcast_to(f32_of_bits(vhat), of.shape)), (scale, key_splits)


@pytest.mark.parametrize("key_splits", [1, 3])
def test_attention_deterministic(nv, orc, key_splits):
    """Fixed tile order, fixed in-tile order and a fixed merge order: two
    calls agree bit for bit, and a third without the lse output gives the
    same o."""
    cfg = small_cfg(nv)
    qbits, _ = queries(3009, 300, cfg.heads, cfg.head_dim)

    def at(ring, chunks, t, shot):
        if t == 7:
            q = bf16_gpu(qbits, (300, cfg.heads, cfg.head_dim))
            l1 = torch.empty((300, cfg.heads), dtype=torch.float32, device="cuda")
            l2 = torch.empty_like(l1)
            o1 = ring.attention(t, q, lse=l1, key_splits=key_splits)
            o2 = ring.attention(t, q, lse=l2, key_splits=key_splits)
            o3 = ring.attention(t, q, key_splits=key_splits)  # no lse output
            torch.cuda.synchronize()
            assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(o1, o3)

    drive(nv, orc, cfg, {0, 4}, 8, 3010, at)


def test_attention_validation(nv):
    cfg = small_cfg(nv)
    ring = nv.KVRing(cfg)
    q = torch.zeros((4, 2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError):
        ring.attention(1, q)  # step != next chunk
    with pytest.raises(ValueError):
        ring.attention(0, q[:, :1])  # wrong head count
    with pytest.raises(ValueError):
        ring.attention(0, q, out=torch.empty((3, 2, 128), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        ring.attention(0, q, lse=torch.empty((4, 3), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        ring.attention(0, q, key_splits=2,
                       workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(RuntimeError):
        ring.attention(0, q, key_splits=9)
    ring64 = nv.KVRing(small_cfg(nv, head_dim=64))
    with pytest.raises(RuntimeError):
        ring64.attention(0, torch.zeros((4, 2, 64), dtype=torch.bfloat16, device="cuda"))


def test_attention_auto_splits_follow_the_model(nv):
    """The library's split choice equals the cost model its header states,
    evaluated here with this device's compute-unit count: ceil(n s / CUs)
    rounds of 1/s, times 1 + 0.015 s, the cheapest s in 1..8 taken if it
    saves 3% over one split and every split keeps 8 tiles (white-box: the
    ring's counters are set as stores and shot starts would set them)."""
    import math

    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def model(units, ntile):
        if units == 0 or ntile < 16:
            return 1
        cost = lambda sp: math.ceil(units * sp / cus) / sp * (1.0 + 0.015 * sp)
        best = 1
        for sp in range(2, 9):
            if ntile < 8 * sp:
                break
            if cost(sp) < cost(best):
                best = sp
        return best if cost(best) <= 0.97 * cost(1) else 1

    cfg = nv.KVConfig()
    ring = nv.KVRing(cfg)
    Tc = cfg.chunk_tokens
    g = cfg.sink_frames_global * cfg.tokens_per_frame
    for step, shot in [(1, 0), (3, 0), (15, 10), (25, 20)]:
        ring.ring.next_chunk = step
        ring.ring.s_start = shot * Tc
        # the segments: the global sink below the window, the shot sink's
        # part above the global sink and below the window, the window chunks
        win_lo = max(0, step - cfg.window_chunks) * Tc
        n_g = min(g, win_lo)
        s_hi = min(shot * Tc + cfg.sink_frames_shot * cfg.tokens_per_frame, win_lo)
        n_s = max(0, s_hi - max(shot * Tc, n_g))
        n_chunks = step - max(0, step - cfg.window_chunks)
        assert n_g + n_s + n_chunks * Tc == ring.effective_tokens(step), step
        ntile = -(-n_g // 64) + -(-n_s // 64) + n_chunks * -(-Tc // 64)
        for nq in [0, 1, 256, 2048, 7040, 14080, 70400]:
            sp, wsb = ring.attention_plan(step, nq)
            units = -(-nq // 256) * cfg.heads
            assert sp == model(units, ntile), (step, nq, sp, model(units, ntile))
            rows = sp * nq * cfg.heads
            assert wsb == (0 if sp == 1 else -(-rows * 8 // 256) * 256 + rows * 512)
    print("case: auto splits on", cus, "CUs", flush=True)
