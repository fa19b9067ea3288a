"""GPU parity: KV-cache chunk store and window gather vs the CPU oracle.

Bar: ring contents (codes, scales, mu, s_dec) and gathered bf16 K/V bit-exact.
"""
import numpy as np
import pytest
import torch

import synth
from helpers import kmean_fp64_exact

pytestmark = pytest.mark.gpu
THREADS = synth.host_threads()


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_quantization_amd as m

    m.lib()
    return m


def chunk_inputs(seed, c, T, H, d):
    kb, vb = synth.kv_chunk(seed, c, T, H, d, threads=THREADS)
    Kg = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).cuda()
    Vg = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).cuda()
    K = synth.bf16_bits_to_f32(kb).reshape(T, H * d)
    V = synth.bf16_bits_to_f32(vb).reshape(T, H * d)
    # the kernels' double key sums are exact (so equal the oracle's exact
    # mean) on inputs like these; the library leaves other inputs' mean
    # unspecified up to that rounding
    assert kmean_fp64_exact(K), f"chunk {c} of seed {seed} outside the key-mean domain"
    return Kg, Vg, K, V


def bf16_np(t):
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16).reshape(t.shape[0], -1)


def run_ring(nv, orc, cfg, cuts, steps, seed):
    """Drive the ring through `steps` steps (shot cuts at `cuts`) and compare
    every gathered value with the oracle's gather."""
    ring = nv.KVRing(cfg)
    Tc, H, d = cfg.chunk_tokens, cfg.heads, cfg.head_dim
    g_tok = cfg.sink_frames_global * cfg.tokens_per_frame
    s_tok = cfg.sink_frames_shot * cfg.tokens_per_frame
    chunks = {}
    shot = 0
    for t in range(steps):
        if t in cuts:
            shot = t
            ring.begin_shot(t)
        # gather of step t, then store chunk t
        Kw, Vw = ring.gather_window(t)
        toks = orc.effective_tokens(t, Tc, cfg.window_chunks, g_tok, shot * Tc, s_tok)
        assert Kw.shape[0] == len(toks), (t, Kw.shape, len(toks))
        if len(toks):
            _, Kr, Vr = orc.gather_window(chunks, t, Tc, cfg.window_chunks, g_tok, shot * Tc,
                                          s_tok)
            kg, vg = bf16_np(Kw), bf16_np(Vw)
            assert np.array_equal(kg, Kr), f"step {t}: K differs"
            assert np.array_equal(vg, Vr), f"step {t}: V differs"
        Kg, Vg, K, V = chunk_inputs(seed, t, Tc, H, d)
        ring.store_chunk(t, Kg, Vg)
        chunks[t] = orc.kv_encode_chunk(K, V, search=cfg.search, threads=THREADS)
        # drop chunks no step can reference any more (window and sinks)
        for old in list(chunks):
            if old not in (0, shot) and old < t + 1 - cfg.window_chunks:
                del chunks[old]
    torch.cuda.synchronize()
    return ring, chunks


def region(mem, off, T, HD):
    """Arrays of one ring region at byte offset `off`: K codes, K scales, V
    codes, V scales (each 256-byte aligned), mu, s_dec."""
    a = lambda n: (n + 255) // 256 * 256
    o = off
    out = {}
    for name, n in (("kc", T * HD // 2), ("ks", T * HD // 16), ("vc", T * HD // 2),
                    ("vs", T * HD // 16)):
        out[name] = mem[o:o + n]
        o += a(n)
    out["mu"] = mem[o:o + HD * 4].view(np.float32)
    o += a(HD * 4)
    out["sd"] = mem[o:o + 8].view(np.float32)
    return out


def ring_bytes(ring):
    torch.cuda.synchronize()
    return ring.mem.cpu().numpy()[ring._base - ring.mem.data_ptr():]


def assert_region(reg, ref, ntok, HD):
    """Region holding the first ntok tokens of the oracle's chunk `ref`."""
    assert np.array_equal(reg["mu"], ref["mu"])
    assert reg["sd"][0] == ref["sdk"] and reg["sd"][1] == ref["sdv"]
    for name, per in (("kc", HD // 2), ("ks", HD // 16), ("vc", HD // 2), ("vs", HD // 16)):
        got, want = reg[name], ref[name].ravel()[:ntok * per]
        bad = np.flatnonzero(got[:ntok * per] != want)
        assert bad.size == 0, f"{name}: {bad.size} bytes differ, first at {bad[:4]}"


# (tokens per frame, frames per chunk, heads, head_dim, S_g, S_s): ragged last
# 64-token node, chunks shorter than a tile, channel counts that are not
# multiples of 128, a 1024-node key-mean tree (65536 tokens), sinks
STORE_CASES = [
    (40, 5, 3, 32, 2, 1),
    (7, 1, 1, 16, 1, 0),
    (16, 4, 2, 64, 1, 2),
    (13, 10, 1, 48, 3, 2),
    (125, 8, 5, 16, 3, 3),
    (520, 8, 2, 128, 3, 3),
    (880, 8, 3, 128, 3, 3),
    (8192, 8, 1, 16, 1, 1),
    (880, 8, 24, 128, 3, 3),  # the 5B model's whole chunk: 7040 tokens x 24 heads x 128
]


@pytest.mark.parametrize("case", STORE_CASES, ids=lambda c: "x".join(map(str, c)))
def test_store_bit_exact_ragged_and_sinks(nv, orc, case):
    """Slot and both sink copies after storing chunk 0 equal the oracle's
    encoding byte for byte."""
    Lf, Fc, H, d, Sg, Ss = case
    T, HD = Lf * Fc, H * d
    print("case: store", case, flush=True)
    cfg = nv.KVConfig(tokens_per_frame=Lf, frames_per_chunk=Fc, heads=H, head_dim=d,
                      sink_frames_global=Sg, sink_frames_shot=Ss, window_chunks=2)
    ring = nv.KVRing(cfg)
    Kg, Vg, K, V = chunk_inputs(2100 + T, 0, T, H, d)
    ring.store_chunk(0, Kg, Vg)
    ref = orc.kv_encode_chunk(K, V, threads=THREADS)
    mem = ring_bytes(ring)
    assert_region(region(mem, 0, T, HD), ref, T, HD)
    if Sg:
        assert_region(region(mem, ring.ring.gsink_offset, Sg * Lf, HD), ref, Sg * Lf, HD)
    if Ss:
        assert_region(region(mem, ring.ring.ssink_offset, Ss * Lf, HD), ref, Ss * Lf, HD)


def test_store_chunk_ring_bytes_bit_exact(nv, orc):
    """Ring slot contents after one store equal the oracle's chunk encoding."""
    cfg = nv.KVConfig(tokens_per_frame=40, frames_per_chunk=5, heads=3, head_dim=32,
                      sink_frames_global=2, sink_frames_shot=1, window_chunks=2)
    print("case: store chunk T=200 H=3 d=32", flush=True)
    ring = nv.KVRing(cfg)
    Kg, Vg, K, V = chunk_inputs(2002, 0, 200, 3, 32)
    ring.store_chunk(0, Kg, Vg)
    ref = orc.kv_encode_chunk(K, V)
    torch.cuda.synchronize()
    mem = ring.mem.cpu().numpy()[ring._base - ring.mem.data_ptr():]
    T, HD = 200, 96
    # slot 0 layout: K codes, K scales, V codes, V scales, mu, s_dec (each 256-aligned)
    a = lambda n: (n + 255) // 256 * 256
    o = 0
    kc = mem[o:o + T * HD // 2]; o += a(T * HD // 2)
    ks = mem[o:o + T * HD // 16]; o += a(T * HD // 16)
    vc = mem[o:o + T * HD // 2]; o += a(T * HD // 2)
    vs = mem[o:o + T * HD // 16]; o += a(T * HD // 16)
    mu = mem[o:o + HD * 4].view(np.float32); o += a(HD * 4)
    sd = mem[o:o + 8].view(np.float32)
    assert np.array_equal(mu, ref["mu"])
    assert sd[0] == ref["sdk"] and sd[1] == ref["sdv"]
    assert np.array_equal(kc, ref["kc"].ravel())
    assert np.array_equal(ks, ref["ks"].ravel())
    assert np.array_equal(vc, ref["vc"].ravel())
    assert np.array_equal(vs, ref["vs"].ravel())


def test_ring_small_geometry_all_segments(nv, orc):
    """Small ring over 14 steps: global sink in and out of the window, shot
    sinks rebound at prompt switches, overlapping sinks, window wrap-around."""
    print("case: ring Tc=48 W=2 14 steps", flush=True)
    cfg = nv.KVConfig(tokens_per_frame=12, frames_per_chunk=4, heads=2, head_dim=32,
                      sink_frames_global=2, sink_frames_shot=1, window_chunks=2)
    run_ring(nv, orc, cfg, cuts={0, 3, 4, 9}, steps=14, seed=77)


def test_ring_search6_and_window1(nv, orc):
    cfg = nv.KVConfig(tokens_per_frame=16, frames_per_chunk=2, heads=1, head_dim=64,
                      sink_frames_global=1, sink_frames_shot=2, window_chunks=1,
                      search=nv.SEARCH_6)
    run_ring(nv, orc, cfg, cuts={0, 2, 5}, steps=9, seed=78)


def test_ring_64s_schedule_one_head(nv, orc):
    """The 64 s schedule (40 chunks of 7040 tokens, cuts every 10 chunks, 3-frame
    sinks, W = 4) with one 128-wide head, every gathered value checked."""
    print("case: ring 64s schedule H=1", flush=True)
    cfg = nv.KVConfig(heads=1, head_dim=128)
    run_ring(nv, orc, cfg, cuts={0, 10, 20, 30}, steps=40, seed=1005)


def sample_plan(cfg, cuts, steps, n_sample, rng_seed):
    """Per step t, the positions of E(t) to check (first, last, both sides of
    every segment boundary, and n_sample random ones), and per chunk the
    local tokens any step will check."""
    Tc, W = cfg.chunk_tokens, cfg.window_chunks
    g_tok = cfg.sink_frames_global * cfg.tokens_per_frame
    s_tok = cfg.sink_frames_shot * cfg.tokens_per_frame
    import oracle as orc

    plan, need, shot = {}, {}, 0
    for t in range(steps):
        if t in cuts:
            shot = t
        toks = orc.effective_tokens(t, Tc, W, g_tok, shot * Tc, s_tok)
        if len(toks) == 0:
            plan[t] = (toks, np.zeros(0, np.int64))
            continue
        jumps = np.flatnonzero(np.diff(toks) != 1)
        edges = np.concatenate([[0, len(toks) - 1], jumps, jumps + 1,
                                np.flatnonzero(np.diff(toks // Tc) != 0) + 1])
        rnd = np.random.default_rng(rng_seed + t).integers(0, len(toks), n_sample)
        idx = np.unique(np.concatenate([edges, rnd]))
        plan[t] = (toks, idx)
        for tok in toks[idx]:
            need.setdefault(int(tok // Tc), set()).add(int(tok % Tc))
    return plan, {c: np.array(sorted(v), np.int64) for c, v in need.items()}


def test_ring_64s_schedule_24_heads_sampled(nv, orc):
    """The 64 s schedule at full geometry (40 chunks of 7040 tokens x 24 heads
    x 128, cuts every 10 chunks, 3-frame sinks, W = 4): every step's gather
    on at least 256 sampled tokens plus every segment edge, against the
    oracle's encoding of each chunk (statistics over the whole chunk)."""
    cfg = nv.KVConfig()
    cuts = {0, 10, 20, 30}
    steps, seed = 40, 1005
    Tc, H, d = cfg.chunk_tokens, cfg.heads, cfg.head_dim
    plan, need = sample_plan(cfg, cuts, steps, 256, 6400)
    ring = nv.KVRing(cfg)
    enc = {}  # chunk -> (oracle encoding of its needed tokens, token -> row)
    for t in range(steps):
        print("case: ring 64s 24 heads step", t, flush=True)
        if t in cuts:
            ring.begin_shot(t)
        Kw, Vw = ring.gather_window(t)
        toks, idx = plan[t]
        assert Kw.shape[0] == len(toks), (t, Kw.shape, len(toks))
        if len(idx):
            sel = torch.from_numpy(idx).cuda()
            kg, vg = bf16_np(Kw[sel]), bf16_np(Vw[sel])
            for j, i in enumerate(idx):
                tok = int(toks[i])
                c, local = tok // Tc, tok % Tc
                ch, row = enc[c]
                r = row[local]
                kr = orc.kv_dequant_tokens(ch, r, 1, key=True)
                vr = orc.kv_dequant_tokens(ch, r, 1, key=False)
                assert np.array_equal(kg[j], kr[0]), f"step {t} token {tok}: K differs"
                assert np.array_equal(vg[j], vr[0]), f"step {t} token {tok}: V differs"
        Kg, Vg, K, V = chunk_inputs(seed, t, Tc, H, d)
        ring.store_chunk(t, Kg, Vg)
        rows = need.get(t, np.zeros(0, np.int64))
        if len(rows):
            enc[t] = (orc.kv_encode_chunk(K, V, threads=THREADS, rows=rows),
                      {int(v): k for k, v in enumerate(rows)})
        del Kg, Vg, K, V
    torch.cuda.synchronize()


def test_gather_capacity_error(nv):
    cfg = nv.KVConfig(tokens_per_frame=8, frames_per_chunk=2, heads=1, head_dim=16,
                      sink_frames_global=1, sink_frames_shot=1, window_chunks=2)
    ring = nv.KVRing(cfg)
    Kg = torch.zeros((16, 1, 16), dtype=torch.bfloat16, device="cuda")
    ring.store_chunk(0, Kg, Kg)
    small = torch.empty((4, 1, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nv.NVFP4Error):
        ring.gather_window(1, small, small)
    with pytest.raises(nv.NVFP4Error):
        ring.store_chunk(5, Kg, Kg)
    torch.cuda.synchronize()


@pytest.mark.parametrize("search", [1, 0], ids=["4o6", "6only"])
@pytest.mark.parametrize("factor", [1.0, 2.5, 0.5])
def test_store_value_amax_from_producer(nv, orc, factor, search):
    """The value tensor scale from a producer's amax (the statistics pass then
    reads the keys only): with the true max|V| the ring holds the same bytes
    as a plain store; with another amax the value codes, scales and decode
    scale are the oracle's quantization of V with that amax (values beyond
    it saturate), the keys unchanged.  Both scale searches."""
    Lf, Fc, H, d = 40, 5, 3, 128
    T, HD = Lf * Fc, H * d
    print("case: store with producer value amax x", factor, "search", search, flush=True)
    cfg = nv.KVConfig(tokens_per_frame=Lf, frames_per_chunk=Fc, heads=H, head_dim=d,
                      sink_frames_global=1, sink_frames_shot=1, window_chunks=2, search=search)
    Kg, Vg, K, V = chunk_inputs(2400, 0, T, H, d)
    vmax = np.float32(np.abs(V).max() * np.float32(factor))
    ring = nv.KVRing(cfg)
    ring.store_chunk(0, Kg, Vg, v_amax=torch.tensor([vmax], dtype=torch.float32, device="cuda"))
    mem = ring_bytes(ring)
    ref = orc.kv_encode_chunk(K, V, search=search)
    vc, vs, sdv = orc.quantize(V, amax=float(vmax), search=search)
    ref.update(vc=vc, vs=vs, sdv=sdv)
    assert_region(region(mem, 0, T, HD), ref, T, HD)
    assert_region(region(mem, ring.ring.gsink_offset, Lf, HD), ref, Lf, HD)
    if factor == 1.0:  # the same bytes as a plain store, region by region
        plain = nv.KVRing(cfg)
        plain.store_chunk(0, Kg, Vg)
        pm = ring_bytes(plain)
        for off, n in ((0, T), (ring.ring.gsink_offset, Lf), (ring.ring.ssink_offset, Lf)):
            got, want = region(mem, off, n, HD), region(pm, off, n, HD)
            assert all(np.array_equal(got[k], want[k]) for k in got)


def test_store_value_amax_full_chunk_matches_plain(nv):
    """The 5B model's whole chunk (7040 tokens x 24 heads x 128, three sink
    frames each): a store given the true max|V| writes the same slot and
    sink bytes as a plain store (whose bytes the oracle checks above)."""
    Lf, Fc, H, d = 880, 8, 24, 128
    T, HD = Lf * Fc, H * d
    print("case: full chunk, producer value amax vs plain store", flush=True)
    cfg = nv.KVConfig(tokens_per_frame=Lf, frames_per_chunk=Fc, heads=H, head_dim=d,
                      sink_frames_global=3, sink_frames_shot=3, window_chunks=2)
    kb, vb = synth.kv_chunk(2600, 0, T, H, d, threads=THREADS)
    Kg = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).cuda()
    Vg = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).cuda()
    vmax = Vg.float().abs().max().reshape(1).contiguous()
    a, b = nv.KVRing(cfg), nv.KVRing(cfg)
    a.store_chunk(0, Kg, Vg, v_amax=vmax)
    b.store_chunk(0, Kg, Vg)
    ma, mb = ring_bytes(a), ring_bytes(b)
    for off, n in ((0, T), (a.ring.gsink_offset, 3 * Lf), (a.ring.ssink_offset, 3 * Lf)):
        got, want = region(ma, off, n, HD), region(mb, off, n, HD)
        for k in got:
            assert np.array_equal(got[k], want[k]), (off, k)
