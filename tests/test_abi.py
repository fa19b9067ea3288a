"""The C ABI library: loads, exports every declared symbol, and rejects bad
arguments on the host before anything is enqueued (CPU only: no call here
reaches a kernel launch)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import nvfp4_bit_quantization_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 256-byte aligned host-side stand-in, never dereferenced


def declared_functions():
    src = open(os.path.join(ROOT, "include", "nvfp4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return nv.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert set(names) <= set(nv._EXPORTS), set(names) - set(nv._EXPORTS)


def test_version_and_status_strings(L):
    assert L.nvfp4_abi_version() == 2
    assert len(L.nvfp4_build_hash()) == 16
    for s in range(0, -7, -1):
        assert L.nvfp4_status_string(s)
    assert L.nvfp4_status_string(-99) == b"unknown status"


def test_sizes(L):
    assert L.nvfp4_codes_bytes(7040, 3072) == 7040 * 3072 // 2
    assert L.nvfp4_scales_bytes(7040, 3072, nv.LAYOUT_1D) == 7040 * 3072 // 16
    assert L.nvfp4_scales_bytes(3072, 3072, nv.LAYOUT_2D) == 192 * 192
    assert L.nvfp4_quantize_workspace_bytes(4096, 128, 0) > 0


def tensor(rows, cols, layout=0, codes=FAKE, scales=FAKE, sdec=FAKE):
    return nv.CTensor(codes, scales, sdec, rows, cols, layout, 0)


def status(L, fn, *args):
    return getattr(L, fn)(*args)


def test_quantize_validation(L):
    q = lambda t, **kw: L.nvfp4_quantize(kw.get("x", FAKE), kw.get("dt", 1), C.byref(t) if t else None,
                                         kw.get("search", 1), None, kw.get("ws", FAKE),
                                         kw.get("wsb", 1 << 20), None)
    assert q(None) == -1  # EINVAL
    assert q(tensor(4, 24)) == -3
    assert q(tensor(24, 32, nv.LAYOUT_2D)) == -3
    assert q(tensor(4, 32, 5)) == -1
    assert q(tensor(4, 32), dt=7) == -1
    assert q(tensor(4, 32), search=3) == -1
    assert q(tensor(4, 32), x=FAKE + 4) == -2
    assert q(tensor(4, 32, codes=FAKE + 8)) == -2
    assert q(tensor(4, 32), wsb=4) == -4
    assert q(tensor(4, 32), ws=None) == -4
    assert b"workspace" in L.nvfp4_last_error()
    assert q(tensor(4, 32), x=None) == -1


def test_dequantize_and_gemm_validation(L):
    t = tensor(32, 64)
    assert L.nvfp4_dequantize(C.byref(t), FAKE, 9, None) == -1
    assert L.nvfp4_dequantize(C.byref(t), FAKE + 2, 1, None) == -2
    a, w = tensor(64, 64), tensor(32, 64, nv.LAYOUT_2D)
    assert L.nvfp4_gemm_w4a4(C.byref(w), C.byref(w), FAKE, 1, None, None) == -1  # A must be 1-D
    w7 = tensor(32, 64, 7)
    assert L.nvfp4_gemm_w4a4(C.byref(a), C.byref(w7), FAKE, 1, None, None) == -1  # bad W layout
    w2 = tensor(32, 128, nv.LAYOUT_2D)
    assert L.nvfp4_gemm_w4a4(C.byref(a), C.byref(w2), FAKE, 1, None, None) == -3
    assert L.nvfp4_gemm_w4a4(C.byref(a), C.byref(w), FAKE, 4, None, None) == -1
    assert L.nvfp4_gemm_w4a4(C.byref(a), C.byref(w), None, 1, None, None) == -1
    assert L.nvfp4_gemm_w4a4(C.byref(a), C.byref(w), FAKE, 1, FAKE + 2, None) == -2  # amax_out


def test_gemm_quant_validation(L):
    # nvfp4_gemm_w4a4_quant(a, w, y, search, amax_in, amax_out, stream)
    a, w = tensor(64, 64), tensor(32, 64, nv.LAYOUT_2D)
    y = tensor(64, 32)
    g = lambda yt, **kw: L.nvfp4_gemm_w4a4_quant(
        C.byref(kw.get("a", a)), C.byref(w), C.byref(yt) if yt else None, kw.get("search", 1),
        kw.get("amax_in", FAKE), kw.get("amax_out", None), None)
    assert g(None) == -1                                  # NULL y
    assert g(tensor(64, 32, nv.LAYOUT_2D)) == -1          # Y must be 1-D
    assert g(tensor(48, 32)) == -3                        # rows != M
    assert g(tensor(64, 48)) == -3                        # cols != N
    assert g(y, search=2) == -1
    assert g(y, amax_in=None) == -1
    assert b"amax_in" in L.nvfp4_last_error()
    assert g(y, amax_in=FAKE + 2) == -2
    assert g(y, amax_out=FAKE + 1) == -2
    assert g(y, a=tensor(64, 64, nv.LAYOUT_2D)) == -1     # A must be 1-D
    assert g(tensor(64, 32, codes=FAKE + 8)) == -2


def test_quantize_rht_validation(L):
    # nvfp4_quantize_rht(x, dtype, out, search, signs, amax_in, ws, ws_bytes, stream)
    t1, t2 = tensor(32, 64), tensor(32, 64, nv.LAYOUT_2D)
    assert L.nvfp4_quantize_rht(FAKE, 1, C.byref(t2), 1, 0x1234, None, FAKE, 1 << 20, None) == -1
    assert L.nvfp4_quantize_rht(FAKE, 1, C.byref(t1), 1, 0x10000, None, FAKE, 1 << 20, None) == -1
    assert L.nvfp4_quantize_rht(FAKE, 1, C.byref(t1), 3, 0x1234, None, FAKE, 1 << 20, None) == -1
    assert L.nvfp4_quantize_rht(FAKE, 1, C.byref(t1), 1, 0x1234, None, FAKE, 4, None) == -4
    assert L.nvfp4_quantize_rht(FAKE + 8, 1, C.byref(t1), 1, 0x1234, None, FAKE, 1 << 20, None) == -2


def test_mx_reference_validation(L):
    # nvfp4_mx_quantize(x, dtype, rows, cols, codes, scales, stream)
    assert L.nvfp4_mx_quantize(FAKE, 0, 4, 48, FAKE, FAKE, None) == -3      # cols % 32
    assert L.nvfp4_mx_quantize(FAKE, 7, 4, 64, FAKE, FAKE, None) == -1      # dtype
    assert L.nvfp4_mx_quantize(None, 0, 4, 64, FAKE, FAKE, None) == -1      # NULL x
    assert L.nvfp4_mx_quantize(FAKE + 4, 0, 4, 64, FAKE, FAKE, None) == -2  # alignment
    assert L.nvfp4_mx_quantize(None, 0, 0, 64, None, None, None) == 0       # empty: no-op
    # nvfp4_gemm_mx(ac, as, wc, ws, M, N, K, y, dtype, stream)
    assert L.nvfp4_gemm_mx(FAKE, FAKE, FAKE, FAKE, 32, 32, 128, FAKE, 1, None) == -3  # K % 256
    assert L.nvfp4_gemm_mx(FAKE, FAKE, FAKE, FAKE, 32, 32, 256, FAKE, 5, None) == -1  # dtype
    assert L.nvfp4_gemm_mx(FAKE, FAKE, FAKE, FAKE, 32, 32, 256, None, 1, None) == -1  # NULL y
    assert L.nvfp4_gemm_mx(FAKE, FAKE + 8, FAKE, FAKE, 32, 32, 256, FAKE, 1, None) == -2
    assert L.nvfp4_gemm_mx(FAKE, FAKE, FAKE, FAKE, 0, 32, 256, None, 1, None) == 0   # empty


CFG = nv.KVConfig()


def make_ring(L, cfg=CFG):
    c = cfg.c()
    r = nv.CKvRing()
    n = L.nvfp4_kv_ring_bytes(C.byref(c))
    assert L.nvfp4_kv_ring_init(C.byref(r), C.byref(c), FAKE, n) == 0
    return r


def test_ring_bytes_closed_form(L):
    c = CFG.c()
    n = L.nvfp4_kv_ring_bytes(C.byref(c))
    T, H, d, W = 7040, 24, 128, 4
    packed = T * H * d * 9 // 8  # (9/8) T_c H d bytes per chunk
    assert packed == 24330240
    r = make_ring(L)
    assert packed + H * d * 4 + 8 <= r.slot_bytes <= packed + H * d * 4 + 8 + 6 * 256
    sink = 3 * 880 * H * d * 9 // 8
    assert n == W * r.slot_bytes + 2 * (r.ssink_offset - r.gsink_offset)
    assert n >= W * packed + 2 * sink


def test_ring_validation(L):
    c = CFG.c()
    r = nv.CKvRing()
    assert L.nvfp4_kv_ring_init(C.byref(r), C.byref(c), FAKE, 16) == -4
    assert L.nvfp4_kv_ring_init(C.byref(r), C.byref(c), FAKE + 16, 1 << 40) == -2
    bad = nv.KVConfig(window_chunks=0).c()
    assert L.nvfp4_kv_ring_init(C.byref(r), C.byref(bad), FAKE, 1 << 40) == -1
    bad = nv.KVConfig(window_chunks=17).c()
    assert L.nvfp4_kv_ring_init(C.byref(r), C.byref(bad), FAKE, 1 << 40) == -1
    bad = nv.KVConfig(head_dim=40).c()
    assert L.nvfp4_kv_ring_init(C.byref(r), C.byref(bad), FAKE, 1 << 40) == -3
    bad = nv.KVConfig(sink_frames_shot=9).c()
    assert L.nvfp4_kv_ring_init(C.byref(r), C.byref(bad), FAKE, 1 << 40) == -1
    r = make_ring(L)
    ws = L.nvfp4_kv_store_workspace_bytes(C.byref(c))
    assert L.nvfp4_kv_store_chunk(C.byref(r), 1, FAKE, FAKE, None, FAKE, ws, None) == -5
    assert L.nvfp4_kv_store_chunk(C.byref(r), 0, FAKE, FAKE, None, FAKE, ws - 1, None) == -4
    assert L.nvfp4_kv_store_chunk(C.byref(r), 0, FAKE + 2, FAKE, None, FAKE, ws, None) == -2
    assert L.nvfp4_kv_store_chunk(C.byref(r), 0, FAKE, FAKE, FAKE + 2, FAKE, ws, None) == -2
    # sums, max, min per channel; value max, ticket counter, key and value amax
    # per 512-channel group
    assert ws == 3072 * 16 + 4 * 256
    assert L.nvfp4_kv_begin_shot(C.byref(r), 3) == -5
    n = C.c_int64()
    assert L.nvfp4_kv_effective_tokens(C.byref(r), 1, C.byref(n)) == -5
    assert L.nvfp4_kv_effective_tokens(C.byref(r), 0, C.byref(n)) == 0 and n.value == 0
    r.next_chunk = 2  # white-box: pretend two chunks were stored
    assert L.nvfp4_gather_window(C.byref(r), 2, FAKE, FAKE, 100, C.byref(n), None) == -4
    assert n.value == 2 * 7040


def test_attention_window_validation(L):
    # nvfp4_attention_window(ring, step, q, n_q, scale, o, lse, key_splits,
    # ws, ws_bytes, stream): every call below is rejected on the host before
    # a launch
    r = make_ring(L)
    a = lambda **kw: L.nvfp4_attention_window(
        C.byref(kw.get("ring", r)), kw.get("step", 0), kw.get("q", FAKE), kw.get("nq", 64),
        kw.get("scale", 0.088), kw.get("o", FAKE), kw.get("lse", None), kw.get("splits", 1),
        kw.get("ws", None), kw.get("wsb", 0), None)
    assert a(step=1) == -5                         # not the next chunk
    assert a(nq=-1) == -3
    assert a(scale=float("nan")) == -1
    assert a(scale=float("inf")) == -1
    assert a(scale=-0.5) == -1
    assert a(q=None) == -1
    assert a(o=None) == -1
    assert a(q=FAKE + 2) == -2
    assert a(lse=FAKE + 1) == -2
    assert a(splits=-1) == -1 and a(splits=9) == -1
    assert a(splits=2) == -4                       # two splits need a workspace
    need = 64 * 24 * 2 * 8 + 64 * 24 * 2 * 512    # (max, sum) block is a multiple of 256
    assert a(splits=2, ws=FAKE, wsb=need - 1) == -4
    assert a(splits=2, ws=FAKE + 16, wsb=need) == -2
    c64 = nv.KVConfig(head_dim=64).c()
    r64 = nv.CKvRing()
    assert L.nvfp4_kv_ring_init(C.byref(r64), C.byref(c64), FAKE,
                                L.nvfp4_kv_ring_bytes(C.byref(c64))) == 0
    assert a(ring=r64) == -3                       # head_dim must be 128
    assert b"128" in L.nvfp4_last_error()


def test_attention_plan(L):
    """Forced split counts and their workspace size need no device; the
    automatic choice below 8 tiles takes one split without asking it."""
    r = make_ring(L)
    sp, wsb = C.c_int32(), C.c_size_t()
    plan = lambda step, nq, ks: L.nvfp4_attention_plan(C.byref(r), step, nq, ks, C.byref(sp),
                                                       C.byref(wsb))
    assert plan(0, 7040, 0) == 0 and (sp.value, wsb.value) == (1, 0)   # empty set
    assert plan(0, 7040, 1) == 0 and (sp.value, wsb.value) == (1, 0)
    rows = 3 * 100 * 24
    assert plan(0, 100, 3) == 0 and sp.value == 3
    assert wsb.value == (rows * 8 + 255) // 256 * 256 + rows * 512
    assert plan(0, 100, 8) == 0 and sp.value == 8
    assert plan(0, 100, 9) == -1 and plan(0, 100, -1) == -1
    assert plan(1, 100, 2) == -5
    assert plan(0, -1, 2) == -3
    assert L.nvfp4_attention_plan(C.byref(r), 0, 100, 2, None, C.byref(wsb)) == -1


def test_ring_plan_matches_oracle(L, orc):
    """The host planner's |K_eff(t)| equals the oracle's brute force, for
    several geometries and shot schedules (white-box: the ring's counters are
    set directly, as stores and prompt switches would set them)."""
    for cfg, cuts, steps in [
        (CFG, [0, 10, 20, 30], 40),
        (nv.KVConfig(tokens_per_frame=5, frames_per_chunk=4, sink_frames_global=2,
                     sink_frames_shot=3, window_chunks=2), [0, 3, 4, 9], 14),
        (nv.KVConfig(tokens_per_frame=7, frames_per_chunk=2, sink_frames_global=0,
                     sink_frames_shot=2, window_chunks=1), [0, 2, 5], 9),
        (nv.KVConfig(tokens_per_frame=7, frames_per_chunk=2, sink_frames_global=2,
                     sink_frames_shot=0, window_chunks=3), [0, 6], 9),
    ]:
        r = make_ring(L, cfg)
        Tc = cfg.chunk_tokens
        for t in range(steps):
            shot = max(c for c in cuts if c <= t)
            r.next_chunk = t
            r.s_start = shot * Tc
            n = C.c_int64()
            assert L.nvfp4_kv_effective_tokens(C.byref(r), t, C.byref(n)) == 0
            ref = orc.effective_tokens(t, Tc, cfg.window_chunks,
                                       cfg.sink_frames_global * cfg.tokens_per_frame, shot * Tc,
                                       cfg.sink_frames_shot * cfg.tokens_per_frame,
                                       want_list=False)
            assert n.value == ref, (cfg, t)
