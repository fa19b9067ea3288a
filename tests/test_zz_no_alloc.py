"""GPU: the allocation-free KV store (nvfp4_kv_store_chunk_noalloc) against
nvfp4_kv_store_chunk with a workspace, through the C ABI: the same ring bytes
on two calls in a row (the second on a smaller chunk), later chunks of both
rings, and the channel limit."""
import ctypes as C

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


def bf16(bits, shape):
    return torch.from_numpy(bits.view(np.int16).reshape(shape)).view(torch.bfloat16).cuda()


def written_regions(ring, n_slots):
    """The arrays the stores so far have written, each at its exact length
    (the 256-byte alignment padding between them is never written): of the
    first n_slots chunk slots and both sink regions, K and V codes and
    scales, mu and the two decode scales."""
    torch.cuda.synchronize()
    mem = ring.mem.cpu().numpy()[ring._base - ring.mem.data_ptr():]
    r = ring.ring
    cfg = r.cfg
    T, hd = r.chunk_tokens, r.hd
    a = lambda n: (n + 255) // 256 * 256

    def reg(off, ntok):
        out, o = [], off
        for n in (ntok * hd // 2, ntok * hd // 16, ntok * hd // 2, ntok * hd // 16, hd * 4, 8):
            out.append(mem[o:o + n])
            o += a(n)
        return out

    out = []
    for k in range(n_slots):
        out += reg(k * r.slot_bytes, T)
    out += reg(r.gsink_offset, cfg.sink_frames_global * cfg.tokens_per_frame)
    out += reg(r.ssink_offset, cfg.sink_frames_shot * cfg.tokens_per_frame)
    return out


def store_both(nv, cfg, seed, chunks):
    """The same chunks into two rings: one through the C ABI's allocation-free
    entry point, one through the workspace entry point."""
    L = nv.lib()
    r_noalloc, r_ws = nv.KVRing(cfg), nv.KVRing(cfg)
    T, H, d = cfg.chunk_tokens, cfg.heads, cfg.head_dim
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    for t in range(chunks):
        kb, vb = synth.kv_chunk(seed, t, T, H, d)
        K, V = bf16(kb, (T, H, d)), bf16(vb, (T, H, d))
        st = L.nvfp4_kv_store_chunk_noalloc(C.byref(r_noalloc.ring), t, C.c_void_p(K.data_ptr()),
                                            C.c_void_p(V.data_ptr()), None, stream)
        assert st == 0, L.nvfp4_last_error()
        st = L.nvfp4_kv_store_chunk(C.byref(r_ws.ring), t, C.c_void_p(K.data_ptr()),
                                    C.c_void_p(V.data_ptr()), None, C.c_void_p(r_ws.ws.data_ptr()),
                                    r_ws.ws.numel(), stream)
        assert st == 0, L.nvfp4_last_error()
        torch.cuda.synchronize()
    n_slots = min(chunks, cfg.window_chunks)
    for got, want in zip(written_regions(r_noalloc, n_slots), written_regions(r_ws, n_slots)):
        assert np.array_equal(got, want)
    return r_noalloc, r_ws


def test_noalloc_store_matches_workspace_store(nv):
    """Two calls in a row: the 5B model's chunk (7040 x 24 x 128), then a
    smaller one (200 tokens x 3 heads x 32) twice, the second chunk too."""
    print("case: noalloc store 7040x24x128", flush=True)
    big = nv.KVConfig(window_chunks=1)
    store_both(nv, big, 4100, 1)
    print("case: noalloc store 200x3x32, two chunks", flush=True)
    small = nv.KVConfig(tokens_per_frame=40, frames_per_chunk=5, heads=3, head_dim=32,
                        sink_frames_global=2, sink_frames_shot=1, window_chunks=2)
    store_both(nv, small, 4101, 2)


def test_noalloc_store_with_producer_amax_and_gather(nv):
    """Three chunks with a shot cut, the value amax from the producer, and
    the gather of the next step equal between the two entry points."""
    print("case: noalloc store ring with gather", flush=True)
    cfg = nv.KVConfig(tokens_per_frame=16, frames_per_chunk=4, heads=2, head_dim=64,
                      sink_frames_global=1, sink_frames_shot=1, window_chunks=2)
    T, H, d = cfg.chunk_tokens, cfg.heads, cfg.head_dim
    a, b = nv.KVRing(cfg), nv.KVRing(cfg)
    for t in range(3):
        if t == 2:
            a.begin_shot(t)
            b.begin_shot(t)
        kb, vb = synth.kv_chunk(4102, t, T, H, d)
        K, V = bf16(kb, (T, H, d)), bf16(vb, (T, H, d))
        vmax = V.float().abs().max().reshape(1)
        a.store_chunk_noalloc(t, K, V, v_amax=vmax)
        b.store_chunk(t, K, V, v_amax=vmax)
    ka, va = a.gather_window(3)
    kb_, vb_ = b.gather_window(3)
    torch.cuda.synchronize()
    assert torch.equal(ka.view(torch.int16), kb_.view(torch.int16))
    assert torch.equal(va.view(torch.int16), vb_.view(torch.int16))


def test_noalloc_store_channel_limit(nv):
    L = nv.lib()
    cfg = nv.KVConfig(tokens_per_frame=1, frames_per_chunk=1, heads=129, head_dim=128,
                      sink_frames_global=0, sink_frames_shot=0, window_chunks=1)
    c = cfg.c()
    ring = nv.CKvRing()
    FAKE = 0x7F0000000000
    assert L.nvfp4_kv_ring_init(C.byref(ring), C.byref(c), FAKE, 1 << 40) == 0
    st = L.nvfp4_kv_store_chunk_noalloc(C.byref(ring), 0, FAKE, FAKE, None, None)
    assert st == -4 and b"16384" in L.nvfp4_last_error()
