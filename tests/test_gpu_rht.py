"""GPU parity: random-Hadamard-transform quantize and the GEMM with a 1-D W.

Bar: codes, scales and s_dec of nvfp4_quantize_rht bit-exact against the
oracle's quantize_rht (rht16 then the 1-D quantizer); the GEMM with a 1-D
scaled W within 1e-5 * sum_k |a_k b_k| of the oracle's fp64 product.
"""
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


def as_f32(x32, dtype):
    if dtype == torch.bfloat16:
        return synth.bf16_bits_to_f32(synth.to_bf16_bits(x32))
    return np.ascontiguousarray(x32, np.float32)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("signs", [0x0000, 0xFFFF, 0xB7E1])
def test_quantize_rht_matches_oracle(nv, orc, dtype, signs):
    print("case: quantize_rht", dtype, hex(signs), flush=True)
    x = synth.activations(1011, 0, 1031, 768, 0.01, 30.0)
    q = nv.quantize_rht(torch.from_numpy(x).to(dtype).cuda(), signs)
    c_ref, s_ref, d_ref = orc.quantize_rht(as_f32(x, dtype), signs)
    torch.cuda.synchronize()
    assert np.float32(q.s_dec).view(np.uint32) == np.float32(d_ref).view(np.uint32)
    c = q.codes.cpu().numpy()
    bad = np.argwhere(c != c_ref)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:4].tolist()}"
    assert np.array_equal(q.scales.cpu().numpy().reshape(s_ref.shape), s_ref)


def test_quantize_rht_amax_in_and_search6(nv, orc):
    x = synth.activations(1012, 0, 64, 4096, 0.02, 20.0)
    xo = as_f32(x, torch.float32)
    amax = float(np.abs(orc.rht16(xo, 0x5A5A)).max()) * 1.25
    g = torch.from_numpy(x).cuda()
    q = nv.quantize_rht(g, 0x5A5A, search=0,
                        amax_in=torch.tensor([amax], dtype=torch.float32, device="cuda"))
    c_ref, s_ref, d_ref = orc.quantize_rht(xo, 0x5A5A, search=0, amax=amax)
    torch.cuda.synchronize()
    assert q.s_dec == d_ref
    assert np.array_equal(q.codes.cpu().numpy(), c_ref)
    assert np.array_equal(q.scales.cpu().numpy().reshape(s_ref.shape), s_ref)


@pytest.mark.parametrize("M,N,K", [(300, 272, 512), (129, 100, 272), (64, 512, 1024)])
def test_gemm_1d_weight_matches_oracle(nv, orc, M, N, K):
    """Both operands 1-D (the weight-gradient GEMM's layout), RHT'd along K."""
    print("case: gemm 1-D W", M, N, K, flush=True)
    A = synth.activations(1013, 1, M, K, 0.01, 20.0)
    W = synth.activations(1013, 2, N, K, 0.01, 20.0)
    qa = nv.quantize_rht(torch.from_numpy(A).cuda(), 0x2D4B)
    qw = nv.quantize_rht(torch.from_numpy(W).cuda(), 0x2D4B)
    y = nv.gemm_w4a4(qa, qw, out_dtype=torch.float32)
    ca, sa, da = orc.quantize_rht(A, 0x2D4B)
    cw, sw, dw = orc.quantize_rht(W, 0x2D4B)
    yr, bound = orc.gemm_ref(ca, sa, da, cw, sw, dw, w_layout=orc.LAYOUT_1D)
    torch.cuda.synchronize()
    err = np.abs(y.cpu().numpy().astype(np.float64) - yr)
    assert np.all(err <= 1e-5 * bound), f"max excess {np.max(err - 1e-5 * bound)}"
