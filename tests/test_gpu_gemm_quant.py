"""GPU parity: the W4A4 GEMM with its epilogue encoding Y to NVFP4.

The fused output must be nvfp4_quantize(bf16(Y), search, amax_in) bit for bit.
Against the oracle this is checked where Y itself is exact in fp32 whatever
the summation order: power-of-two block scales (0.5, 1, 2) and tensor scales
make every product a multiple of 2^-4 below 144 in magnitude, so partial sums
stay below 2^19 (K <= 3072) and need at most 23 significant bits; the oracle's
fp64 product is then the GPU's fp32 one, and the oracle quantizes its bf16
rounding with the same amax.  On general operands the fused output is checked
against the two-call path (GEMM to bf16, then quantize with the GEMM's
amax_out), each call pinned to the oracle by its own tests.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

POW2_SCALES = np.array([0x30, 0x38, 0x40], np.uint8)  # E4M3 0.5, 1, 2


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_quantization_amd as m

    m.lib()
    return m


def upload(nv, codes, scales, s_dec, layout):
    rows, half = codes.shape
    t = nv.NVFP4Tensor.empty(rows, half * 2, layout)
    t.codes.copy_(torch.from_numpy(codes))
    t.scales.copy_(torch.from_numpy(np.ascontiguousarray(scales).reshape(t.scales.shape)))
    t.s_dec_bits[0] = int(np.float32(s_dec).view(np.int32))
    return t


def exact_operands(seed, M, N, K, w_layout):
    rng = np.random.default_rng(seed)
    ca = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    cw = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa = POW2_SCALES[rng.integers(0, 3, (M, K // 16))]
    nsw = N // 16 if w_layout == 1 else N
    sw = POW2_SCALES[rng.integers(0, 3, (nsw, K // 16))]
    return (ca, sa, np.float32(0.25)), (cw, sw, np.float32(8.0))


def bf16_of(orc, y):
    """The oracle's bf16 rounding of y, as float32 values."""
    bits = orc.bf16_rne(np.asarray(y, np.float32)).astype(np.uint32) << 16
    return bits.view(np.float32)


def device_amax(v):
    return torch.tensor([float(v)], dtype=torch.float32, device="cuda")


def check_against_oracle(nv, orc, qa, qw, w_layout, amax, search, rows=None):
    a, w = upload(nv, *qa, 0), upload(nv, *qw, w_layout)
    M, N = a.rows, w.rows
    amax_out = torch.zeros(1, dtype=torch.float32, device="cuda")
    yq = nv.gemm_w4a4_quant(a, w, device_amax(amax), search=search, amax_out=amax_out)
    y_ref, _ = orc.gemm_ref(*qa, *qw, w_layout=w_layout, rows=rows)
    yb = bf16_of(orc, y_ref)
    codes, scales, s_dec = orc.quantize(yb, search=search, amax=amax)
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else torch.from_numpy(rows).cuda()
    gc = yq.codes[sel].cpu().numpy()
    gs = yq.scales[sel].cpu().numpy()
    bad = np.argwhere(gc != codes)
    assert bad.size == 0, f"codes differ at {bad[:4].tolist()}"
    assert np.array_equal(gs, scales)
    assert yq.s_dec_bits[0].item() == int(np.float32(s_dec).view(np.int32))
    if rows is None:
        assert amax_out.item() == float(np.abs(yb).max())
    return yb


@pytest.mark.parametrize("M,N,K,w_layout", [(300, 272, 512, 1), (300, 272, 320, 1),
                                            (256, 208, 512, 0), (33, 16, 256, 1)],
                         ids=["lds_path", "general_path", "w_1d", "tiny"])
@pytest.mark.parametrize("search", [1, 0], ids=["4o6", "6only"])
@pytest.mark.parametrize("amax_mode", ["exact", "stale", "headroom", "zero"])
def test_gemm_quant_exact_vs_oracle(nv, orc, M, N, K, w_layout, search, amax_mode):
    print("case: gemm_quant exact", M, N, K, w_layout, search, amax_mode, flush=True)
    qa, qw = exact_operands(2001, M, N, K, w_layout)
    y_ref, _ = orc.gemm_ref(*qa, *qw, w_layout=w_layout)
    true_amax = float(np.abs(bf16_of(orc, y_ref)).max())
    amax = {"exact": true_amax, "stale": 0.5 * true_amax, "headroom": 3.0 * true_amax,
            "zero": 0.0}[amax_mode]  # zero: tensor scales 1 and 1, large values saturate
    check_against_oracle(nv, orc, qa, qw, w_layout, amax, search)


def test_gemm_quant_ffn_up_sampled(nv, orc):
    """7040 x 14336 x 3072 (the FFN up-projection) in the exact construction;
    the oracle computes 32 sampled rows (first and last M tiles included) and
    quantizes them with the amax the GPU is given."""
    print("case: gemm_quant ffn up 7040x14336x3072 sampled", flush=True)
    M, N, K = 7040, 14336, 3072
    qa, qw = exact_operands(2002, M, N, K, 1)
    rows = np.unique(np.concatenate([[0, 255, 6912, M - 1],
                                     np.random.default_rng(3).integers(0, M, 28)]))
    y_rows, _ = orc.gemm_ref(*qa, *qw, rows=rows)
    amax = 0.9 * float(np.abs(y_rows).max())
    check_against_oracle(nv, orc, qa, qw, 1, amax, 1, rows=rows)


@pytest.mark.parametrize("M,N,K", [(300, 272, 512), (7040, 3072, 3072)])
def test_gemm_quant_matches_two_call_path(nv, orc, M, N, K):
    print("case: gemm_quant vs gemm + quantize", M, N, K, flush=True)
    A = synth.activations(2003, 0, M, K, 0.005, 30.0)
    W = synth.weights(2003, 1, N, K)
    a = upload(nv, *orc.quantize(A), 0)
    w = upload(nv, *orc.quantize(W, layout=orc.LAYOUT_2D), 1)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    y = nv.gemm_w4a4(a, w, out_dtype=torch.bfloat16, amax_out=amax)
    ref = nv.quantize(y, amax_in=amax)
    amax2 = torch.zeros(1, dtype=torch.float32, device="cuda")
    yq = nv.gemm_w4a4_quant(a, w, amax, amax_out=amax2)
    torch.cuda.synchronize()
    assert torch.equal(yq.codes, ref.codes)
    assert torch.equal(yq.scales, ref.scales)
    assert yq.s_dec_bits[0].item() == ref.s_dec_bits[0].item()
    assert amax2.item() == amax.item()


def test_gemm_quant_empty(nv, orc):
    a = nv.NVFP4Tensor.empty(0, 64)
    w = nv.NVFP4Tensor.empty(32, 64, 1)
    w.s_dec_bits.zero_()
    yq = nv.gemm_w4a4_quant(a, w, device_amax(100.0))
    _, s_dec = orc.tensor_scales(100.0)
    torch.cuda.synchronize()
    assert yq.codes.shape == (0, 16)
    assert yq.s_dec_bits[0].item() == int(np.float32(s_dec).view(np.int32))
