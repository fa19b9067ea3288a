"""GPU parity: W4A4 GEMM vs the oracle's fp64 product.

Bar (fp32 output): |y - y_ref| <= 1e-5 * s_A s_W sum_k |A_hat W_hat|;
bf16 output adds the output rounding, 2^-8 |y_ref|.  Operands are quantized by
the oracle on the CPU and uploaded, so the GEMM is checked on its own.
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


def upload(nv, codes, scales, s_dec, layout):
    rows, half = codes.shape
    t = nv.NVFP4Tensor.empty(rows, half * 2, layout)
    t.codes.copy_(torch.from_numpy(codes))
    t.scales.copy_(torch.from_numpy(np.ascontiguousarray(scales).reshape(t.scales.shape)))
    t.s_dec_bits[0] = int(np.float32(s_dec).view(np.int32))
    return t


def operands(orc, M, N, K, seed, w_std=None):
    A = synth.activations(seed, 1, M, K, 0.01, 20.0)
    if w_std is None:
        W = synth.activations(seed, 2, N, K, 0.01, 20.0)
    else:
        W = synth.weights(seed, 2, N, K, w_std)
    qa = orc.quantize(A)
    qw = orc.quantize(W, layout=orc.LAYOUT_2D)
    return qa, qw


def check(nv, orc, qa, qw, out_dtype, rows=None):
    a = upload(nv, *qa, 0)
    w = upload(nv, *qw, 1)
    y = nv.gemm_w4a4(a, w, out_dtype=out_dtype)
    yr, bound = orc.gemm_ref(*qa, *qw, rows=rows)
    torch.cuda.synchronize()
    yg = y.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        yg = yg[rows]
    tol = 1e-5 * bound
    if out_dtype == torch.bfloat16:
        tol = tol + 2.0 ** -8 * np.abs(yr)
    err = np.abs(yg - yr)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), f"max excess at {worst}: err {err[worst]} tol {tol[worst]}"
    return yg, yr


def test_gemm_cfg1_fp32(nv, orc):
    print("case: gemm 256x256x512 fp32", flush=True)
    qa, qw = operands(orc, 256, 256, 512, 1001)
    check(nv, orc, qa, qw, torch.float32)


def test_gemm_cfg1_bf16(nv, orc):
    qa, qw = operands(orc, 256, 256, 512, 1001)
    check(nv, orc, qa, qw, torch.bfloat16)


@pytest.mark.parametrize("M,N,K", [(1, 16, 16), (100, 48, 80), (129, 144, 272), (300, 272, 64)])
def test_gemm_ragged(nv, orc, M, N, K):
    print("case: gemm ragged", M, N, K, flush=True)
    qa, qw = operands(orc, M, N, K, 1003)
    check(nv, orc, qa, qw, torch.float32)


def test_gemm_exact_integer_case(nv, orc):
    """All block scales 1.0 and s_dec = 1: every partial sum is a multiple of
    1/4 below 2^22, so the result must be exact in any summation order."""
    rng = np.random.default_rng(5)
    M, N, K = 192, 160, 320
    ca = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    cw = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    qa = (ca, np.full((M, K // 16), 0x38, np.uint8), np.float32(1.0))
    qw = (cw, np.full((N // 16, K // 16), 0x38, np.uint8), np.float32(1.0))
    a = upload(nv, *qa, 0)
    w = upload(nv, *qw, 1)
    y = nv.gemm_w4a4(a, w, out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    yr, _ = orc.gemm_ref(*qa, *qw)
    assert np.array_equal(y, yr)


def test_gemm_k_zero_and_m_zero(nv):
    a = nv.NVFP4Tensor.empty(0, 64)
    w = nv.NVFP4Tensor.empty(32, 64, 1)
    w.s_dec_bits.zero_()
    y = nv.gemm_w4a4(a, w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert y.shape == (0, 32)


def test_gemm_attention_projection_sampled(nv, orc):
    """7040x3072 activations times 3072x3072 weights (the attention projection
    shape), 48 sampled rows (first and last M tile included)."""
    print("case: gemm 7040x3072x3072 sampled", flush=True)
    qa, qw = operands(orc, 7040, 3072, 3072, 1003, w_std=0.02)
    # on 256 CUs rows 0..4095 go in 256-row tiles and 4096..7039 in 192-row
    # tiles: both sides of that boundary and of the 192-row tiles' edges
    rows = np.unique(np.concatenate([[0, 1, 127, 4095, 4096, 4287, 4288, 6912, 6911, 7039],
                                     np.random.default_rng(1).integers(0, 7040, 43)]))
    check(nv, orc, qa, qw, torch.bfloat16, rows=rows)


@pytest.mark.parametrize("K", [512, 272])
def test_gemm_256_row_tiles_only(nv, orc, K):
    """4096 x 3072: on 256 CUs exactly one round of 256-row tiles, so no row
    goes to a 192-row tile; K = 272 takes the general (per-lane load) path."""
    print("case: gemm 4096x3072 all 256-row tiles, K", K, flush=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus == 256:
        assert nv.gemm_plan(4096, 3072, cus) == (4096, 256)
    qa, qw = operands(orc, 4096, 3072, K, 1006, w_std=0.02)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 4095],
                                     np.random.default_rng(3).integers(0, 4096, 40)]))
    check(nv, orc, qa, qw, torch.float32, rows=rows)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_gemm_split_tiles_ragged_tail(nv, orc, out_dtype):
    """4296 x 3072 x 512: on 256 CUs 272 tiles of 256 rows would take two
    rounds, so rows 4096..4295 go in two 192-row tiles (the second holds 8
    rows); every output row near the boundaries and a random sample."""
    print("case: gemm 4296x3072x512 split tiles", out_dtype, flush=True)
    qa, qw = operands(orc, 4296, 3072, 512, 1005, w_std=0.02)
    rows = np.unique(np.concatenate([np.arange(4088, 4296),
                                     np.random.default_rng(2).integers(0, 4088, 40)]))
    check(nv, orc, qa, qw, out_dtype, rows=rows)


@pytest.mark.parametrize("N,K", [(14336, 3072), (3072, 14336)], ids=["ffn_up", "ffn_down"])
def test_gemm_ffn_shapes_sampled(nv, orc, N, K):
    """The FFN projections at full size (M = 7040): the GPU quantizes the whole
    bf16 activation, the oracle quantizes the sampled rows with the exact
    tensor amax (1-D blocks are independent once the tensor scale is fixed)
    and takes the fp64 product with the oracle-quantized weight."""
    print("case: gemm ffn", 7040, N, K, flush=True)
    M = 7040
    A = synth.bf16_bits_to_f32(synth.to_bf16_bits(synth.activations(1004, 0, M, K, 0.005, 30.0)))
    W = synth.weights(1004, 1 if N > K else 2, N, K)
    qw = orc.quantize(W, layout=orc.LAYOUT_2D)
    rows = np.unique(np.concatenate([[0, 255, 6912, M - 1],
                                     np.random.default_rng(2).integers(0, M, 28)]))
    qa_rows = orc.quantize(A[rows], amax=float(np.abs(A).max()))
    a = nv.quantize(torch.from_numpy(A).cuda().to(torch.bfloat16))
    w = upload(nv, *qw, 1)
    y = nv.gemm_w4a4(a, w, out_dtype=torch.bfloat16)
    yr, bound = orc.gemm_ref(*qa_rows, *qw)
    torch.cuda.synchronize()
    yg = y[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    tol = 1e-5 * bound + 2.0 ** -8 * np.abs(yr)
    err = np.abs(yg - yr)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), f"max excess at {worst}: err {err[worst]} tol {tol[worst]}"


def test_gemm_deterministic(nv, orc):
    qa, qw = operands(orc, 512, 384, 1024, 1007)
    a = upload(nv, *qa, 0)
    w = upload(nv, *qw, 1)
    y1 = nv.gemm_w4a4(a, w, out_dtype=torch.float32)
    y2 = nv.gemm_w4a4(a, w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("K", [512, 272])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_gemm_amax_out(nv, orc, K, out_dtype):
    """amax_out is max|Y| of the stored values (bit-exact), so requantizing Y
    with it as amax_in gives the same codes, scales and s_dec as a plain
    quantize of Y."""
    print("case: gemm amax_out", K, out_dtype, flush=True)
    qa, qw = operands(orc, 300, 272, K, 1005)
    a = upload(nv, *qa, 0)
    w = upload(nv, *qw, 1)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    y = nv.gemm_w4a4(a, w, out_dtype=out_dtype, amax_out=amax)
    ref = y.float().abs().max()
    torch.cuda.synchronize()
    assert amax.item() == ref.item() and amax.item() > 0
    q1 = nv.quantize(y)
    q2 = nv.quantize(y, amax_in=amax)
    torch.cuda.synchronize()
    assert q1.s_dec == q2.s_dec
    assert torch.equal(q1.codes, q2.codes) and torch.equal(q1.scales, q2.scales)
    # a larger preset value is kept
    big = torch.full((1,), 1e30, dtype=torch.float32, device="cuda")
    nv.gemm_w4a4(a, w, out_dtype=out_dtype, amax_out=big)
    torch.cuda.synchronize()
    assert big.item() == np.float32(1e30)
