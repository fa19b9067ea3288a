"""GPU parity: quantize / dequantize through the C ABI vs the CPU oracle.

Bar: codes, scales and s_dec bit-exact; dequantized values bit-exact.
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
    assert torch.cuda.is_available()
    return m


def to_gpu(x32: np.ndarray, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32))
    return t.to(dtype).cuda()


def oracle_input(x32: np.ndarray, dtype):
    """The exact float32 values the GPU sees (bf16 rounding happens in the input)."""
    if dtype == torch.bfloat16:
        return synth.bf16_bits_to_f32(synth.to_bf16_bits(x32))
    return np.ascontiguousarray(x32, np.float32)


def check_quant(nv, orc, x32, dtype, layout, search, amax=None):
    xg = to_gpu(x32, dtype)
    xo = oracle_input(x32, dtype)
    amax_t = None
    if amax is not None:
        amax_t = torch.tensor([amax], dtype=torch.float32, device="cuda")
    q = nv.quantize(xg, layout=layout, search=search, amax_in=amax_t)
    c_ref, s_ref, d_ref = orc.quantize(xo, layout=layout, search=search, amax=amax)
    torch.cuda.synchronize()
    c = q.codes.cpu().numpy()
    s = q.scales.cpu().numpy()
    assert np.float32(q.s_dec).view(np.uint32) == np.float32(d_ref).view(np.uint32)
    bad = np.argwhere(c != c_ref)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:4].tolist()}"
    assert np.array_equal(s, s_ref)
    return q, (c_ref, s_ref, d_ref)


@pytest.mark.parametrize("search", [1, 0])
def test_quantize_1d_cfg1_fp32(nv, orc, search):
    print("case: 1-D fp32 4096x128 (round-trip workload), search", search, flush=True)
    x = synth.activations(1001, 0, 4096, 128, 0.01, 20.0)
    q, ref = check_quant(nv, orc, x, torch.float32, 0, search)
    y = nv.dequantize(q, dtype=torch.float32).cpu().numpy()
    y_ref = orc.dequantize(*ref)
    assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))


# 174776 x 48: 524,328 blocks on the 512 x 256 lanes of the 1-D encode, so
# the lanes' last loop iteration holds a fifth block for lanes 0..39 only
# (a partial wave) and empty slots for everyone else.
@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (1001, 3072), (257, 14336), (174776, 48)])
def test_quantize_1d_bf16_shapes(nv, orc, rows, cols):
    print("case: 1-D bf16", rows, cols, flush=True)
    x = synth.activations(1003, rows, rows, cols, 0.005, 30.0)
    q, ref = check_quant(nv, orc, x, torch.bfloat16, 0, 1)
    y = nv.dequantize(q, dtype=torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, orc.bf16_rne(orc.dequantize(*ref)))


@pytest.mark.parametrize("rows,cols,dtype", [(16, 16, torch.float32), (256, 512, torch.float32),
                                             (3072, 3072, torch.bfloat16),
                                             (48, 80, torch.bfloat16)])
def test_quantize_2d(nv, orc, rows, cols, dtype):
    print("case: 2-D", rows, cols, dtype, flush=True)
    w = synth.weights(1003, rows + cols, rows, cols)
    q, ref = check_quant(nv, orc, w, dtype, 1, 1)
    y = nv.dequantize(q, dtype=torch.float32).cpu().numpy()
    assert np.array_equal(y.view(np.uint32), orc.dequantize(*ref, layout=1).view(np.uint32))


def test_quantize_amax_in(nv, orc):
    x = synth.activations(1001, 9, 640, 256, 0.01, 20.0)
    check_quant(nv, orc, x, torch.float32, 0, 1, amax=float(np.abs(x).max()) * 1.5)


def test_quantize_zero_and_signed_zero(nv, orc):
    x = np.zeros((64, 64), np.float32)
    x[1::2] = -0.0
    check_quant(nv, orc, x, torch.float32, 0, 1)
    check_quant(nv, orc, x, torch.float32, 1, 1)


def test_quantize_wide_dynamic_range(nv, orc):
    # blocks whose scale underflows to zero and blocks at the largest scale
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((512, 256)) * np.exp2(rng.integers(-40, 20, (512, 1)))).astype(np.float32)
    check_quant(nv, orc, x, torch.float32, 0, 1)
    check_quant(nv, orc, x, torch.float32, 0, 0)


def test_quantize_subnormal_blocks(nv, orc):
    # blocks of subnormal values next to normal ones: block amax below 2^-125
    rng = np.random.default_rng(13)
    x = rng.standard_normal((256, 128)).astype(np.float32)
    x[::3, :64] = (rng.standard_normal((86, 64)) * 1e-39).astype(np.float32)
    x[1::5, 64:80] = np.float32(2.0 ** -149)
    check_quant(nv, orc, x, torch.float32, 0, 1)
    check_quant(nv, orc, x, torch.float32, 1, 1)


def test_quantize_empty(nv):
    x = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    q = nv.quantize(x)
    y = nv.dequantize(q)
    torch.cuda.synchronize()
    assert y.shape == (0, 32)


def test_quantize_deterministic(nv):
    x = to_gpu(synth.activations(1001, 3, 2048, 3072, 0.005, 30.0), torch.bfloat16)
    a = nv.quantize(x)
    b = nv.quantize(x)
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)


def test_quantize_full_size_activation_sampled(nv, orc):
    """Activations 7040x3072 bf16 at full size: the tensor scale from the full
    tensor, codes and scales of 256 sampled rows (first and last included)."""
    print("case: 1-D bf16 7040x3072 sampled", flush=True)
    x = synth.activations(1003, 0, 7040, 3072, 0.005, 30.0)
    xo = oracle_input(x, torch.bfloat16)
    q = nv.quantize(to_gpu(x, torch.bfloat16))
    amax = float(orc.amax(xo))
    rows = np.unique(np.concatenate([[0, 7039], np.random.default_rng(0).integers(0, 7040, 254)]))
    c_ref, s_ref, d_ref = orc.quantize(xo[rows], amax=amax)
    torch.cuda.synchronize()
    assert q.s_dec == d_ref
    assert np.array_equal(q.codes.cpu().numpy()[rows], c_ref)
    assert np.array_equal(q.scales.cpu().numpy()[rows], s_ref)


def test_quantize_1d_fp32_past_2gib_sampled(nv, orc):
    """fp32 input of 2^29 + 524288 elements (2.15 GB): past the 2^31-byte
    limit of the buffer-offset encoder, so the pointer path runs.  The tensor
    scale comes from the whole input; codes and scales of 64 sampled rows
    (first and last included) against the oracle."""
    rows_n, cols = (1 << 20) + 1024, 512
    print("case: 1-D fp32", rows_n, "x", cols, flush=True)
    x = np.random.default_rng(1008).standard_normal((rows_n, cols), dtype=np.float32)
    x[7, :16] *= 50.0  # one outlier block sets the tensor scale
    q = nv.quantize(torch.from_numpy(x).cuda())
    amax = float(orc.amax(x))
    rows = np.unique(np.concatenate([[0, 7, rows_n - 1],
                                     np.random.default_rng(9).integers(0, rows_n, 61)]))
    c_ref, s_ref, d_ref = orc.quantize(x[rows], amax=amax)
    torch.cuda.synchronize()
    assert q.s_dec == d_ref
    idx = torch.from_numpy(rows).cuda()
    assert np.array_equal(q.codes[idx].cpu().numpy(), c_ref)
    assert np.array_equal(q.scales[idx].cpu().numpy(), s_ref)
