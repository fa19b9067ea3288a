"""GPU checks of the MXFP4 speed reference (not part of the method).

The MX path is compared with NVFP4 for speed and error only; here it is
checked against its own definition (OCP Microscaling v1.0 MXFP4, as the C
header states it): the quantizer bit-exactly against a numpy statement of the
rule (element rounding by the oracle's E2M1 encoder), the GEMM against the
fp64 product of the decoded MX operands with the W4A4 tolerance
1e-5 * sum_k |a_k b_k| (plus the bf16 output rounding).
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_quantization_amd as m

    m.lib()
    return m


def mx_ref(orc, x32: np.ndarray):
    """(codes [rows, cols/2], scales [rows, cols/32]) of float32 x."""
    rows, cols = x32.shape
    xb = x32.reshape(rows, cols // 32, 32)
    am = np.abs(xb).max(axis=2).astype(np.float32)
    be = ((am.view(np.uint32) >> 23) & 0xFF).astype(np.int64)
    e = np.clip(np.where(be == 0, -127, be - 129), -127, 127)
    inv = np.ldexp(np.float32(1.0), -e).astype(np.float32)
    y = (xb * inv[..., None]).astype(np.float32)
    nib = orc.e2m1_encode(y).reshape(rows, cols)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = np.where(am == 0, 0, e + 127).astype(np.uint8)
    return codes, scales


def mx_decode(codes, scales):
    rows, half = codes.shape
    nib = np.empty((rows, half * 2), np.uint8)
    nib[:, 0::2] = codes & 15
    nib[:, 1::2] = codes >> 4
    v = E2M1[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    s = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return v * np.repeat(s, 32, axis=1)


def gpu(x32, dtype):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(dtype).cuda()


def as_f32(x32, dtype):
    if dtype == torch.bfloat16:
        return synth.bf16_bits_to_f32(synth.to_bf16_bits(x32))
    return np.ascontiguousarray(x32, np.float32)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_mx_quantize_matches_rule(nv, orc, dtype):
    print("case: mx_quantize", dtype, flush=True)
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((300, 512)) * np.exp2(rng.integers(-30, 30, (300, 1)))).astype(np.float32)
    x[3, :32] = 0.0                           # all-zero block
    x[4, 32:64] = np.float32(1e-39)           # subnormal amax
    x[5, 64:96] = np.float32(7.9) * np.exp2(rng.integers(-5, 5, 32)).astype(np.float32)
    x[6, 96:128] = np.float32(3.0e38)         # near the top of the range
    codes, scales = nv.mx_quantize(gpu(x, dtype))
    c_ref, s_ref = mx_ref(orc, as_f32(x, dtype))
    torch.cuda.synchronize()
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    c = codes.cpu().numpy()
    bad = np.argwhere(c != c_ref)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("M,N,K", [(256, 192, 512), (300, 200, 768), (1, 32, 256)])
def test_gemm_mx_matches_decoded_product(nv, M, N, K):
    print("case: gemm_mx", M, N, K, flush=True)
    A = synth.activations(1007, 1, M, K, 0.01, 20.0)
    W = synth.weights(1007, 2, N, K)
    qa = nv.mx_quantize(gpu(A, torch.bfloat16))
    qw = nv.mx_quantize(gpu(W, torch.bfloat16))
    for out_dtype in (torch.float32, torch.bfloat16):
        y = nv.gemm_mx(qa, qw, out_dtype=out_dtype).float().cpu().numpy().astype(np.float64)
        a = mx_decode(qa[0].cpu().numpy(), qa[1].cpu().numpy())
        w = mx_decode(qw[0].cpu().numpy(), qw[1].cpu().numpy())
        ref = a @ w.T
        tol = 1e-5 * (np.abs(a) @ np.abs(w).T)
        if out_dtype == torch.bfloat16:
            tol = tol + 2.0 ** -8 * np.abs(ref)
        err = np.abs(y - ref)
        assert np.all(err <= tol), f"max excess {np.max(err - tol)}"


def test_mx_validation(nv):
    x = torch.zeros((4, 48), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError):
        nv.mx_quantize(x)  # cols % 32 != 0
    q = nv.mx_quantize(torch.zeros((32, 128), dtype=torch.float32, device="cuda"))
    with pytest.raises(RuntimeError):
        nv.gemm_mx(q, q)  # K = 128 is not a multiple of 256
