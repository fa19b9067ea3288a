"""GPU parity: LoRA on the frozen NVFP4 backbone.

lora_down: XA = bf16(x A^T) within one bf16 rounding of the exact product
(plus the fp32 accumulation bound).  gemm_w4a4_lora: the W4A4 bar
1e-5 * sum_k |a_k b_k| on the backbone part, plus, on the adapter part,
2^-7 * (alpha/r) * sum_j |XA_j B_j| (XA may sit one bf16 rounding from the
oracle's), plus the bf16 output rounding.
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


def bf16(x32):
    return synth.bf16_bits_to_f32(synth.to_bf16_bits(np.ascontiguousarray(x32, np.float32)))


def gpu_bf16(x32):
    return torch.from_numpy(bf16(x32)).to(torch.bfloat16).cuda()


def upload(nv, codes, scales, s_dec, layout):
    rows, half = codes.shape
    t = nv.NVFP4Tensor.empty(rows, half * 2, layout)
    t.codes.copy_(torch.from_numpy(codes))
    t.scales.copy_(torch.from_numpy(np.ascontiguousarray(scales).reshape(t.scales.shape)))
    t.s_dec_bits[0] = int(np.float32(s_dec).view(np.int32))
    return t


@pytest.mark.parametrize("r", [16, 32, 64, 128])
def test_lora_down(nv, orc, r):
    print("case: lora_down r", r, flush=True)
    M, K = 300, 1024
    x = bf16(synth.activations(1031, 0, M, K, 0.01, 20.0))
    a = bf16(synth.weights(1031, 1, r, K, 0.05))
    xa = nv.lora_down(gpu_bf16(x), gpu_bf16(a)).float().cpu().numpy().astype(np.float64)
    exact = x.astype(np.float64) @ a.astype(np.float64).T
    bound = np.abs(x.astype(np.float64)) @ np.abs(a.astype(np.float64)).T
    err = np.abs(xa - exact)
    assert np.all(err <= 2.0 ** -8 * np.abs(exact) + 2.0 ** -20 * bound)


@pytest.mark.parametrize("M,N,K,r", [(300, 272, 512, 16), (129, 144, 288, 32), (256, 192, 1024, 64)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gemm_lora(nv, orc, M, N, K, r, out_dtype):
    print("case: gemm_lora", M, N, K, r, out_dtype, flush=True)
    x = bf16(synth.activations(1032, 0, M, K, 0.01, 20.0))
    w0 = synth.weights(1032, 1, N, K)
    la = bf16(synth.weights(1032, 2, r, K, 0.05))
    lb = bf16(synth.weights(1032, 3, N, r, 0.05))
    scale = np.float32(16.0 / r)
    qa = orc.quantize(x)
    qw = orc.quantize(w0, layout=orc.LAYOUT_2D)
    a, w = upload(nv, *qa, 0), upload(nv, *qw, 1)
    xa = nv.lora_down(gpu_bf16(x), gpu_bf16(la))
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    y = nv.gemm_w4a4_lora(a, w, xa, gpu_bf16(lb), float(scale), out_dtype=out_dtype, amax_out=amax)
    y_main, b_main = orc.gemm_ref(*qa, *qw)
    y_lora, b_lora, _ = orc.lora_ref(x, la, lb, scale)
    torch.cuda.synchronize()
    yg = y.float().cpu().numpy().astype(np.float64)
    ref = y_main + y_lora
    tol = 1e-5 * b_main + 2.0 ** -7 * b_lora
    if out_dtype == torch.bfloat16:
        tol = tol + 2.0 ** -8 * np.abs(ref)
    err = np.abs(yg - ref)
    assert np.all(err <= tol), f"max excess {np.max(err - tol)}"
    assert amax.item() == y.float().abs().max().item()


def test_lora_validation(nv):
    x = torch.zeros((32, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError):
        nv.lora_down(x, torch.zeros((24, 64), dtype=torch.bfloat16, device="cuda"))  # r = 24
    with pytest.raises(RuntimeError):
        nv.lora_down(torch.zeros((32, 48), dtype=torch.bfloat16, device="cuda"),
                     torch.zeros((16, 48), dtype=torch.bfloat16, device="cuda"))  # K % 32
