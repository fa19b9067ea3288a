"""GPU parity at the rounding points of the hardware converters.

The quantizer's bit-exactness rests on gfx950's converters rounding to
nearest with ties to even: v_cvt_scalef32_pk_fp4_f32 for the E2M1 codes,
v_cvt_pk_fp8_f32 for the E4M3 block scales, v_cvt_pk_bf16_f32 for bf16
outputs.  Random data almost never lands on a tie, so these tests put the
converters' inputs on every rounding midpoint of the E2M1 grid and of the
E4M3 grid, and next to them, through nvfp4_quantize / nvfp4_dequantize, and
compare bytes with the oracle (whose encoders are nearest-value searches, not
converters) and, where the answer is fixed by hand, with that answer.

With amax_in = 2688 the tensor scales are s_enc = s_dec = 1, so a block
whose amax is 6 * sigma (sigma a power of two) has scale sigma, decode scale
S = sigma and encode multiplier r = 1/sigma, all exact: the E2M1 converter
sees x / sigma exactly.  A block whose amax is 6 * m has the ideal scale
RN(6 m / 6) = m exactly, so the E4M3 converter sees m.
"""
import numpy as np
import pytest
import torch

from test_oracle_quant import TIE_BLOCKS, tie_block

pytestmark = pytest.mark.gpu

E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_quantization_amd as m

    m.lib()
    assert torch.cuda.is_available()
    return m


def e4m3_values():
    """The 127 non-negative finite E4M3FN values from the bit layout (bias 7,
    subnormals m * 2^-9), ascending."""
    out = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        out.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(out)


def run(nv, orc, x, dtype, layout=0, search=1):
    """nvfp4_quantize with amax_in = 2688 against the oracle, bytes compared."""
    amax = torch.tensor([2688.0], dtype=torch.float32, device="cuda")
    xg = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dtype).cuda()
    xo = xg.float().cpu().numpy()  # the values the GPU sees
    q = nv.quantize(xg, layout=layout, search=search, amax_in=amax)
    c_ref, s_ref, d_ref = orc.quantize(xo, layout=layout, search=search, amax=2688.0)
    torch.cuda.synchronize()
    c, s = q.codes.cpu().numpy(), q.scales.cpu().numpy()
    assert q.s_dec == 1.0 and d_ref == 1.0
    bad = np.argwhere(c != c_ref)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:4].tolist()}"
    bad = np.argwhere(s != s_ref)
    assert bad.size == 0, f"{len(bad)} scale bytes differ, first at {bad[:4].tolist()}"
    return c, s, xo


def e2m1_blocks(dtype):
    """Blocks of 16: element 0 = 6 sigma (the block amax), the rest sigma * y
    for every E2M1 midpoint y, its neighbours one float (or one bf16) either
    side, both signs, and -0; sigma over powers of two from 2^-8 (an E4M3
    subnormal) to 2^8.  Plus blocks whose amax is one step above 6 sigma
    (saturation to 6)."""
    if dtype == torch.float32:
        up = np.nextafter(E2M1_MIDPOINTS, np.float32(np.inf))
        dn = np.nextafter(E2M1_MIDPOINTS, np.float32(0))
    else:  # neighbours on the bf16 grid: the adjacent bf16 bit patterns
        b = (E2M1_MIDPOINTS.view(np.uint32) >> 16).astype(np.uint32)
        up = ((b + 1) << 16).view(np.float32)
        dn = ((b - 1) << 16).view(np.float32)
    y = np.concatenate([E2M1_MIDPOINTS, up, dn]).astype(np.float32)
    y = np.concatenate([y, -y, [np.float32(-0.0), np.float32(0.0), np.float32(6.0)]])
    nfill = -len(y) % 15
    y = np.concatenate([y, np.zeros(nfill, np.float32)]).reshape(-1, 15)
    blocks = []
    for k in (-8, -3, -1, 0, 1, 4, 8):
        sig = np.float32(2.0 ** k)
        b = np.empty((y.shape[0], 16), np.float32)
        b[:, 0] = 6 * sig
        b[:, 1:] = y * sig
        blocks.append(b)
        sat = b.copy()
        step = np.float32(2.0 ** (k + 2 - (23 if dtype == torch.float32 else 7)))
        sat[:, 0] = 6 * sig + step  # RN(amax / 6) still rounds to sigma
        sat[:, 1] = -(6 * sig + step)
        blocks.append(sat)
    return np.concatenate(blocks)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("search", [0, 1], ids=["search6", "search4o6"])
def test_e2m1_midpoints(nv, orc, dtype, search):
    print("case: E2M1 midpoints", dtype, search, flush=True)
    x = e2m1_blocks(dtype)
    c, s, xo = run(nv, orc, x, dtype, search=search)
    if search == 0:
        # the hand answer for the exact midpoints: ties go to the even code
        nib = np.stack([c & 0xF, c >> 4], axis=-1).reshape(c.shape[0], 16)
        sig = np.ldexp(1.0, (np.floor(np.log2(np.abs(xo[:, 0]) / 6))).astype(int))
        yv = xo[:, 1:] / sig[:, None]
        even = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
        for mid, k in even.items():
            for sgn in (1, -1):
                hit = yv == sgn * mid
                assert np.all(nib[:, 1:][hit] == (k | (8 if sgn < 0 else 0))), (mid, sgn)


def test_e2m1_midpoints_2d(nv, orc):
    """The 2-D encoder on the same values: 16 rows of one 16x16 tile share
    the block amax (row 0's element 0)."""
    print("case: E2M1 midpoints 2-D", flush=True)
    x = e2m1_blocks(torch.float32)
    n = x.shape[0] // 16 * 16
    run(nv, orc, x[:n], torch.float32, layout=1, search=1)


def e4m3_blocks(target=6):
    """Blocks whose ideal scale for `target` (6 or 4) is every midpoint m of
    the E4M3 grid (126 of them, 2^-10 between 0 and the smallest subnormal
    included), m + d and m - d with d = 2^(floor(log2 m) - 18) (so
    target * (m +- d) stays exact), and 448, 464 and 500 (saturation); the
    other 15 elements a fixed spread of fractions of the amax."""
    v = e4m3_values()
    mids = (v[:-1] + v[1:]) / 2
    d = np.ldexp(1.0, (np.floor(np.log2(mids)) - 18).astype(int))
    ideal = np.concatenate([mids, mids + d, mids - d, [448.0, 464.0, 500.0]])
    frac = np.linspace(-0.97, 0.97, 15).astype(np.float32)
    x = np.empty((len(ideal), 16), np.float32)
    x[:, 0] = (target * ideal).astype(np.float32)
    assert np.all(x[:, 0].astype(np.float64) == target * ideal)  # exact
    x[:, 1:] = x[:, :1] * frac[None, :]
    return x, ideal


def test_e4m3_midpoints_scale_bytes(nv, orc):
    print("case: E4M3 midpoints", flush=True)
    x, ideal = e4m3_blocks()
    _, s, _ = run(nv, orc, x, torch.float32, search=0)
    # the hand answer: nearest E4M3 value, ties to the even code, >= 448 -> 0x7E
    v = e4m3_values()
    for i, t in enumerate(ideal):
        if t >= 448:
            want = 0x7E
        else:
            dist = np.abs(v - t)
            cands = np.flatnonzero(dist == dist.min())
            want = int(cands[0] if len(cands) == 1 else cands[cands % 2 == 0][0])
        assert s[i, 0] == want, (t, hex(s[i, 0]), hex(want))


@pytest.mark.parametrize("scale_by", [6, 4])
def test_e4m3_midpoints_four_over_six(nv, orc, scale_by):
    """Both candidates through the converter: amax 6 m puts the target-6
    ideal on m, amax 4 m the target-4 ideal."""
    print("case: E4M3 midpoints 4/6, amax = %d m" % scale_by, flush=True)
    x, _ = e4m3_blocks(scale_by)
    run(nv, orc, x, torch.float32, search=1)
    run(nv, orc, x, torch.bfloat16, search=1)


@pytest.mark.parametrize("vals,err,codes", TIE_BLOCKS, ids=["tie_nonzero", "tie_zero"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_four_over_six_tie_keeps_six(nv, orc, vals, err, codes, dtype):
    """A block whose two candidates have exactly equal error keeps target 6
    (scale 0x38) in the 1-D and the 2-D encoder."""
    print("case: 4/6 tie", vals, dtype, flush=True)
    x = np.repeat(tie_block(vals), 16, axis=0)
    c, s, _ = run(nv, orc, x, dtype, layout=0, search=1)
    assert np.all(s == 0x38) and all(list(r) == codes for r in c)
    c2, s2, _ = run(nv, orc, x, dtype, layout=1, search=1)
    assert s2[0, 0] == 0x38 and all(list(r) == codes for r in c2)


# (s_dec, whether V * sigma * s_dec hits a bf16 midpoint for some code)
BF16_TIE_CASES = [(1 + 2.0 ** -8, True), (1 + 3 * 2.0 ** -8, True), (1 - 2.0 ** -9, True),
                  (1 + 2.0 ** -8 + 2.0 ** -23, False), (1 + 2.0 ** -8 - 2.0 ** -23, False),
                  (0.75 + 2.0 ** -10, False)]


@pytest.mark.parametrize("s_dec,has_tie", BF16_TIE_CASES,
                         ids=lambda v: np.float32(v).view(np.uint32).tobytes().hex()
                         if not isinstance(v, bool) else str(v))
def test_dequantize_bf16_midpoints(nv, orc, s_dec, has_tie):
    """bf16 output of values on and next to bf16 midpoints: every code with
    power-of-two block scales 2^-4..2^4 and decode scales S = sigma * s_dec
    chosen so V * S lands on a bf16 rounding midpoint for some V."""
    print("case: dequantize bf16 midpoints", s_dec, flush=True)
    rows, cols = 9, 256
    codes = np.tile(np.arange(128, dtype=np.uint8), (rows, 1))
    codes[:, 64:] += 128
    codes = np.ascontiguousarray(codes)
    sig_codes = np.array([0x18, 0x20, 0x28, 0x30, 0x38, 0x40, 0x48, 0x50, 0x58], np.uint8)
    scales = np.ascontiguousarray(np.repeat(sig_codes[:, None], cols // 16, axis=1))
    bits = int(np.float32(s_dec).view(np.int32))
    t = nv.NVFP4Tensor(codes=torch.from_numpy(codes).cuda(), scales=torch.from_numpy(scales).cuda(),
                       s_dec_bits=torch.tensor([bits, 0, 0, 0], dtype=torch.int32, device="cuda"),
                       rows=rows, cols=cols, layout=0)
    y16 = nv.dequantize(t, dtype=torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16)
    y32 = nv.dequantize(t, dtype=torch.float32).cpu().numpy()
    ref = orc.dequantize(codes, scales, np.float32(s_dec))
    assert np.array_equal(y32.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(y16, orc.bf16_rne(ref))
    # a float whose low 16 bits are 0x8000 lies exactly between two bf16 values
    ties = int(np.count_nonzero((ref.view(np.uint32) & 0xFFFF) == 0x8000))
    assert (ties > 0) == has_tie, ties
