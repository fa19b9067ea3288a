"""CPU oracle of the NVFP4 data path (TEST INFRASTRUCTURE).

A plain, slow, obviously-correct C implementation (nvfp4_oracle.c) behind
ctypes.  Only tests/, the smoke check in __graft_entry__ and the CPU-baseline
leg of bench.py may import this package.  It never imports, and is never
imported by, the GPU library nvfp4_bit_quantization_amd.

Parity pins for every function live in tests/test_oracle_*.py; none of the
oracle's functions is "parity unpinned".
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

LAYOUT_1D = 0
LAYOUT_2D = 1
SEARCH_6 = 0
SEARCH_4O6 = 1

_lib = None


def lib():
    global _lib
    if _lib is None:
        if _build.stale():
            _build.build()
        _lib = C.CDLL(_build.LIB)
        _declare(_lib)
    return _lib


_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_i64 = C.c_int64


def _declare(L):
    L.orc_e2m1_value.argtypes = [C.c_uint8]
    L.orc_e2m1_value.restype = C.c_float
    L.orc_e2m1_encode.argtypes = [C.c_float]
    L.orc_e2m1_encode.restype = C.c_uint8
    L.orc_e4m3_value.argtypes = [C.c_uint8]
    L.orc_e4m3_value.restype = C.c_float
    L.orc_e4m3_encode.argtypes = [C.c_float]
    L.orc_e4m3_encode.restype = C.c_uint8
    L.orc_bf16_rne.argtypes = [C.c_float]
    L.orc_bf16_rne.restype = C.c_uint16
    L.orc_amax.argtypes = [_f32p, _i64]
    L.orc_amax.restype = C.c_float
    L.orc_tensor_scales.argtypes = [C.c_float, C.POINTER(C.c_float), C.POINTER(C.c_float)]
    L.orc_tensor_scales.restype = None
    L.orc_quantize.argtypes = [_f32p, _i64, _i64, C.c_int, C.c_int, C.c_void_p, _u8p, _u8p,
                               C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
    L.orc_quantize.restype = C.c_int
    L.orc_dequant_value.argtypes = [C.c_uint8, C.c_uint8, C.c_float]
    L.orc_dequant_value.restype = C.c_float
    L.orc_dequantize.argtypes = [_u8p, _u8p, C.c_float, _i64, _i64, C.c_int, _f32p]
    L.orc_dequantize.restype = None
    L.orc_to_bf16.argtypes = [_f32p, _i64, _u16p]
    L.orc_to_bf16.restype = None
    L.orc_kv_mean.argtypes = [_f32p, _i64, _i64, _f32p]
    L.orc_kv_mean.restype = None
    L.orc_kv_encode_chunk.argtypes = [_f32p, _f32p, _i64, _i64, C.c_int, _u8p, _u8p,
                                      C.POINTER(C.c_float), _u8p, _u8p, C.POINTER(C.c_float),
                                      _f32p]
    L.orc_kv_encode_chunk.restype = C.c_int
    L.orc_kv_dequant_tokens.argtypes = [_u8p, _u8p, C.c_float, C.c_void_p, _i64, _i64, _i64,
                                        _u16p]
    L.orc_kv_dequant_tokens.restype = None
    L.orc_effective_tokens.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, C.c_void_p]
    L.orc_effective_tokens.restype = _i64
    L.orc_gemm_ref.argtypes = [_u8p, _u8p, C.c_float, _i64, _i64, _u8p, _u8p, C.c_float, _i64,
                               C.c_int, C.c_void_p, _i64, _f64p, C.c_void_p]
    L.orc_gemm_ref.restype = C.c_int
    L.orc_e2m1_encode_array.argtypes = [_f32p, _i64, _u8p]
    L.orc_e2m1_encode_array.restype = None
    L.orc_e4m3_encode_array.argtypes = [_f32p, _i64, _u8p]
    L.orc_e4m3_encode_array.restype = None
    L.orc_rht16.argtypes = [_f32p, _i64, _i64, C.c_uint32, _f32p]
    L.orc_rht16.restype = None
    L.orc_lora_ref.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, _i64, _i64, C.c_float,
                               C.c_void_p, _i64, _f64p, C.c_void_p, C.c_void_p]
    L.orc_lora_ref.restype = C.c_int
    L.orc_attention_ref.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, _i64, _i64, C.c_double,
                                    C.c_void_p, _i64, _f64p, C.c_void_p, C.c_void_p]
    L.orc_attention_ref.restype = C.c_int


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# --------------------------------------------------------------------------
# Formats
# --------------------------------------------------------------------------

def e2m1_value(nib: int) -> float:
    return float(lib().orc_e2m1_value(nib))


def e2m1_encode(y) -> np.ndarray:
    y = _f32(y)
    out = np.empty(y.shape, np.uint8)
    lib().orc_e2m1_encode_array(y.reshape(-1), y.size, out.reshape(-1))
    return out


def e4m3_value(code: int) -> float:
    return float(lib().orc_e4m3_value(code))


def e4m3_encode(t) -> np.ndarray:
    t = _f32(t)
    out = np.empty(t.shape, np.uint8)
    lib().orc_e4m3_encode_array(t.reshape(-1), t.size, out.reshape(-1))
    return out


def bf16_rne(x) -> np.ndarray:
    x = _f32(x)
    out = np.empty(x.shape, np.uint16)
    lib().orc_to_bf16(x.reshape(-1), x.size, out.reshape(-1))
    return out


def tensor_scales(amax: float):
    e, d = C.c_float(), C.c_float()
    lib().orc_tensor_scales(float(amax), C.byref(e), C.byref(d))
    return np.float32(e.value), np.float32(d.value)


# --------------------------------------------------------------------------
# Quantize / dequantize
# --------------------------------------------------------------------------

def quantize(x, layout: int = LAYOUT_1D, search: int = SEARCH_4O6, amax=None,
             return_errors: bool = False):
    """x float32 [R, C] -> (codes u8 [R, C/2], scales u8, s_dec float32[, err6, err4])."""
    x = _f32(x)
    R, Cc = x.shape
    codes = np.zeros((R, Cc // 2), np.uint8)
    nsc = (R // 16 if layout == LAYOUT_2D else R) * (Cc // 16)
    scales = np.zeros(nsc, np.uint8)
    sdec = C.c_float()
    amax_c = C.c_float(float(amax)) if amax is not None else None
    e6 = np.zeros(nsc, np.float32) if return_errors else None
    e4 = np.zeros(nsc, np.float32) if return_errors else None
    rc = lib().orc_quantize(x.reshape(-1), R, Cc, layout, search,
                            C.cast(C.byref(amax_c), C.c_void_p) if amax_c is not None else None,
                            codes.reshape(-1) if codes.size else np.zeros(1, np.uint8),
                            scales if nsc else np.zeros(1, np.uint8), C.byref(sdec),
                            e6.ctypes.data if e6 is not None else None,
                            e4.ctypes.data if e4 is not None else None)
    if rc != 0:
        raise ValueError(f"orc_quantize: bad shape {x.shape} for layout {layout}")
    shape = (R // 16, Cc // 16) if layout == LAYOUT_2D else (R, Cc // 16)
    out = (codes, scales.reshape(shape), np.float32(sdec.value))
    if return_errors:
        out = out + (e6.reshape(shape), e4.reshape(shape))
    return out


def dequantize(codes, scales, s_dec, layout: int = LAYOUT_1D) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    R, half = codes.shape
    out = np.empty((R, half * 2), np.float32)
    if out.size:
        lib().orc_dequantize(codes.reshape(-1), np.ascontiguousarray(scales, np.uint8).reshape(-1),
                             float(s_dec), R, half * 2, layout, out.reshape(-1))
    return out


def amax(x) -> np.float32:
    x = _f32(x)
    return np.float32(lib().orc_amax(x.reshape(-1), x.size))


def rht16(x, signs: int) -> np.ndarray:
    """Random Hadamard transform of every 1x16 block of float32 x [R, C]
    (C % 16 == 0): (1/4) H16 diag(s) x by the fp32 butterfly; bit j of
    `signs` set flips element j of each block."""
    x = _f32(x)
    R, Cc = x.shape
    out = np.empty_like(x)
    if x.size:
        lib().orc_rht16(x.reshape(-1), R, Cc, int(signs) & 0xFFFF, out.reshape(-1))
    return out


def quantize_rht(x, signs: int, search: int = SEARCH_4O6, amax=None):
    """RHT then 1-D quantize: (codes, scales, s_dec) of rht16(x, signs)."""
    return quantize(rht16(x, signs), layout=LAYOUT_1D, search=search, amax=amax)


# --------------------------------------------------------------------------
# KV cache
# --------------------------------------------------------------------------

def kv_mean(K) -> np.ndarray:
    """K float32 [T, HD] -> per-channel mean float32 [HD]."""
    K = _f32(K)
    T, HD = K.shape
    mu = np.empty(HD, np.float32)
    lib().orc_kv_mean(K.reshape(-1), T, HD, mu)
    return mu


def kv_encode_chunk(K, V, search: int = SEARCH_4O6, threads: int = 1, rows=None) -> dict:
    """K, V float32 [T, HD] (bf16 values) -> packed chunk dict.

    threads == 1 and rows is None: one call of the C routine
    orc_kv_encode_chunk.  Otherwise the same encoding assembled from the C
    routines by a driver: the key mean over the whole chunk (orc_kv_mean),
    K_s = RN(K - mu) (one float32 subtraction per element), the tensor amax
    of K_s and of V over the whole chunk, then orc_quantize with that amax on
    contiguous row ranges, `threads` of them at once (ctypes releases the GIL
    during each C call; the blocks of a row depend only on the row and the
    tensor scale, so the split changes nothing).  With `rows` (token indices)
    only those tokens are encoded (the statistics still cover every token):
    the arrays then hold those rows, in the order given.
    """
    K = _f32(K)
    V = _f32(V)
    T, HD = K.shape
    if threads <= 1 and rows is None:
        kc = np.zeros((T, HD // 2), np.uint8)
        ks = np.zeros((T, HD // 16), np.uint8)
        vc = np.zeros((T, HD // 2), np.uint8)
        vs = np.zeros((T, HD // 16), np.uint8)
        mu = np.zeros(HD, np.float32)
        sdk, sdv = C.c_float(), C.c_float()
        rc = lib().orc_kv_encode_chunk(K.reshape(-1), V.reshape(-1), T, HD, search,
                                       kc.reshape(-1), ks.reshape(-1), C.byref(sdk),
                                       vc.reshape(-1), vs.reshape(-1), C.byref(sdv), mu)
        if rc != 0:
            raise RuntimeError("orc_kv_encode_chunk failed")
        return dict(kc=kc, ks=ks, sdk=np.float32(sdk.value), vc=vc, vs=vs,
                    sdv=np.float32(sdv.value), mu=mu)
    mu = kv_mean(K)
    Ks = K - mu[None, :]
    ak, av = amax(Ks), amax(V)
    if rows is not None:
        rows = np.asarray(rows, np.int64)
        Ks, V = np.ascontiguousarray(Ks[rows]), np.ascontiguousarray(V[rows])
    n = Ks.shape[0]
    parts = max(1, min(threads, n // 16)) if n else 1
    cuts = [n * i // parts for i in range(parts + 1)]

    def enc(i):
        a, b = cuts[i], cuts[i + 1]
        return quantize(Ks[a:b], search=search, amax=ak), quantize(V[a:b], search=search, amax=av)

    if parts > 1:
        from concurrent.futures import ThreadPoolExecutor

        with ThreadPoolExecutor(parts) as ex:
            out = list(ex.map(enc, range(parts)))
    else:
        out = [enc(0)]
    cat = lambda j, which: np.concatenate([o[which][j] for o in out]) if n else \
        np.zeros((0, HD // (2 if j == 0 else 16)), np.uint8)
    sdk = tensor_scales(ak)[1]
    sdv = tensor_scales(av)[1]
    return dict(kc=cat(0, 0), ks=cat(1, 0), sdk=sdk, vc=cat(0, 1), vs=cat(1, 1), sdv=sdv, mu=mu)


def kv_dequant_rows(chunk: dict, key: bool, threads: int = 1) -> np.ndarray:
    """bf16 bits of every row of an encoded chunk (the whole chunk, or the
    rows it was encoded for), `threads` row ranges at once."""
    n = chunk["kc"].shape[0]
    parts = max(1, min(threads, n // 16)) if n else 1
    cuts = [n * i // parts for i in range(parts + 1)]
    if parts == 1:
        return kv_dequant_tokens(chunk, 0, n, key)
    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(parts) as ex:
        out = list(ex.map(lambda i: kv_dequant_tokens(chunk, cuts[i], cuts[i + 1] - cuts[i], key),
                          range(parts)))
    return np.concatenate(out)


def kv_dequant_tokens(chunk: dict, tok0: int, ntok: int, key: bool) -> np.ndarray:
    """bf16 bits [ntok, HD] of tokens [tok0, tok0+ntok) of an encoded chunk."""
    codes = chunk["kc"] if key else chunk["vc"]
    scales = chunk["ks"] if key else chunk["vs"]
    sd = chunk["sdk"] if key else chunk["sdv"]
    HD = codes.shape[1] * 2
    out = np.empty((ntok, HD), np.uint16)
    if ntok:
        mu = chunk["mu"] if key else None
        lib().orc_kv_dequant_tokens(codes.reshape(-1), scales.reshape(-1), float(sd),
                                    mu.ctypes.data if mu is not None else None, tok0, ntok, HD,
                                    out.reshape(-1))
    return out


def effective_tokens(t: int, Tc: int, W: int, g_tokens: int, s_start: int, s_tokens: int,
                     want_list: bool = True):
    """E(t) as an int64 array of global token indices (ascending)."""
    n = lib().orc_effective_tokens(t, Tc, W, g_tokens, s_start, s_tokens, None)
    if not want_list:
        return int(n)
    out = np.empty(max(n, 1), np.int64)
    lib().orc_effective_tokens(t, Tc, W, g_tokens, s_start, s_tokens, out.ctypes.data)
    return out[:n]


def gather_window(chunks: dict, t: int, Tc: int, W: int, g_tokens: int, s_start: int,
                  s_tokens: int):
    """Oracle gather: dequantized K, V (bf16 bits [n, HD]) of E(t).

    ``chunks`` maps chunk index -> kv_encode_chunk() result.  Sinks are byte
    copies of their source chunk's leading tokens, so every token is read
    from its own chunk's encoding.
    """
    toks = effective_tokens(t, Tc, W, g_tokens, s_start, s_tokens)
    HD = next(iter(chunks.values()))["kc"].shape[1] * 2 if chunks else 0
    Kout = np.empty((len(toks), HD), np.uint16)
    Vout = np.empty((len(toks), HD), np.uint16)
    i = 0
    while i < len(toks):
        c = int(toks[i] // Tc)
        j = i
        while j < len(toks) and toks[j] // Tc == c and toks[j] - toks[i] == j - i:
            j += 1
        tok0 = int(toks[i] - c * Tc)
        Kout[i:j] = kv_dequant_tokens(chunks[c], tok0, j - i, key=True)
        Vout[i:j] = kv_dequant_tokens(chunks[c], tok0, j - i, key=False)
        i = j
    return toks, Kout, Vout


# --------------------------------------------------------------------------
# GEMM
# --------------------------------------------------------------------------

def gemm_ref(a_codes, a_scales, a_sdec, w_codes, w_scales, w_sdec, w_layout: int = LAYOUT_2D,
             rows=None):
    """fp64 reference Y [len(rows) or M, N] and the abs-sum bound term."""
    a_codes = np.ascontiguousarray(a_codes, np.uint8)
    w_codes = np.ascontiguousarray(w_codes, np.uint8)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = w_codes.shape[0]
    if rows is not None:
        rows = np.ascontiguousarray(rows, np.int64)
        nr = len(rows)
    else:
        nr = M
    y = np.empty((nr, N), np.float64)
    s = np.empty((nr, N), np.float64)
    rc = lib().orc_gemm_ref(a_codes.reshape(-1), np.ascontiguousarray(a_scales, np.uint8).reshape(-1),
                            float(a_sdec), M, K, w_codes.reshape(-1),
                            np.ascontiguousarray(w_scales, np.uint8).reshape(-1), float(w_sdec), N,
                            w_layout, rows.ctypes.data if rows is not None else None, nr,
                            y.reshape(-1), s.ctypes.data)
    if rc != 0:
        raise RuntimeError("orc_gemm_ref failed")
    return y, s


def lora_ref(x, a, b, scale: float, rows=None):
    """LoRA branch of the frozen-backbone linear layer: (alpha/r) XA B^T with
    XA = bf16(x A^T).  x [M, K], a [r, K], b [N, r] float32 (bf16 values).
    Returns (y fp64 [len(rows) or M, N], abs-sum bound term, XA float32 [M, r])."""
    x, a, b = _f32(x), _f32(a), _f32(b)
    M, K = x.shape
    r = a.shape[0]
    N = b.shape[0]
    if a.shape[1] != K or b.shape[1] != r:
        raise ValueError("lora_ref: shapes do not chain")
    if rows is not None:
        rows = np.ascontiguousarray(rows, np.int64)
    nr = len(rows) if rows is not None else M
    y = np.empty((nr, N), np.float64)
    s = np.empty((nr, N), np.float64)
    xa = np.zeros((M, r), np.float32)
    rc = lib().orc_lora_ref(x.reshape(-1), a.reshape(-1), b.reshape(-1), M, K, N, r,
                            float(scale), rows.ctypes.data if rows is not None else None, nr,
                            y.reshape(-1), s.ctypes.data, xa.ctypes.data)
    if rc != 0:
        raise RuntimeError("orc_lora_ref failed")
    return y, s, xa


# --------------------------------------------------------------------------
# Attention over the effective set
# --------------------------------------------------------------------------

def attention_ref(q, k, v, scale: float, rows=None):
    """Softmax attention per head in double: q [nq, H, d], k and v [nk, H, d]
    float32 (bf16 values).  Returns (o fp64 [len(rows) or nq, H, d],
    sum_j w_j |v_j| / sum_j w_j of the same shape, lse fp64 [.., H])."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    nq, H, d = q.shape
    nk = k.shape[0]
    if k.shape != (nk, H, d) or v.shape != (nk, H, d):
        raise ValueError("attention_ref: k and v must be [nk, H, d] like q")
    if rows is not None:
        rows = np.ascontiguousarray(rows, np.int64)
    nr = len(rows) if rows is not None else nq
    o = np.empty((nr, H, d), np.float64)
    ao = np.empty((nr, H, d), np.float64)
    lse = np.empty((nr, H), np.float64)
    kk = k.reshape(-1) if k.size else np.zeros(1, np.float32)
    vv = v.reshape(-1) if v.size else np.zeros(1, np.float32)
    rc = lib().orc_attention_ref(q.reshape(-1), kk, vv, nq, nk, H, d, float(scale),
                                 rows.ctypes.data if rows is not None else None, nr,
                                 o.reshape(-1), ao.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise RuntimeError("orc_attention_ref failed")
    return o, ao, lse
