"""nvfp4_bit_quantization_amd -- Python binding of libnvfp4 (MI355X / gfx950).

Argument marshalling only: every step of the NVFP4 path runs in the HIP
kernels of libnvfp4.so, called through its C ABI (include/nvfp4.h).  PyTorch
provides device memory and the current stream.  There is no CPU fallback: if
the library is not built, or the device is not a GPU, the calls raise.

Entry points mirror the C ABI:
    quantize, dequantize, gemm_w4a4, KVRing (kv_ring_init, kv_begin_shot,
    kv_store_chunk, kv_effective_tokens, gather_window)
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1
LAYOUT_1D = 0
LAYOUT_2D = 1
SEARCH_6 = 0
SEARCH_4O6 = 1
KV_MAX_WINDOW = 16

_STATUS = {0: "ok", -1: "EINVAL", -2: "EALIGN", -3: "ESHAPE", -4: "ENOSPC", -5: "ESTATE",
           -6: "EHIP"}


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class CTensor(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("s_dec", C.c_void_p),
                ("rows", C.c_int64), ("cols", C.c_int64), ("layout", C.c_int32),
                ("reserved", C.c_int32)]


class CKvConfig(C.Structure):
    _fields_ = [("tokens_per_frame", C.c_int32), ("frames_per_chunk", C.c_int32),
                ("heads", C.c_int32), ("head_dim", C.c_int32),
                ("sink_frames_global", C.c_int32), ("sink_frames_shot", C.c_int32),
                ("window_chunks", C.c_int32), ("search", C.c_int32)]


class CKvRing(C.Structure):
    _fields_ = [("cfg", CKvConfig), ("base", C.c_void_p), ("bytes", C.c_uint64),
                ("chunk_tokens", C.c_int64), ("hd", C.c_int64), ("slot_bytes", C.c_int64),
                ("gsink_offset", C.c_int64), ("ssink_offset", C.c_int64),
                ("next_chunk", C.c_int64), ("g_end", C.c_int64), ("s_start", C.c_int64)]


_lib = None

_EXPORTS = {
    "nvfp4_abi_version": ([], C.c_int),
    "nvfp4_build_hash": ([], C.c_char_p),
    "nvfp4_status_string": ([C.c_int], C.c_char_p),
    "nvfp4_last_error": ([], C.c_char_p),
    "nvfp4_codes_bytes": ([C.c_int64, C.c_int64], C.c_size_t),
    "nvfp4_scales_bytes": ([C.c_int64, C.c_int64, C.c_int32], C.c_size_t),
    "nvfp4_quantize_workspace_bytes": ([C.c_int64, C.c_int64, C.c_int32], C.c_size_t),
    "nvfp4_quantize": ([C.c_void_p, C.c_int32, C.POINTER(CTensor), C.c_int32, C.c_void_p,
                        C.c_void_p, C.c_size_t, C.c_void_p], C.c_int),
    "nvfp4_dequantize": ([C.POINTER(CTensor), C.c_void_p, C.c_int32, C.c_void_p], C.c_int),
    "nvfp4_quantize_rht": ([C.c_void_p, C.c_int32, C.POINTER(CTensor), C.c_int32, C.c_uint32,
                            C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p], C.c_int),
    "nvfp4_gemm_w4a4": ([C.POINTER(CTensor), C.POINTER(CTensor), C.c_void_p, C.c_int32,
                         C.c_void_p, C.c_void_p], C.c_int),
    "nvfp4_gemm_w4a4_quant": ([C.POINTER(CTensor), C.POINTER(CTensor), C.POINTER(CTensor),
                               C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p], C.c_int),
    "nvfp4_lora_down": ([C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p,
                         C.c_void_p], C.c_int),
    "nvfp4_gemm_w4a4_lora": ([C.POINTER(CTensor), C.POINTER(CTensor), C.c_void_p, C.c_void_p,
                              C.c_int64, C.c_float, C.c_void_p, C.c_int32, C.c_void_p,
                              C.c_void_p], C.c_int),
    "nvfp4_mx_quantize": ([C.c_void_p, C.c_int32, C.c_int64, C.c_int64, C.c_void_p,
                           C.c_void_p, C.c_void_p], C.c_int),
    "nvfp4_gemm_mx": ([C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_int64,
                       C.c_int64, C.c_void_p, C.c_int32, C.c_void_p], C.c_int),
    "nvfp4_gemm_plan": ([C.c_int64, C.c_int64, C.c_int32, C.POINTER(C.c_int64),
                         C.POINTER(C.c_int64)], C.c_int),
    "nvfp4_kv_ring_bytes": ([C.POINTER(CKvConfig)], C.c_size_t),
    "nvfp4_kv_store_workspace_bytes": ([C.POINTER(CKvConfig)], C.c_size_t),
    "nvfp4_kv_ring_init": ([C.POINTER(CKvRing), C.POINTER(CKvConfig), C.c_void_p, C.c_size_t],
                           C.c_int),
    "nvfp4_kv_begin_shot": ([C.POINTER(CKvRing), C.c_int64], C.c_int),
    "nvfp4_kv_store_chunk": ([C.POINTER(CKvRing), C.c_int64, C.c_void_p, C.c_void_p,
                              C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p], C.c_int),
    "nvfp4_kv_store_chunk_noalloc": ([C.POINTER(CKvRing), C.c_int64, C.c_void_p, C.c_void_p,
                                      C.c_void_p, C.c_void_p], C.c_int),
    "nvfp4_kv_effective_tokens": ([C.POINTER(CKvRing), C.c_int64, C.POINTER(C.c_int64)],
                                  C.c_int),
    "nvfp4_gather_window": ([C.POINTER(CKvRing), C.c_int64, C.c_void_p, C.c_void_p, C.c_int64,
                             C.POINTER(C.c_int64), C.c_void_p], C.c_int),
    "nvfp4_attention_window": ([C.POINTER(CKvRing), C.c_int64, C.c_void_p, C.c_int64, C.c_float,
                                C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t,
                                C.c_void_p], C.c_int),
    "nvfp4_attention_plan": ([C.POINTER(CKvRing), C.c_int64, C.c_int64, C.c_int32,
                              C.POINTER(C.c_int32), C.POINTER(C.c_size_t)], C.c_int),
    "nvfp4_profile_enable": ([C.c_int], C.c_int),
    "nvfp4_profile_collect": ([C.c_char_p, C.c_int, C.c_void_p, C.c_void_p, C.c_int], C.c_int),
}


def lib():
    """The loaded libnvfp4.so (raises if it has not been built, or was built
    from other sources than the ones beside it)."""
    global _lib
    if _lib is None:
        from . import build as _build

        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run python -m "
                               "nvfp4_bit_quantization_amd.build")
        L = C.CDLL(LIB_PATH)
        L.nvfp4_build_hash.restype = C.c_char_p
        built, now = L.nvfp4_build_hash().decode(), _build.source_hash()
        if built != now:
            raise RuntimeError(f"{LIB_PATH} was built from other sources (digest {built}, "
                               f"sources {now}): rebuild with python -m "
                               "nvfp4_bit_quantization_amd.build")
        for name, (args, res) in _EXPORTS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise NVFP4Error(status, lib().nvfp4_last_error().decode())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return C.c_void_p(t.data_ptr())


_DT = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}


# --------------------------------------------------------------------------
# NVFP4 tensors
# --------------------------------------------------------------------------

@dataclass
class NVFP4Tensor:
    """Packed NVFP4 tensor on the GPU.

    codes  uint8 [rows, cols/2]; scales uint8 (E4M3FN bytes) [rows, cols/16]
    (1-D) or [rows/16, cols/16] (2-D); s_dec_bits int32 [1]: the raw bits of
    the FP32 tensor decode scale, kept in an integer tensor so that a dtype
    cast of a module cannot alter it.
    """
    codes: torch.Tensor
    scales: torch.Tensor
    s_dec_bits: torch.Tensor
    rows: int
    cols: int
    layout: int

    @staticmethod
    def empty(rows: int, cols: int, layout: int = LAYOUT_1D, device="cuda") -> "NVFP4Tensor":
        nsr = rows // 16 if layout == LAYOUT_2D else rows
        return NVFP4Tensor(
            codes=torch.empty((rows, cols // 2), dtype=torch.uint8, device=device),
            scales=torch.empty((nsr, cols // 16), dtype=torch.uint8, device=device),
            s_dec_bits=torch.empty(4, dtype=torch.int32, device=device),
            rows=rows, cols=cols, layout=layout)

    @property
    def s_dec(self) -> float:
        return float(self.s_dec_bits[:1].view(torch.float32).item())

    def c(self) -> CTensor:
        return CTensor(self.codes.data_ptr(), self.scales.data_ptr(), self.s_dec_bits.data_ptr(),
                       self.rows, self.cols, self.layout, 0)


def quantize_workspace_bytes(rows: int, cols: int, layout: int = LAYOUT_1D) -> int:
    return int(lib().nvfp4_quantize_workspace_bytes(rows, cols, layout))


def quantize(x: torch.Tensor, layout: int = LAYOUT_1D, search: int = SEARCH_4O6,
             amax_in: torch.Tensor | None = None, out: NVFP4Tensor | None = None,
             workspace: torch.Tensor | None = None, stream=None) -> NVFP4Tensor:
    """nvfp4_quantize: x (GPU, float32 or bfloat16, [rows, cols]) -> NVFP4Tensor."""
    if x.dim() != 2:
        raise ValueError("quantize expects a 2-D tensor")
    if x.dtype not in _DT:
        raise ValueError(f"unsupported dtype {x.dtype}")
    rows, cols = x.shape
    if out is None:
        out = NVFP4Tensor.empty(rows, cols, layout, x.device)
    if workspace is None and amax_in is None:
        workspace = torch.empty(quantize_workspace_bytes(rows, cols, layout), dtype=torch.uint8,
                                device=x.device)
    ct = out.c()
    _check(lib().nvfp4_quantize(
        _dev(x, "x"), _DT[x.dtype], C.byref(ct), search,
        C.c_void_p(amax_in.data_ptr()) if amax_in is not None else None,
        C.c_void_p(workspace.data_ptr()) if workspace is not None else None,
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream)))
    return out


def quantize_rht(x: torch.Tensor, signs: int, search: int = SEARCH_4O6,
                 amax_in: torch.Tensor | None = None, out: NVFP4Tensor | None = None,
                 workspace: torch.Tensor | None = None, stream=None) -> NVFP4Tensor:
    """nvfp4_quantize_rht: random Hadamard transform of every 1x16 block
    (16-bit sign mask `signs`), then 1-D NVFP4 quantize."""
    if x.dim() != 2 or x.dtype not in _DT:
        raise ValueError("quantize_rht expects a 2-D float32 or bfloat16 tensor")
    rows, cols = x.shape
    if out is None:
        out = NVFP4Tensor.empty(rows, cols, LAYOUT_1D, x.device)
    if workspace is None and amax_in is None:
        workspace = torch.empty(quantize_workspace_bytes(rows, cols, LAYOUT_1D),
                                dtype=torch.uint8, device=x.device)
    ct = out.c()
    _check(lib().nvfp4_quantize_rht(
        _dev(x, "x"), _DT[x.dtype], C.byref(ct), search, int(signs),
        C.c_void_p(amax_in.data_ptr()) if amax_in is not None else None,
        C.c_void_p(workspace.data_ptr()) if workspace is not None else None,
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream)))
    return out


def dequantize(t: NVFP4Tensor, dtype=torch.bfloat16, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """nvfp4_dequantize: NVFP4Tensor -> [rows, cols] float32 or bfloat16."""
    if out is None:
        out = torch.empty((t.rows, t.cols), dtype=dtype, device=t.codes.device)
    ct = t.c()
    _check(lib().nvfp4_dequantize(C.byref(ct), _dev(out, "out"), _DT[out.dtype],
                                  _stream(stream)))
    return out


def gemm_w4a4(a: NVFP4Tensor, w: NVFP4Tensor, out_dtype=torch.bfloat16,
              out: torch.Tensor | None = None, amax_out: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """nvfp4_gemm_w4a4: Y[M, N] = s_A s_W A_hat W_hat^T (A 1-D, W 2-D).

    amax_out: optional one-element float32 device tensor, raised to
    max(amax_out, max|Y|) (set it to 0 first for a fresh maximum)."""
    if out is None:
        out = torch.empty((a.rows, w.rows), dtype=out_dtype, device=a.codes.device)
    if amax_out is not None and (amax_out.dtype != torch.float32 or amax_out.numel() != 1
                                 or not amax_out.is_cuda):
        raise ValueError("amax_out must be a one-element float32 device tensor")
    ca, cw = a.c(), w.c()
    _check(lib().nvfp4_gemm_w4a4(C.byref(ca), C.byref(cw), _dev(out, "out"), _DT[out.dtype],
                                 None if amax_out is None else amax_out.data_ptr(),
                                 _stream(stream)))
    return out


def _amax_arg(t, name):
    if t is not None and (t.dtype != torch.float32 or t.numel() != 1 or not t.is_cuda):
        raise ValueError(f"{name} must be a one-element float32 device tensor")
    return None if t is None else t.data_ptr()


def gemm_w4a4_quant(a: NVFP4Tensor, w: NVFP4Tensor, amax_in: torch.Tensor,
                    search: int = SEARCH_4O6, out: NVFP4Tensor | None = None,
                    amax_out: torch.Tensor | None = None, stream=None) -> NVFP4Tensor:
    """nvfp4_gemm_w4a4_quant: the W4A4 product encoded by the GEMM's epilogue
    to a 1-D NVFP4Tensor [M, N], with the tensor amax taken from amax_in (a
    one-element float32 device tensor).  amax_out as in gemm_w4a4."""
    if out is None:
        out = NVFP4Tensor.empty(a.rows, w.rows, LAYOUT_1D, a.codes.device)
    if amax_in is None:
        raise ValueError("gemm_w4a4_quant needs amax_in")
    pin, pout = _amax_arg(amax_in, "amax_in"), _amax_arg(amax_out, "amax_out")
    ca, cw, cy = a.c(), w.c(), out.c()
    _check(lib().nvfp4_gemm_w4a4_quant(C.byref(ca), C.byref(cw), C.byref(cy), search, pin, pout,
                                       _stream(stream)))
    return out


def gemm_plan(M: int, N: int, compute_units: int):
    """nvfp4_gemm_plan: (rows in 256-row tiles, workgroups) of the W4A4 grid
    for an M x N output on `compute_units` CUs (pure host)."""
    r, g = C.c_int64(), C.c_int64()
    _check(lib().nvfp4_gemm_plan(M, N, compute_units, C.byref(r), C.byref(g)))
    return r.value, g.value


def lora_down(x: torch.Tensor, a: torch.Tensor, out: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """nvfp4_lora_down: XA = bf16(x A^T); x [M, K], a [r, K] bfloat16."""
    if x.dtype != torch.bfloat16 or a.dtype != torch.bfloat16 or x.dim() != 2 or a.dim() != 2:
        raise ValueError("lora_down expects 2-D bfloat16 x and a")
    M, K = x.shape
    r = a.shape[0]
    if a.shape[1] != K:
        raise ValueError("lora_down: K mismatch")
    if out is None:
        out = torch.empty((M, r), dtype=torch.bfloat16, device=x.device)
    _check(lib().nvfp4_lora_down(_dev(x, "x"), _dev(a, "a"), M, K, r, _dev(out, "out"),
                                 _stream(stream)))
    return out


def gemm_w4a4_lora(a: NVFP4Tensor, w: NVFP4Tensor, xa: torch.Tensor, b: torch.Tensor,
                   lora_scale: float, out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
                   amax_out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """nvfp4_gemm_w4a4_lora: W4A4 product plus lora_scale * XA B^T
    (xa [M, r], b [N, r] bfloat16)."""
    if xa.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        raise ValueError("xa and b must be bfloat16")
    r = xa.shape[1]
    if xa.shape[0] != a.rows or b.shape != (w.rows, r):
        raise ValueError("gemm_w4a4_lora: adapter shapes do not match")
    if out is None:
        out = torch.empty((a.rows, w.rows), dtype=out_dtype, device=a.codes.device)
    ca, cw = a.c(), w.c()
    _check(lib().nvfp4_gemm_w4a4_lora(C.byref(ca), C.byref(cw), _dev(xa, "xa"), _dev(b, "b"), r,
                                      float(lora_scale), _dev(out, "out"), _DT[out.dtype],
                                      None if amax_out is None else amax_out.data_ptr(),
                                      _stream(stream)))
    return out


# --------------------------------------------------------------------------
# MXFP4 speed reference (not part of the method)
# --------------------------------------------------------------------------

def mx_quantize(x: torch.Tensor, stream=None):
    """nvfp4_mx_quantize: x [rows, cols] (float32 or bfloat16, cols % 32 == 0)
    -> (codes uint8 [rows, cols/2], scales uint8 [rows, cols/32] E8M0)."""
    if x.dim() != 2 or x.dtype not in _DT:
        raise ValueError("mx_quantize expects a 2-D float32 or bfloat16 tensor")
    x = x.contiguous()
    rows, cols = x.shape
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, max(cols // 32, 0)), dtype=torch.uint8, device=x.device)
    _check(lib().nvfp4_mx_quantize(_dev(x, "x"), _DT[x.dtype], rows, cols, codes.data_ptr(),
                                   scales.data_ptr(), _stream(stream)))
    return codes, scales


def gemm_mx(a, w, out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
            stream=None) -> torch.Tensor:
    """nvfp4_gemm_mx: Y = A_mx W_mx^T for (codes, scales) pairs from mx_quantize."""
    (ac, as_), (wc, ws) = a, w
    M, N, K = ac.shape[0], wc.shape[0], ac.shape[1] * 2
    if wc.shape[1] * 2 != K:
        raise ValueError("gemm_mx: K mismatch")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=ac.device)
    _check(lib().nvfp4_gemm_mx(ac.data_ptr(), as_.data_ptr(), wc.data_ptr(), ws.data_ptr(), M, N,
                               K, _dev(out, "out"), _DT[out.dtype], _stream(stream)))
    return out


# --------------------------------------------------------------------------
# KV ring
# --------------------------------------------------------------------------

@dataclass
class KVConfig:
    tokens_per_frame: int = 880
    frames_per_chunk: int = 8
    heads: int = 24
    head_dim: int = 128
    sink_frames_global: int = 3
    sink_frames_shot: int = 3
    window_chunks: int = 4
    search: int = SEARCH_4O6

    def c(self) -> CKvConfig:
        return CKvConfig(self.tokens_per_frame, self.frames_per_chunk, self.heads, self.head_dim,
                         self.sink_frames_global, self.sink_frames_shot, self.window_chunks,
                         self.search)

    @property
    def chunk_tokens(self) -> int:
        return self.tokens_per_frame * self.frames_per_chunk


def kv_ring_bytes(cfg: KVConfig) -> int:
    c = cfg.c()
    return int(lib().nvfp4_kv_ring_bytes(C.byref(c)))


def kv_store_workspace_bytes(cfg: KVConfig) -> int:
    c = cfg.c()
    return int(lib().nvfp4_kv_store_workspace_bytes(C.byref(c)))


class KVRing:
    """Streaming NVFP4 KV cache: W chunk slots plus global and shot sink copies.

    Device memory comes from torch (uint8 tensors) and is owned by this
    object; the ring state is the C struct nvfp4_kv_ring.
    """

    def __init__(self, cfg: KVConfig, device="cuda"):
        self.cfg = cfg
        c = cfg.c()
        nbytes = int(lib().nvfp4_kv_ring_bytes(C.byref(c)))
        if nbytes == 0:
            _check(lib().nvfp4_kv_ring_init(None, C.byref(c), None, 0))
        self.mem = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.mem.data_ptr()) % 256
        self._base = self.mem.data_ptr() + off
        # zero-filled; every store leaves it so (the first store clears it too)
        self.ws = torch.zeros(kv_store_workspace_bytes(cfg), dtype=torch.uint8, device=device)
        self.ring = CKvRing()
        _check(lib().nvfp4_kv_ring_init(C.byref(self.ring), C.byref(c), C.c_void_p(self._base),
                                        nbytes))

    @property
    def next_chunk(self) -> int:
        return int(self.ring.next_chunk)

    def begin_shot(self, chunk_idx: int):
        _check(lib().nvfp4_kv_begin_shot(C.byref(self.ring), chunk_idx))

    def store_chunk(self, chunk_idx: int, K: torch.Tensor, V: torch.Tensor,
                    v_amax: torch.Tensor | None = None, stream=None):
        """nvfp4_kv_store_chunk; v_amax (optional one-element float32 device
        tensor): max|V| over the chunk from its producer."""
        if K.dtype != torch.bfloat16 or V.dtype != torch.bfloat16:
            raise ValueError("K and V must be bfloat16")
        T, hd = self.cfg.chunk_tokens, self.cfg.heads * self.cfg.head_dim
        if K.numel() != T * hd or V.numel() != T * hd:
            raise ValueError(f"K and V must hold [{T}, {self.cfg.heads}, {self.cfg.head_dim}]")
        _check(lib().nvfp4_kv_store_chunk(C.byref(self.ring), chunk_idx, _dev(K, "K"),
                                          _dev(V, "V"), _amax_arg(v_amax, "v_amax"),
                                          C.c_void_p(self.ws.data_ptr()), self.ws.numel(),
                                          _stream(stream)))

    def store_chunk_noalloc(self, chunk_idx: int, K: torch.Tensor, V: torch.Tensor,
                            v_amax: torch.Tensor | None = None, stream=None):
        """nvfp4_kv_store_chunk_noalloc: as store_chunk, with the library's
        fixed device scratch instead of this ring's workspace."""
        if K.dtype != torch.bfloat16 or V.dtype != torch.bfloat16:
            raise ValueError("K and V must be bfloat16")
        T, hd = self.cfg.chunk_tokens, self.cfg.heads * self.cfg.head_dim
        if K.numel() != T * hd or V.numel() != T * hd:
            raise ValueError(f"K and V must hold [{T}, {self.cfg.heads}, {self.cfg.head_dim}]")
        _check(lib().nvfp4_kv_store_chunk_noalloc(C.byref(self.ring), chunk_idx, _dev(K, "K"),
                                                  _dev(V, "V"), _amax_arg(v_amax, "v_amax"),
                                                  _stream(stream)))

    def effective_tokens(self, step: int) -> int:
        n = C.c_int64()
        _check(lib().nvfp4_kv_effective_tokens(C.byref(self.ring), step, C.byref(n)))
        return int(n.value)

    def gather_window(self, step: int, K_out: torch.Tensor | None = None,
                      V_out: torch.Tensor | None = None, stream=None):
        """Dequantized K_eff(step), V_eff(step): bf16 [n, heads, head_dim]."""
        n = self.effective_tokens(step)
        shape = (n, self.cfg.heads, self.cfg.head_dim)
        dev = self.mem.device
        if K_out is None:
            K_out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        if V_out is None:
            V_out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        cap = min(K_out.shape[0], V_out.shape[0]) if K_out.dim() else 0
        got = C.c_int64()
        _check(lib().nvfp4_gather_window(C.byref(self.ring), step, _dev(K_out, "K_out"),
                                         _dev(V_out, "V_out"), cap, C.byref(got),
                                         _stream(stream)))
        return K_out[:got.value], V_out[:got.value]

    def attention_plan(self, step: int, n_q: int, key_splits: int = 0) -> tuple[int, int]:
        """nvfp4_attention_plan: (key splits, workspace bytes) of attention()
        with these arguments (key_splits 0 = the library's choice)."""
        sp, wsb = C.c_int32(), C.c_size_t()
        _check(lib().nvfp4_attention_plan(C.byref(self.ring), step, n_q, key_splits,
                                          C.byref(sp), C.byref(wsb)))
        return sp.value, wsb.value

    def attention(self, step: int, q: torch.Tensor, softmax_scale: float | None = None,
                  out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                  key_splits: int = 0, workspace: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
        """nvfp4_attention_window: attention of q (bf16 [n_q, heads, 128]) over
        K_eff(step), read packed from the ring.  softmax_scale defaults to
        1/sqrt(head_dim); lse (optional float32 [n_q, heads]) receives the
        log-sum-exp of the scaled scores.  key_splits: 0 = the library's
        choice, else 1..8; the workspace the splits need is allocated here
        unless `workspace` (uint8, on q's device) is given."""
        if q.dtype != torch.bfloat16 or q.dim() != 3 or q.shape[1:] != (self.cfg.heads,
                                                                        self.cfg.head_dim):
            raise ValueError(f"q must be bfloat16 [n_q, {self.cfg.heads}, {self.cfg.head_dim}]")
        if softmax_scale is None:
            softmax_scale = self.cfg.head_dim ** -0.5
        if out is None:
            out = torch.empty_like(q)
        elif out.dtype != torch.bfloat16 or out.shape != q.shape:
            raise ValueError("out must be bfloat16 with q's shape")
        if lse is not None and (lse.dtype != torch.float32 or lse.shape != q.shape[:2]):
            raise ValueError("lse must be float32 [n_q, heads]")
        _, wsb = self.attention_plan(step, q.shape[0], key_splits)
        ws = None
        if wsb > 0:
            if workspace is None:
                workspace = torch.empty(wsb, dtype=torch.uint8, device=q.device)
            elif workspace.dtype != torch.uint8 or workspace.numel() < wsb:
                raise ValueError(f"workspace must be uint8 with at least {wsb} elements")
            ws = _dev(workspace, "workspace")
        _check(lib().nvfp4_attention_window(
            C.byref(self.ring), step, _dev(q, "q"), q.shape[0], float(softmax_scale),
            _dev(out, "out"), None if lse is None else _dev(lse, "lse"), key_splits, ws,
            workspace.numel() if wsb > 0 else 0, _stream(stream)))
        return out


# --------------------------------------------------------------------------
# Kernel timing
# --------------------------------------------------------------------------

def profile_enable(on: bool = True):
    """nvfp4_profile_enable: bracket every library kernel launch with HIP events."""
    _check(lib().nvfp4_profile_enable(1 if on else 0))


def profile_collect(cap: int = 64) -> dict:
    """nvfp4_profile_collect: {kernel name: (launches, total ms)}; clears the record."""
    name_len = 64
    names = C.create_string_buffer(cap * name_len)
    launches = (C.c_int64 * cap)()
    total = (C.c_double * cap)()
    n = lib().nvfp4_profile_collect(names, name_len, launches, total, cap)
    if n < 0:
        _check(n)
    out = {}
    for i in range(min(n, cap)):
        nm = names.raw[i * name_len:(i + 1) * name_len].split(b"\0", 1)[0].decode()
        out[nm] = (int(launches[i]), float(total[i]))
    return out
