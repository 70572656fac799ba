"""quantized_collective_payloads_amd -- blockwise quantization of ZeRO-3
communication payloads on MI355X (gfx950).

A thin ctypes binding over libqcp.so, whose C-ABI is include/qcp.h.  This
module only marshals arguments: it allocates outputs with torch (device memory)
and passes raw device pointers plus the current HIP stream; every step of the
computation runs in the library's HIP kernels.  If libqcp.so is missing the
calls raise -- there is no CPU fallback.

Functions (same names as the C entry points):
    quantize_blockwise(x, G, fmt)                      -> (codes, scales)
    dequantize_blockwise(codes, scales, fmt, n, G, dtype) -> y
    pack_subbyte(x, b, G)                              -> (packed, scales)
    unpack_subbyte(packed, scales, n, b, G, dtype)     -> y
    dequant_reduce_requant(codes_in, slice_stride, scales_in, scale_stride,
                           n_slices, slice_len, G, fmt_in, fmt_out, ...)
                                                       -> (codes, scales[, sums])
    fp8_accum_requant(state_codes, state_scales, grad, G)   (in place)
    payload_bytes(n, bits, G)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["quantize_blockwise", "dequantize_blockwise", "pack_subbyte", "unpack_subbyte",
           "dequant_reduce_requant", "fp8_accum_requant", "payload_bytes", "code_bytes",
           "n_blocks", "QcpError", "library", "FORMATS", "DTYPES", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqcp.so")

# numbering of include/qcp.h
DTYPES = {torch.float16: 1, torch.bfloat16: 2, torch.float32: 3}
FORMATS = {"int2": 2, "int4": 4, "int6": 6, "int8": 8, "e4m3": 0x43}
_STATUS = {0: "QCP_OK", -1: "QCP_EINVAL", -2: "QCP_EALIGN", -3: "QCP_EUNSUPPORTED", -4: "QCP_EHIP"}

_lib = None


class QcpError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)} ({detail})")
        self.status = status


def library():
    """The loaded libqcp.so (ctypes).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m quantized_collective_payloads_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        p, i64, i32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
        sig = {
            "quantize_blockwise": [p, ci, i64, i32, ci, p, p, p],
            "dequantize_blockwise": [p, p, ci, i64, i32, p, ci, p],
            "pack_subbyte": [p, ci, i64, i32, i32, p, p, p],
            "unpack_subbyte": [p, p, i64, i32, i32, p, ci, p],
            "dequant_reduce_requant": [p, i64, p, i64, i32, i64, i32, ci, ci, p, p, p, p],
            "fp8_accum_requant": [p, p, p, ci, i64, i32, p],
            "reorder_quantize": [p, ci, i64, i32, i32, i32, ci, p, i64, p, i64, p],
            "pack_subbyte_records": [p, ci, i64, i32, i32, p, p],
            "unpack_subbyte_records": [p, i64, i32, i32, p, ci, p],
            "qcp_aquavit_level": [i64, i64, ctypes.c_double, ctypes.c_double,
                                  ctypes.POINTER(i32), ctypes.POINTER(i32)],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ci
        lib.qcp_aquavit_target.argtypes = [i64, i64, ctypes.c_double, ctypes.c_double]
        lib.qcp_aquavit_target.restype = ctypes.c_double
        lib.qcp_payload_bytes.argtypes = [i64, i32, i32]
        lib.qcp_payload_bytes.restype = i64
        lib.qcp_strerror.argtypes = [ci]
        lib.qcp_strerror.restype = ctypes.c_char_p
        lib.qcp_version.argtypes = []
        lib.qcp_version.restype = ctypes.c_char_p
        lib.qcp_max_elements.argtypes = []
        lib.qcp_max_elements.restype = i64
        _lib = lib
    return _lib


def _check(fn: str, rc: int):
    if rc != 0:
        raise QcpError(fn, rc, library().qcp_strerror(rc).decode())


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _bits(fmt) -> int:
    f = _fmt(fmt)
    return 8 if f == FORMATS["e4m3"] else f


def code_bytes(n: int, fmt) -> int:
    return (n * _bits(fmt) + 7) // 8


def n_blocks(n: int, G: int) -> int:
    return (n + G - 1) // G


def payload_bytes(n: int, bits: int, G: int) -> int:
    """ceil(n*bits/8) code bytes + one fp32 scale per block of G."""
    return int(library().qcp_payload_bytes(n, bits, G))


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("qcp operates on GPU tensors only")
    dev = ts[0].device
    for t in ts:
        if t is not None and t.device != dev:
            raise ValueError(f"qcp: tensors on different devices ({t.device} and {dev})")
    return dev


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _dtype_code(dt) -> int:
    if dt not in DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    return DTYPES[dt]


def _need(t, what: str, dtypes, numel: int):
    """A buffer the library reads or writes through a raw pointer: it must be a
    contiguous tensor of one of `dtypes` holding at least `numel` elements (the
    C-ABI cannot check lengths).  Raises ValueError otherwise."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{what}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise ValueError(f"{what}: dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{what}: holds {t.numel()} elements, needs at least {numel}")
    return t


_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_ELEMS = tuple(DTYPES)


def _check_n_G(n: int, G: int):
    if n < 0:
        raise ValueError(f"element count {n} is negative")
    if G < 32 or G > 1024 or G & (G - 1):
        raise ValueError(f"block size {G} is not a power of two in [32, 1024]")


def quantize_blockwise(x: torch.Tensor, G: int, fmt="int8", codes=None, scales=None):
    """Blockwise quantize an fp16/bf16/fp32 GPU tensor (flattened; a non-contiguous
    input is copied first).  Caller-supplied `codes` (uint8) and `scales`
    (float32) must be contiguous and large enough."""
    _need(x, "x", _ELEMS, 0)
    x = x.contiguous().view(-1)
    n = x.numel()
    _check_n_G(n, G)
    if codes is not None:
        _need(codes, "codes", _U8, code_bytes(n, fmt))
    if scales is not None:
        _need(scales, "scales", _F32, n_blocks(n, G))
    dev = _dev(x, codes, scales)
    if codes is None:
        codes = torch.empty(code_bytes(n, fmt), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(n_blocks(n, G), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check("quantize_blockwise", library().quantize_blockwise(
            _ptr(x), _dtype_code(x.dtype), n, G, _fmt(fmt), _ptr(codes), _ptr(scales), _stream(dev)))
    return codes, scales


def dequantize_blockwise(codes: torch.Tensor, scales: torch.Tensor, fmt, n: int, G: int,
                         dtype=torch.bfloat16, out=None):
    _check_n_G(n, G)
    _need(codes, "codes", _U8, code_bytes(n, fmt))
    _need(scales, "scales", _F32, n_blocks(n, G))
    if out is not None:
        _need(out, "out", _ELEMS, n)
    dev = _dev(codes, scales, out)
    if out is None:
        out = torch.empty(n, dtype=dtype, device=dev)
    with torch.cuda.device(dev):
        _check("dequantize_blockwise", library().dequantize_blockwise(
            _ptr(codes), _ptr(scales), _fmt(fmt), n, G, _ptr(out), _dtype_code(out.dtype),
            _stream(dev)))
    return out


def pack_subbyte(x: torch.Tensor, b: int, G: int, packed=None, scales=None):
    _need(x, "x", _ELEMS, 0)
    x = x.contiguous().view(-1)
    n = x.numel()
    _check_n_G(n, G)
    if packed is not None:
        _need(packed, "packed", _U8, (n * b + 7) // 8)
    if scales is not None:
        _need(scales, "scales", _F32, n_blocks(n, G))
    dev = _dev(x, packed, scales)
    if packed is None:
        packed = torch.empty((n * b + 7) // 8, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(n_blocks(n, G), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check("pack_subbyte", library().pack_subbyte(
            _ptr(x), _dtype_code(x.dtype), n, b, G, _ptr(packed), _ptr(scales), _stream(dev)))
    return packed, scales


def unpack_subbyte(packed: torch.Tensor, scales: torch.Tensor, n: int, b: int, G: int,
                   dtype=torch.bfloat16, out=None):
    _check_n_G(n, G)
    _need(packed, "packed", _U8, (n * b + 7) // 8)
    _need(scales, "scales", _F32, n_blocks(n, G))
    if out is not None:
        _need(out, "out", _ELEMS, n)
    dev = _dev(packed, scales, out)
    if out is None:
        out = torch.empty(n, dtype=dtype, device=dev)
    with torch.cuda.device(dev):
        _check("unpack_subbyte", library().unpack_subbyte(
            _ptr(packed), _ptr(scales), n, b, G, _ptr(out), _dtype_code(out.dtype), _stream(dev)))
    return out


def dequant_reduce_requant(codes_in: torch.Tensor, slice_stride: int, scales_in: torch.Tensor,
                           scale_stride: int, n_slices: int, slice_len: int, G: int,
                           fmt_in="int4", fmt_out="int4", want_sum: bool = False,
                           codes_out=None, scales_out=None, sum_out=None):
    """Reduce the n_slices received slices held in one buffer: slice j's codes at
    byte offset j*slice_stride of codes_in, its scales at float offset
    j*scale_stride of scales_in."""
    _check_n_G(slice_len, G)
    if n_slices < 1:
        raise ValueError(f"n_slices {n_slices} < 1")
    nb = n_blocks(slice_len, G)
    if slice_len > 0:
        _need(codes_in, "codes_in", _U8, (n_slices - 1) * slice_stride + code_bytes(slice_len, fmt_in))
        _need(scales_in, "scales_in", _F32, (n_slices - 1) * scale_stride + nb)
    if codes_out is not None:
        _need(codes_out, "codes_out", _U8, code_bytes(slice_len, fmt_out))
    if scales_out is not None:
        _need(scales_out, "scales_out", _F32, nb)
    if sum_out is not None:
        _need(sum_out, "sum_out", _F32, slice_len)
    dev = _dev(codes_in, scales_in, codes_out, scales_out, sum_out)
    if codes_out is None:
        codes_out = torch.empty(code_bytes(slice_len, fmt_out), dtype=torch.uint8, device=dev)
    if scales_out is None:
        scales_out = torch.empty(nb, dtype=torch.float32, device=dev)
    if want_sum and sum_out is None:
        sum_out = torch.empty(slice_len, dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check("dequant_reduce_requant", library().dequant_reduce_requant(
            _ptr(codes_in), slice_stride, _ptr(scales_in), scale_stride, n_slices, slice_len, G,
            _fmt(fmt_in), _fmt(fmt_out), _ptr(codes_out), _ptr(scales_out), _ptr(sum_out),
            _stream(dev)))
    return (codes_out, scales_out, sum_out) if sum_out is not None else (codes_out, scales_out)


def pack_subbyte_records(x: torch.Tensor, b: int, G: int, records=None):
    """Aquavit payload with interleaved metadata: per block [fp32 scale][codes]."""
    _need(x, "x", _ELEMS, 0)
    x = x.contiguous().view(-1)
    n = x.numel()
    _check_n_G(n, G)
    if records is not None:
        _need(records, "records", _U8, payload_bytes(n, b, G))
    dev = _dev(x, records)
    if records is None:
        records = torch.empty(payload_bytes(n, b, G), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        _check("pack_subbyte_records", library().pack_subbyte_records(
            _ptr(x), _dtype_code(x.dtype), n, b, G, _ptr(records), _stream(dev)))
    return records


def unpack_subbyte_records(records: torch.Tensor, n: int, b: int, G: int,
                           dtype=torch.bfloat16, out=None):
    _check_n_G(n, G)
    _need(records, "records", _U8, payload_bytes(n, b, G))
    if out is not None:
        _need(out, "out", _ELEMS, n)
    dev = _dev(records, out)
    if out is None:
        out = torch.empty(n, dtype=dtype, device=dev)
    with torch.cuda.device(dev):
        _check("unpack_subbyte_records", library().unpack_subbyte_records(
            _ptr(records), n, b, G, _ptr(out), _dtype_code(out.dtype), _stream(dev)))
    return out


def aquavit_target(t: int, T: int, a: float = 0.9, c: float = 5.0) -> float:
    """Target bits per weight of the ascending schedule at step t of T."""
    return float(library().qcp_aquavit_target(t, T, a, c))


def aquavit_level(t: int, T: int, a: float = 0.9, c: float = 5.0):
    """(b, G) granularity-modulation level for step t of T (host only)."""
    b, G = ctypes.c_int32(), ctypes.c_int32()
    _check("qcp_aquavit_level", library().qcp_aquavit_level(t, T, a, c, ctypes.byref(b),
                                                            ctypes.byref(G)))
    return b.value, G.value


def slice_layout(slice_len: int, G: int, fmt):
    """(code stride in bytes, scale stride in floats) of an N-slice buffer: each
    slice's codes rounded up to 256 bytes, so every slice starts on a cache-line
    boundary (a stride that is not a multiple of the 128-byte line makes each
    wave's 1 KB segment of a slice touch a ninth line), and its scales to 4 floats."""
    return (code_bytes(slice_len, fmt) + 255) // 256 * 256, (n_blocks(slice_len, G) + 3) // 4 * 4


def reorder_quantize(x: torch.Tensor, n_nodes: int, gpus_per_node: int, G: int, fmt="int4",
                     codes=None, slice_stride=None, scales=None, scale_stride=None):
    """qgZ sender: tensor-slice reordering of one rank's bucket fused with the
    quantization of its gpus_per_node send slices.  Returns (codes, slice_stride,
    scales, scale_stride): slice j's codes at byte offset j*slice_stride."""
    _need(x, "x", _ELEMS, 0)
    x = x.contiguous().view(-1)
    n = x.numel()
    _check_n_G(n, G)
    if gpus_per_node < 1:
        raise ValueError(f"gpus_per_node {gpus_per_node} < 1")
    L = n // gpus_per_node
    cs, ss = slice_layout(L, G, fmt)
    slice_stride = cs if slice_stride is None else slice_stride
    scale_stride = ss if scale_stride is None else scale_stride
    if codes is not None:
        _need(codes, "codes", _U8, (gpus_per_node - 1) * slice_stride + code_bytes(L, fmt))
    if scales is not None:
        _need(scales, "scales", _F32, (gpus_per_node - 1) * scale_stride + n_blocks(L, G))
    dev = _dev(x, codes, scales)
    if codes is None:
        codes = torch.empty(slice_stride * gpus_per_node, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(scale_stride * gpus_per_node, dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check("reorder_quantize", library().reorder_quantize(
            _ptr(x), _dtype_code(x.dtype), n, n_nodes, gpus_per_node, G, _fmt(fmt), _ptr(codes),
            slice_stride, _ptr(scales), scale_stride, _stream(dev)))
    return codes, slice_stride, scales, scale_stride


def fp8_accum_requant(state_codes: torch.Tensor, state_scales: torch.Tensor, grad: torch.Tensor,
                      G: int):
    """In place: state <- E4M3(bf16(bf16(dequant(state)) + grad))."""
    _need(grad, "grad", _ELEMS, 0)
    g = grad.contiguous().view(-1)
    n = g.numel()
    _check_n_G(n, G)
    _need(state_codes, "state_codes", _U8, n)
    _need(state_scales, "state_scales", _F32, n_blocks(n, G))
    dev = _dev(state_codes, state_scales, g)
    with torch.cuda.device(dev):
        _check("fp8_accum_requant", library().fp8_accum_requant(
            _ptr(state_codes), _ptr(state_scales), _ptr(g), _dtype_code(g.dtype), n, G,
            _stream(dev)))
    return state_codes, state_scales
