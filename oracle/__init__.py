"""CPU oracle for blockwise quantization of ZeRO-3 communication payloads.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path (the
HIP library and its binding) never imports it, and this package imports nothing
from the product.

Thin numpy wrappers over ``liboracle.so`` (plain single-threaded C, see
``qcp_oracle.c`` for the method, its sources and the readings taken).  Arrays
are numpy; bfloat16 data is carried as ``np.uint16`` bit patterns and named by
the dtype tag ``"bf16"``.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# this package's own numbering of element types and payload formats
DTYPES = {"f16": 1, "bf16": 2, "f32": 3}
FORMATS = {"int2": 2, "int4": 4, "int6": 6, "int8": 8, "e4m3": 0x43}
_NP = {"f16": np.float16, "bf16": np.uint16, "f32": np.float32}

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


class loaded_from:
    """Context manager: route every oracle call to another build of the oracle
    (used by the test that plants mistakes in copies of it)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.prev = _load()
        _lib = _bind(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.prev
        return False


def _bind(lib):
    p, i64, i32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    lib.oracle_payload_bytes.restype = i64
    lib.oracle_payload_bytes.argtypes = [i64, i32, i32]
    lib.oracle_quantize_blockwise.argtypes = [p, ci, i64, i32, ci, p, p]
    lib.oracle_pack_subbyte.argtypes = [p, ci, i64, i32, i32, p, p]
    lib.oracle_dequantize_blockwise.argtypes = [p, p, ci, i64, i32, p, ci]
    lib.oracle_unpack_subbyte.argtypes = [p, p, i64, i32, i32, p, ci]
    lib.oracle_dequant_reduce_requant.argtypes = [p, i64, p, i64, i32, i64, i32,
                                                  ci, ci, p, p, p]
    lib.oracle_fp8_accum_requant.argtypes = [p, p, p, ci, i64, i32]
    lib.oracle_reorder_slices.argtypes = [p, ci, i64, i32, i32, p]
    lib.oracle_aquavit_target.argtypes = [i64, i64, ctypes.c_double, ctypes.c_double]
    lib.oracle_aquavit_target.restype = ctypes.c_double
    lib.oracle_aquavit_level.argtypes = [i64, i64, ctypes.c_double, ctypes.c_double,
                                         ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.oracle_pack_records.argtypes = [p, ci, i64, i32, i32, p]
    lib.oracle_unpack_records.argtypes = [p, i64, i32, i32, p, ci]
    lib.oracle_reorder_quantize.argtypes = [p, ci, i64, i32, i32, i32, ci, p, i64, p, i64]
    for name in ("oracle_f32_to_f16", "oracle_f32_to_bf16", "oracle_f16_to_f32",
                 "oracle_f32_to_e4m3", "oracle_e4m3_to_f32"):
        getattr(lib, name).argtypes = [p, i64, p]
        getattr(lib, name).restype = None
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def fmt_bits(fmt: str) -> int:
    return 8 if fmt == "e4m3" else FORMATS[fmt]


def code_bytes(n: int, fmt: str) -> int:
    return (n * fmt_bits(fmt) + 7) // 8


def n_blocks(n: int, G: int) -> int:
    return (n + G - 1) // G


def payload_bytes(n: int, bits: int, G: int) -> int:
    """ceil(n*b/8) code bytes + 4 bytes of scale per block."""
    return int(_load().oracle_payload_bytes(n, bits, G))


def _as_input(x, dt):
    x = np.ascontiguousarray(x)
    if x.dtype != _NP[dt]:
        raise TypeError(f"expected {np.dtype(_NP[dt])} data for dtype tag {dt!r}, got {x.dtype}")
    return x


def quantize_blockwise(x, dt: str, G: int, fmt: str):
    """Blockwise quantize -> (codes uint8[ceil(n*b/8)], scales float32[ceil(n/G)])."""
    x = _as_input(x, dt)
    n = x.size
    codes = np.zeros(code_bytes(n, fmt), np.uint8)
    scales = np.zeros(n_blocks(n, G), np.float32)
    _check(_load().oracle_quantize_blockwise(_ptr(x), DTYPES[dt], n, G, FORMATS[fmt],
                                             _ptr(codes), _ptr(scales)), "quantize_blockwise")
    return codes, scales


def pack_subbyte(x, dt: str, b: int, G: int):
    x = _as_input(x, dt)
    n = x.size
    packed = np.zeros((n * b + 7) // 8, np.uint8)
    scales = np.zeros(n_blocks(n, G), np.float32)
    _check(_load().oracle_pack_subbyte(_ptr(x), DTYPES[dt], n, b, G, _ptr(packed),
                                       _ptr(scales)), "pack_subbyte")
    return packed, scales


def dequantize_blockwise(codes, scales, fmt: str, n: int, G: int, yt: str):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.float32)
    assert codes.size >= code_bytes(n, fmt) and scales.size >= n_blocks(n, G)
    y = np.zeros(n, _NP[yt])
    _check(_load().oracle_dequantize_blockwise(_ptr(codes), _ptr(scales), FORMATS[fmt], n, G,
                                               _ptr(y), DTYPES[yt]), "dequantize_blockwise")
    return y


def unpack_subbyte(packed, scales, n: int, b: int, G: int, yt: str):
    packed = np.ascontiguousarray(packed, np.uint8)
    scales = np.ascontiguousarray(scales, np.float32)
    assert packed.size >= (n * b + 7) // 8 and scales.size >= n_blocks(n, G)
    y = np.zeros(n, _NP[yt])
    _check(_load().oracle_unpack_subbyte(_ptr(packed), _ptr(scales), n, b, G, _ptr(y),
                                         DTYPES[yt]), "unpack_subbyte")
    return y


def dequant_reduce_requant(codes_in, slice_stride: int, scales_in, scale_stride: int,
                           n_slices: int, slice_len: int, G: int, fmt_in: str,
                           fmt_out: str, want_sum: bool = False):
    """N-slice dequantize -> fp32 fmaf-chain sum -> blockwise requantize.

    ``codes_in`` is one uint8 buffer holding slice j at byte offset
    j*slice_stride; ``scales_in`` holds slice j's scales at j*scale_stride.
    Returns (codes_out, scales_out[, sum_out])."""
    codes_in = np.ascontiguousarray(codes_in, np.uint8)
    scales_in = np.ascontiguousarray(scales_in, np.float32)
    assert codes_in.size >= (n_slices - 1) * slice_stride + code_bytes(slice_len, fmt_in)
    assert scales_in.size >= (n_slices - 1) * scale_stride + n_blocks(slice_len, G)
    codes_out = np.zeros(code_bytes(slice_len, fmt_out), np.uint8)
    scales_out = np.zeros(n_blocks(slice_len, G), np.float32)
    sums = np.zeros(slice_len, np.float32) if want_sum else None
    _check(_load().oracle_dequant_reduce_requant(
        _ptr(codes_in), slice_stride, _ptr(scales_in), scale_stride, n_slices, slice_len, G,
        FORMATS[fmt_in], FORMATS[fmt_out], _ptr(codes_out), _ptr(scales_out),
        _ptr(sums) if want_sum else None), "dequant_reduce_requant")
    return (codes_out, scales_out, sums) if want_sum else (codes_out, scales_out)


def fp8_accum_requant(state_codes, state_scales, grad, gt: str, G: int):
    """One micro-batch of FP8 main-gradient accumulation; returns the new state
    (copies; the inputs are not modified)."""
    codes = np.array(state_codes, np.uint8, copy=True)
    scales = np.array(state_scales, np.float32, copy=True)
    g = _as_input(grad, gt)
    n = g.size
    assert codes.size >= n and scales.size >= n_blocks(n, G)
    _check(_load().oracle_fp8_accum_requant(_ptr(codes), _ptr(scales), _ptr(g), DTYPES[gt],
                                            n, G), "fp8_accum_requant")
    return codes, scales


def reorder_slices(x, dt: str, n_nodes: int, gpus_per_node: int):
    """qgZ tensor-slice reordering of one rank's bucket: slice j (of N) holds
    the chunks b*N + j, b = 0..K-1.  Returns the reordered copy."""
    x = _as_input(x, dt)
    y = np.zeros_like(x)
    _check(_load().oracle_reorder_slices(_ptr(x), DTYPES[dt], x.size, n_nodes, gpus_per_node,
                                         _ptr(y)), "reorder_slices")
    return y


def slice_layout(slice_len: int, G: int, fmt: str):
    """(code stride in bytes, scale stride in floats) of an N-slice buffer:
    each slice's payload rounded up to 16 bytes / 4 floats."""
    return (code_bytes(slice_len, fmt) + 15) // 16 * 16, (n_blocks(slice_len, G) + 3) // 4 * 4


def reorder_quantize(x, dt: str, n_nodes: int, gpus_per_node: int, G: int, fmt: str):
    """qgZ sender: reorder, then quantize every slice.  Returns (codes, code
    stride, scales, scale stride) in the N-slice layout of ``slice_layout``."""
    x = _as_input(x, dt)
    N = gpus_per_node
    L = x.size // N
    cs, ss = slice_layout(L, G, fmt)
    codes = np.zeros(cs * N, np.uint8)
    scales = np.zeros(ss * N, np.float32)
    _check(_load().oracle_reorder_quantize(_ptr(x), DTYPES[dt], x.size, n_nodes, N, G,
                                           FORMATS[fmt], _ptr(codes), cs, _ptr(scales), ss),
           "reorder_quantize")
    return codes, cs, scales, ss


def aquavit_target(t: int, T: int, a: float = 0.9, c: float = 5.0) -> float:
    """Aquavit's target effective bits per weight at step t of T."""
    return float(_load().oracle_aquavit_target(t, T, a, c))


def aquavit_level(t: int, T: int, a: float = 0.9, c: float = 5.0):
    """(b, G) granularity-modulation level used at step t of T."""
    b, G = ctypes.c_int32(), ctypes.c_int32()
    _check(_load().oracle_aquavit_level(t, T, a, c, ctypes.byref(b), ctypes.byref(G)),
           "aquavit_level")
    return b.value, G.value


def pack_records(x, dt: str, b: int, G: int):
    """Metadata-interleaved payload: per block [fp32 scale][codes]."""
    x = _as_input(x, dt)
    n = x.size
    rec = np.zeros(payload_bytes(n, b, G), np.uint8)
    _check(_load().oracle_pack_records(_ptr(x), DTYPES[dt], n, b, G, _ptr(rec)), "pack_records")
    return rec


def unpack_records(records, n: int, b: int, G: int, yt: str):
    records = np.ascontiguousarray(records, np.uint8)
    assert records.size >= payload_bytes(n, b, G)
    y = np.zeros(n, _NP[yt])
    _check(_load().oracle_unpack_records(_ptr(records), n, b, G, _ptr(y), DTYPES[yt]),
           "unpack_records")
    return y


# --- the oracle's own format converters, exposed so tests can pin them ---

def _conv(name, x, in_dtype, out_dtype):
    x = np.ascontiguousarray(x, in_dtype)
    y = np.zeros(x.size, out_dtype)
    getattr(_load(), name)(_ptr(x), x.size, _ptr(y))
    return y


def f32_to_f16_bits(x):
    return _conv("oracle_f32_to_f16", x, np.float32, np.uint16)


def f32_to_bf16_bits(x):
    return _conv("oracle_f32_to_bf16", x, np.float32, np.uint16)


def f16_bits_to_f32(x):
    return _conv("oracle_f16_to_f32", x, np.uint16, np.float32)


def f32_to_e4m3(x):
    return _conv("oracle_f32_to_e4m3", x, np.float32, np.uint8)


def e4m3_to_f32(x):
    return _conv("oracle_e4m3_to_f32", x, np.uint8, np.float32)


def bf16_bits_to_f32(x):
    """bfloat16 bits -> float32 (exact: the upper half of a binary32)."""
    return (np.ascontiguousarray(x, np.uint16).astype(np.uint32) << 16).view(np.float32)
