"""The C-ABI library loads, exports every symbol include/qcp.h declares, and its
host-side validation rejects bad arguments before any HIP call (CPU only: no
kernel is launched by these tests)."""
import ctypes
import os
import re

import pytest

import quantized_collective_payloads_amd as qcp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qcp.h")

OK, EINVAL, EALIGN, EUNSUP, EHIP = 0, -1, -2, -3, -4
F16, BF16, F32 = 1, 2, 3
INT2, INT4, INT6, INT8, E4M3 = 2, 4, 6, 8, 0x43

# fake, never-dereferenced device addresses (validation only looks at the values)
A = 0x7f0000000000
P = ctypes.c_void_p


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qcp.LIB_PATH):
        pytest.fail(f"{qcp.LIB_PATH} not built (run python -m quantized_collective_payloads_amd.build)")
    return qcp.library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"quantize_blockwise", "dequantize_blockwise", "pack_subbyte",
                          "unpack_subbyte", "dequant_reduce_requant", "fp8_accum_requant",
                          "qcp_payload_bytes", "qcp_strerror", "qcp_version"}
    for name in names:
        assert hasattr(lib, name), f"libqcp.so does not export {name}"


def test_payload_bytes_and_strings(lib):
    assert qcp.payload_bytes(1 << 20, 2, 1024) * 8 / (1 << 20) == 2 + 32 / 1024
    assert qcp.payload_bytes(1 << 20, 6, 32) * 8 / (1 << 20) == 7.0
    assert qcp.payload_bytes(0, 4, 512) == 0
    assert qcp.payload_bytes(1, 4, 512) == 1 + 4
    assert qcp.payload_bytes(-1, 4, 512) == -1
    for st in (OK, EINVAL, EALIGN, EUNSUP, EHIP, 12345):
        assert isinstance(lib.qcp_strerror(st), bytes)
    assert lib.qcp_version() == b"0.1.0"


def q(lib, x=A, xt=BF16, n=1024, G=256, fmt=INT8, codes=A + (1 << 30), scales=A + (2 << 30)):
    return lib.quantize_blockwise(P(x), xt, n, G, fmt, P(codes), P(scales), None)


def test_quantize_validation(lib):
    assert q(lib, n=0) == OK                       # no-op, no launch
    assert q(lib, n=0, x=0, codes=0, scales=0) == OK
    assert q(lib, n=-1) == EINVAL
    assert q(lib, n=(1 << 40) + 1) == EINVAL
    for G in (0, 16, 48, 2048, 100):
        assert q(lib, G=G) == EINVAL, G
    assert q(lib, fmt=3) == EINVAL
    assert q(lib, fmt=16) == EINVAL
    assert q(lib, xt=7) == EINVAL
    assert q(lib, x=0) == EINVAL
    assert q(lib, codes=0) == EINVAL
    assert q(lib, scales=0) == EINVAL
    assert q(lib, x=A + 8) == EALIGN
    assert q(lib, codes=A + (1 << 30) + 4) == EALIGN
    assert q(lib, scales=A + (2 << 30) + 2) == EALIGN
    # outputs overlapping the input
    assert q(lib, codes=A + 1024) == EINVAL
    assert q(lib, scales=A + 16, codes=A + (1 << 30)) == EINVAL
    assert q(lib, codes=A + (1 << 30), scales=A + (1 << 30) + 512) == EINVAL


def test_pack_and_dequant_validation(lib):
    for b in (0, 1, 3, 5, 7, 9, 16):
        assert lib.pack_subbyte(P(A), BF16, 1024, b, 256, P(A + (1 << 30)), P(A + (2 << 30)), None) == EINVAL
        assert lib.unpack_subbyte(P(A), P(A + (1 << 30)), 1024, b, 256, P(A + (2 << 30)), BF16, None) == EINVAL
    d = lib.dequantize_blockwise
    assert d(P(A), P(A + (1 << 30)), INT8, 0, 256, P(A + (2 << 30)), BF16, None) == OK
    assert d(P(A), P(A + (1 << 30)), INT8, 1024, 256, P(0), BF16, None) == EINVAL
    assert d(P(A), P(A + (1 << 30)), INT8, 1024, 256, P(A + (2 << 30)), 9, None) == EINVAL
    assert d(P(A), P(A + (1 << 30)), INT8, 1024, 256, P(A + (2 << 30) + 8), BF16, None) == EALIGN
    assert d(P(A), P(A + (1 << 30)), INT8, 1024, 256, P(A + 256), BF16, None) == EINVAL   # y over codes


def test_reduce_validation(lib):
    r = lib.dequant_reduce_requant
    L, G = 4096, 512
    cb = L // 2                                    # INT4 code bytes per slice
    args = dict(ci=A, ss=cb, si=A + (1 << 30), sst=8, N=8, L=L, G=G, fi=INT4, fo=INT4,
                co=A + (2 << 30), so=A + (3 << 30), su=0)

    def call(**kw):
        a = {**args, **kw}
        return r(P(a["ci"]), a["ss"], P(a["si"]), a["sst"], a["N"], a["L"], a["G"], a["fi"],
                 a["fo"], P(a["co"]), P(a["so"]), P(a["su"]), None)
    assert call(L=0) == OK
    assert call(N=0) == EINVAL
    assert call(N=65) == EINVAL
    assert call(ss=cb - 16) == EINVAL             # stride shorter than a slice
    assert call(ss=cb + 8) == EALIGN              # stride not a multiple of 16
    assert call(sst=7) == EINVAL                  # scale stride shorter than the block count
    assert call(sst=10) == EALIGN
    assert call(fi=5) == EINVAL
    assert call(fo=0) == EINVAL
    assert call(G=100) == EINVAL
    assert call(co=0) == EINVAL
    assert call(su=A + (4 << 30) + 4) == EALIGN
    assert call(co=A + 4 * cb) == EINVAL          # output inside slice 4
    assert call(so=A + (1 << 30) + 64) == EINVAL  # output scales inside input scales
    assert call(su=A + (2 << 30)) == EINVAL       # sums over the output codes


def test_reorder_quantize_validation(lib):
    f = lib.reorder_quantize
    K, N, G = 2, 4, 256
    n = K * N * 512                                # chunks of 512 elements
    L = n // N
    args = dict(x=A, xt=BF16, n=n, K=K, N=N, G=G, fmt=INT4, co=A + (1 << 30), cs=L // 2,
                so=A + (2 << 30), ss=L // G)

    def call(**kw):
        a = {**args, **kw}
        return f(P(a["x"]), a["xt"], a["n"], a["K"], a["N"], a["G"], a["fmt"], P(a["co"]),
                 a["cs"], P(a["so"]), a["ss"], None)
    assert call(n=0) == OK
    assert call(K=0) == EINVAL
    assert call(N=0) == EINVAL
    assert call(N=65) == EINVAL
    assert call(n=n + 8) == EINVAL                 # not K*N equal chunks
    assert call(n=K * N * 12) == EINVAL            # chunk of 12: not a multiple of 8
    assert call(cs=L // 2 - 16) == EINVAL          # slice stride shorter than a slice
    assert call(cs=L // 2 + 8) == EALIGN
    assert call(ss=L // G - 1) == EINVAL
    assert call(ss=L // G + 2) == EALIGN
    assert call(x=A + 8) == EALIGN
    assert call(fmt=5) == EINVAL
    assert call(co=0) == EINVAL
    assert call(co=A + 512) == EINVAL              # codes over the input
    assert call(so=A + (1 << 30) + 256) == EINVAL  # scales over slice 0's codes


def test_accum_validation(lib):
    f = lib.fp8_accum_requant
    n, G = 4096, 128
    assert f(P(A), P(A + (1 << 30)), P(A + (2 << 30)), BF16, 0, G, None) == OK
    assert f(P(A), P(A + (1 << 30)), P(A + (2 << 30)), 4, n, G, None) == EINVAL
    assert f(P(0), P(A + (1 << 30)), P(A + (2 << 30)), BF16, n, G, None) == EINVAL
    assert f(P(A), P(A + (1 << 30)), P(A + (2 << 30)), BF16, n, 96, None) == EINVAL
    assert f(P(A + 1), P(A + (1 << 30)), P(A + (2 << 30)), BF16, n, G, None) == EALIGN
    assert f(P(A), P(A + 1024), P(A + (2 << 30)), BF16, n, G, None) == EINVAL   # scales over codes
    assert f(P(A), P(A + (1 << 30)), P(A + 2048), BF16, n, G, None) == EINVAL   # grad over codes


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        qcp.quantize_blockwise(torch.zeros(1024, dtype=torch.bfloat16), 256, "int8")


def test_aquavit_schedule_matches_oracle():
    import oracle
    for a, c, T in [(0.9, 5.0, 1000), (0.9, 5.0, 37), (0.5, 3.0, 200), (1.2, 8.0, 64)]:
        for t in range(T + 1):
            assert qcp.aquavit_level(t, T, a, c) == oracle.aquavit_level(t, T, a, c), (a, c, T, t)
            assert qcp.aquavit_target(t, T, a, c) == oracle.aquavit_target(t, T, a, c)
    with pytest.raises(qcp.QcpError):
        qcp.aquavit_level(5, 4)


def test_records_validation(lib):
    pr, ur = lib.pack_subbyte_records, lib.unpack_subbyte_records
    assert pr(P(A), BF16, 0, 6, 32, P(A + (1 << 30)), None) == OK
    assert pr(P(A), BF16, 1024, 5, 32, P(A + (1 << 30)), None) == EINVAL
    assert pr(P(A), BF16, 1024, 6, 48, P(A + (1 << 30)), None) == EINVAL
    assert pr(P(A), BF16, 1024, 6, 32, P(A + (1 << 30) + 4), None) == EALIGN
    assert pr(P(A), BF16, 1024, 6, 32, P(A + 1024), None) == EINVAL      # records over x
    assert ur(P(A), 1024, 6, 32, P(A + (1 << 30)), 9, None) == EINVAL
    assert ur(P(A), 1024, 6, 32, P(A + 512), BF16, None) == EINVAL       # y over records
