"""Parity where an INT code hinges on the last bit of the quotient x/s.

The kernels form INT codes in the fast range by rounding x*r (r = RN(1/s)) to an
integer in one step and fall back to the exact quotient when x*r lies near a
half-integer.  These inputs put quotients exactly on, or within a few ulps of,
half-integers, with block scales that are not powers of two (so r differs from
1/s), and compare every byte with the oracle.  Inputs are built here; expected
values come from the oracle, which the CPU tests first check against np.rint
(round half to even) on the same constructions."""
import numpy as np
import pytest

import oracle
import quantized_collective_payloads_amd as qcp
from tests.gpu_util import assert_same_bytes, require_gpu, to_gpu, to_host

QMAX = {"int2": 1, "int4": 7, "int6": 31, "int8": 127}


def odd_mantissa_scales(rng, n, bits=15):
    """Positive float32 values m * 2^e with m odd and `bits` significant bits:
    never a power of two, and small multiples of them stay exact."""
    m = rng.integers(2 ** (bits - 1), 2 ** bits, n) | 1
    e = rng.integers(-40, -10, n)
    return np.ldexp(m.astype(np.float64), e).astype(np.float32)


def near_half_input(fmt, G):
    """400 blocks of G float32 values: x[0] = qmax*s (s with an odd 15-bit
    mantissa, so the block scale is exactly s) and the rest (k + 1/2)*s moved by
    -3..3 ulps, so x/s is a half-integer or within a few ulps of one.  Returns
    (x, s, k + 1/2, ulps)."""
    qm = QMAX[fmt]
    rng = np.random.default_rng(7 * G + qm)
    nb = 400
    s = odd_mantissa_scales(rng, nb)
    a = (s.astype(np.float64) * qm).astype(np.float32)        # block absmax
    h = rng.integers(-qm, qm, (nb, G)).astype(np.float64) + 0.5
    x = (h * s[:, None].astype(np.float64)).astype(np.float32)
    ulps = rng.integers(-3, 4, (nb, G)).astype(np.int32)
    x = (x.view(np.int32) + ulps).view(np.float32)
    x[:, 0] = a                                               # |x| < a elsewhere
    h[:, 0] = qm
    ulps[:, 0] = 0
    x[::7, 1] = -a[::7]
    h[::7, 1] = -qm
    ulps[::7, 1] = 0
    return x, s, h, ulps


GS_NEAR = [32, 64, 256, 1024]


@pytest.mark.parametrize("G", GS_NEAR)
@pytest.mark.parametrize("fmt", ["int2", "int4", "int6", "int8"])
def test_oracle_on_near_half_quotients(fmt, G):
    """Where x/s is an exact half-integer the oracle's code is the even
    neighbour; a few ulps off, the nearer integer."""
    x, s, h, ulps = near_half_input(fmt, G)
    wc, ws = oracle.quantize_blockwise(x.reshape(-1), "f32", G, fmt)
    assert_same_bytes(ws, s, "oracle scales = s")
    want = np.where(ulps == 0, np.rint(h),
                    np.where((ulps > 0) == (x > 0), np.floor(h) + 1, np.floor(h)))
    assert_same_bytes(wc, packed_codes(want.reshape(-1), fmt), "oracle codes")


@pytest.mark.gpu
@pytest.mark.parametrize("G", GS_NEAR)
@pytest.mark.parametrize("fmt", ["int2", "int4", "int6", "int8"])
def test_quantize_near_half_quotients(fmt, G):
    require_gpu()
    x = near_half_input(fmt, G)[0].reshape(-1)
    for n in (x.size, x.size - 5):                            # and a short last block
        codes, scales = qcp.quantize_blockwise(to_gpu(x[:n]), G, fmt)
        wc, ws = oracle.quantize_blockwise(x[:n], "f32", G, fmt)
        assert_same_bytes(to_host(scales), ws, f"scales {fmt} G={G} n={n}")
        assert_same_bytes(to_host(codes), wc, f"codes {fmt} G={G} n={n}")


def pack_int(c, fmt):
    """Signed codes -> LSB-first bytes (INT4 and INT8 only)."""
    c = np.asarray(c, np.int64)
    if fmt == "int8":
        return c.astype(np.int8).view(np.uint8)
    assert fmt == "int4" and c.size % 2 == 0
    u = (c & 0xF).astype(np.uint8)
    return u[0::2] | (u[1::2] << 4)


# (input format, output format, G, slices): the first three run the
# 8-slice INT4 kernel when no fp32 sums are asked for
TIE_CASES = [("int4", "int4", 512, 8), ("int4", "int2", 256, 8), ("int4", "int4", 32, 8),
             ("int4", "int4", 128, 3), ("int8", "int8", 64, 3), ("int8", "int6", 256, 8),
             ("int8", "int4", 1024, 2)]


def tie_slices(fin, fout, G, N):
    """Slice 0 holds codes c0 with scale s0 (odd mantissa), slice 1 codes c1 in
    {-1, 0, 1} with scale s0/2, the other slices zeros.  Every sum
    (c0 + c1/2)*s0 is exact, one element per block has c0 = qmax_out, so the
    output scale is s0 and the quotients are c0 + c1/2: exact ties wherever c1
    is odd.  Returns (buf, stride, sc, ss, L, s0, c0 + c1/2)."""
    qo = QMAX[fout]
    rng = np.random.default_rng(1000 + TIE_CASES.index((fin, fout, G, N)))
    nb = 131 if G >= 256 else 301
    L = nb * G                                         # whole blocks (INT4 needs even L)
    c0 = rng.integers(-(qo - 1), qo, L)
    c1 = rng.integers(-1, 2, L)
    c0[::G] = qo                                       # the block's absmax element
    c1[::G] = 0
    s0 = odd_mantissa_scales(rng, nb)
    cb = oracle.code_bytes(L, fin)
    stride = (cb + 15) // 16 * 16
    ss = (nb + 3) // 4 * 4
    buf = np.zeros(N * stride, np.uint8)
    sc = np.zeros(N * ss, np.float32)
    buf[:cb] = pack_int(c0, fin)
    buf[stride:stride + cb] = pack_int(c1, fin)
    sc[:nb] = s0
    sc[ss:ss + nb] = s0 / np.float32(2)
    for j in range(2, N):
        sc[j * ss:j * ss + nb] = odd_mantissa_scales(rng, nb)
    assert (c1 != 0).sum() > L // 3
    return buf, stride, sc, ss, L, s0, c0 + c1 / 2.0


@pytest.mark.parametrize("fin,fout,G,N", TIE_CASES)
def test_oracle_on_exact_ties(fin, fout, G, N):
    buf, stride, sc, ss, L, s0, q = tie_slices(fin, fout, G, N)
    wc, ws = oracle.dequant_reduce_requant(buf, stride, sc, ss, N, L, G, fin, fout)
    assert_same_bytes(ws, s0, "oracle scales = s0")
    assert_same_bytes(wc, packed_codes(np.rint(q), fout), "oracle codes = rint, ties to even")


@pytest.mark.gpu
@pytest.mark.parametrize("fin,fout,G,N", TIE_CASES)
def test_reduce_exact_ties(fin, fout, G, N):
    require_gpu()
    buf, stride, sc, ss, L, _, _ = tie_slices(fin, fout, G, N)
    wc, ws = oracle.dequant_reduce_requant(buf, stride, sc, ss, N, L, G, fin, fout)
    for want_sum in (False, True):
        out = qcp.dequant_reduce_requant(to_gpu(buf), stride, to_gpu(sc), ss, N, L, G, fin, fout,
                                         want_sum=want_sum)
        tag = f"{fin}->{fout} G={G} N={N} sums={want_sum}"
        assert_same_bytes(to_host(out[1]), ws, "scales " + tag)
        assert_same_bytes(to_host(out[0]), wc, "codes " + tag)


def packed_codes(q, fmt):
    """Integer codes -> packed bytes of `fmt` (INT2/4/6/8, LSB-first)."""
    b = {"int2": 2, "int4": 4, "int6": 6, "int8": 8}[fmt]
    u = (np.asarray(q, np.int64) & ((1 << b) - 1)).astype(np.uint64)
    bits = np.zeros(u.size * b, np.uint8)
    for i in range(b):
        bits[i::b] = (u >> np.uint64(i)) & np.uint64(1)
    return np.packbits(bits, bitorder="little")
