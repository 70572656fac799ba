"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each ``pin_*`` function takes the oracle module and raises AssertionError when
the oracle disagrees with an independent source:
  * figures the pages print (tests/golden/pages_figures.txt);
  * closed forms and invariants (bpw = b + 32/G, the round-trip bound, the
    block maximum mapping to +-qmax, N = 1 reduce = requantize of dequantize);
  * brute force over every candidate code on tiny blocks;
  * library routines that implement the same rounding independently (numpy
    float16 casts, torch bfloat16 / float8_e4m3fn casts, torch.round,
    np.unpackbits, exact rationals from ``fractions``).
The same functions run against deliberately broken copies of the oracle in
test_oracle_mutants.py, which checks that every planted mistake trips a pin.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pages_figures.txt")
QMAX = {"int2": 1, "int4": 7, "int6": 31, "int8": 127, "e4m3": 448}
BITS = {"int2": 2, "int4": 4, "int6": 6, "int8": 8, "e4m3": 8}
INT_FMTS = ["int2", "int4", "int6", "int8"]


def golden_figures():
    out = {}
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val, _src = [p.strip() for p in line.split("|", 2)]
            out[key] = val
    return out


# ---------------------------------------------------------------------------
# independent helpers (library routines, not the oracle's code)
# ---------------------------------------------------------------------------

def fields(stream: np.ndarray, n: int, b: int) -> np.ndarray:
    """Signed b-bit fields of an LSB-first bitstream, via np.unpackbits."""
    bits = np.unpackbits(np.asarray(stream, np.uint8), bitorder="little")[: n * b]
    u = (bits.reshape(n, b).astype(np.int64) << np.arange(b, dtype=np.int64)).sum(1)
    return np.where(u >= (1 << (b - 1)), u - (1 << b), u)


def pack_fields(codes: np.ndarray, b: int) -> np.ndarray:
    """Inverse of ``fields``: two's-complement b-bit fields, LSB first."""
    u = np.asarray(codes, np.int64) & ((1 << b) - 1)
    bits = ((u[:, None] >> np.arange(b, dtype=np.int64)) & 1).astype(np.uint8).reshape(-1)
    return np.packbits(bits, bitorder="little")


def e4m3_table() -> np.ndarray:
    """float32 value of each of the 256 E4M3FN codes, from torch's decoder."""
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()


def bf16_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_torch(x) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def widen(x, dt) -> np.ndarray:
    if dt == "bf16":
        return bf16_to_f32(x)
    return np.asarray(x).astype(np.float32)


def brute_int_codes(x32: np.ndarray, s: np.float32, qmax: int) -> np.ndarray:
    """argmin over every integer code of |fl32(x/s) - c|, ties to the even code."""
    if s == 0:
        return np.zeros(x32.size, np.int64)
    q = (x32.astype(np.float32) / np.float32(s)).astype(np.float64)
    cands = np.arange(-qmax, qmax + 1, dtype=np.float64)
    d = np.abs(q[:, None] - cands[None, :])
    best = d.min(1, keepdims=True)
    tie_ok = (d == best)
    # among the nearest candidates prefer the even one
    even = (np.abs(cands) % 2 == 0)[None, :]
    pick = np.where(tie_ok & even, 1, 0) + np.where(tie_ok, 1, 0)
    return cands[np.argmax(pick, axis=1)].astype(np.int64)


def brute_e4m3(q32: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3FN code to each q (ties to even mantissa; beyond the
    largest finite value the nearest is +-448), sign of zero kept."""
    tab = e4m3_table()[:127].astype(np.float64)        # codes 0x00..0x7e, all >= 0
    a = np.abs(q32.astype(np.float64))
    d = np.abs(a[:, None] - tab[None, :])
    best = d.min(1, keepdims=True)
    tie = d == best
    even = (np.arange(127) % 2 == 0)[None, :]
    code = np.argmax(np.where(tie & even, 2, 0) + np.where(tie, 1, 0), axis=1).astype(np.uint8)
    neg = np.signbit(q32)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def nudge(bits: np.ndarray, deltas) -> np.ndarray:
    """float32 values a few ulps either side of the given bit patterns."""
    b = np.asarray(bits, np.uint32).astype(np.int64)
    out = np.concatenate([b + d for d in deltas])
    out = out[(out >= 0) & (out < (1 << 31))]
    return out.astype(np.uint32).view(np.float32)


def f32_round_exact(fr: Fraction) -> np.float32:
    """Round a rational to the nearest binary32, ties to even (exact compare)."""
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]

    def key(v):
        lsb = int(np.array([v], np.float32).view(np.uint32)[0]) & 1
        return (abs(Fraction(float(v)) - fr), lsb)
    return min(cands, key=key)


# ---------------------------------------------------------------------------
# the pins
# ---------------------------------------------------------------------------

def pin_bpw_table(orc):
    """bpw from real buffer sizes = b + 32/G; the two printed endpoints."""
    fig = golden_figures()
    n = 1 << 16
    x = np.random.default_rng(7).standard_normal(n, dtype=np.float32)
    for b, G in [(2, 1024), (4, 256), (4, 64), (6, 128), (6, 32), (8, 32)]:
        packed, scales = orc.pack_subbyte(x, "f32", b, G)
        nbytes = packed.size + 4 * scales.size
        assert nbytes == orc.payload_bytes(n, b, G), (b, G)
        bpw = 8 * nbytes / n
        assert bpw == b + 32 / G, (b, G, bpw)
    assert f"{8 * orc.payload_bytes(n, 2, 1024) / n:.2f}" == fig["bpw.b2.G1024"]
    assert f"{8 * orc.payload_bytes(n, 6, 32) / n:.2f}" == fig["bpw.b6.G32"]
    # ragged sizes: a short last block still costs one scale; codes round up to a byte
    for n2, b, G in [(1, 2, 1024), (1023, 6, 32), (1025, 4, 512), (7, 2, 32)]:
        packed, scales = orc.pack_subbyte(x[:n2], "f32", b, G)
        assert packed.size + 4 * scales.size == orc.payload_bytes(n2, b, G)
        assert scales.size == -(-n2 // G) and packed.size == -(-n2 * b // 8)


def pin_volume_figures(orc):
    """The pages' per-iteration volumes, in units of M 16-bit values."""
    fig = golden_figures()
    M = 1 << 20                        # model elements (multiple of every G)
    fp16_bytes = 2 * M
    codes8 = orc.payload_bytes(M, 8, 256) - 4 * (M // 256)
    codes4 = orc.payload_bytes(M, 4, 512) - 4 * (M // 512)
    qwz = codes8 / fp16_bytes
    qgz = codes4 / fp16_bytes
    assert qwz == float(fig["qwz.forward_gather"])
    assert qgz == float(fig["qgz.gradient"])
    assert 1 + 1 + 1 == float(fig["zero3.total"]) == float(fig["zero3.stage_volume"])
    assert qwz + float(fig["hpz.cross_node_backward_gather"]) + qgz == float(fig["zeropp.total"])
    N = 8
    assert qgz / N == float(fig["qgz.cross_node_per_gpu.N8"])
    assert N * qgz == float(fig["onehop.cross_node.N8"])
    # the scale words the pages leave out add 4/(2G) per element
    assert orc.payload_bytes(M, 8, 256) / fp16_bytes == 0.5 + 2 / 256
    assert int(float(fig["qgz.bucket_elements"])) == 8 * 62_500_000


def pin_f16_rounding(orc):
    """fp32 -> fp16 round-to-nearest-even matches numpy on every fp16 value's
    neighbourhood (including subnormals, the overflow edge and ties)."""
    h = np.arange(0, 0x7c00, dtype=np.uint32)           # all finite non-negative fp16
    v = np.concatenate([h.astype(np.uint16).view(np.float16).astype(np.float32)])
    mids = []
    f = v.astype(np.float64)
    mids.append(((f[:-1] + f[1:]) / 2).astype(np.float32))   # exact ties (fit in fp32)
    base = np.concatenate([v, mids[0], np.float32([65504, 65519.996, 65520, 65536, 1e-8, 3e-8])])
    bits = base.view(np.uint32)
    near = nudge(bits, (-2, -1, 0, 1, 2))
    near = near[np.isfinite(near)]
    x = np.concatenate([near, -near])
    got = orc.f32_to_f16_bits(x)
    with np.errstate(over="ignore"):                    # values past 65520 become inf
        want = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], want[bad[:5]])
    # widening fp16 -> fp32 is exact
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    w = orc.f16_bits_to_f32(allh)
    ref = allh.view(np.float16).astype(np.float32)
    same = (w.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(w) & np.isnan(ref))
    assert same.all()


def pin_bf16_rounding(orc):
    """fp32 -> bf16 round-to-nearest-even matches torch on every bf16 value's
    neighbourhood, exact ties, and random bit patterns."""
    hb = np.arange(0, 0x7f80, dtype=np.uint32)
    v = (hb << 16).view(np.float32)
    tie = ((hb << 16) | 0x8000).view(np.float32)
    rnd = np.random.default_rng(3).integers(0, 0x7f800000, 200_000, dtype=np.uint32).view(np.float32)
    base = np.concatenate([v, tie, rnd]).view(np.uint32)
    near = nudge(base, (-1, 0, 1))
    near = near[np.isfinite(near)]
    x = np.concatenate([near, -near])
    got = orc.f32_to_bf16_bits(x)
    want = f32_to_bf16_torch(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], want[bad[:5]])


def pin_e4m3_decode(orc):
    """All 256 E4M3FN codes decode to torch's float8_e4m3fn values."""
    codes = np.arange(256, dtype=np.uint32).astype(np.uint8)
    got = orc.e4m3_to_f32(codes)
    want = e4m3_table()
    same = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
    assert same.all(), np.nonzero(~same)[0][:8]
    assert got[0x7e] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def pin_e4m3_encode(orc):
    """fp32 -> E4M3FN: brute-force nearest code and torch's cast agree with
    the oracle on all fp32 values around every code and every midpoint."""
    tab = e4m3_table()[:127].astype(np.float64)
    mids = (tab[:-1] + tab[1:]) / 2
    base = np.concatenate([tab, mids, [448.0, 456.0, 460.0, 463.9, 2.0 ** -10, 2.0 ** -11]]).astype(np.float32)
    bits = base.view(np.uint32)
    near = nudge(bits, range(-3, 4))
    near = near[np.isfinite(near) & (near >= 0)]
    rnd = np.random.default_rng(5).uniform(0, 460, 20000).astype(np.float32)
    x = np.concatenate([near, rnd, np.float32([0.0])])
    x = np.concatenate([x, -x])
    got = orc.f32_to_e4m3(x)
    want = brute_e4m3(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], want[bad[:5]])
    tor = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (tor == got).all()


def pin_int_codes_bruteforce(orc):
    """Tiny blocks (G <= 8): every code is the brute-force nearest integer to
    the binary32 quotient, ties to even, and the scale is fl(absmax/qmax)."""
    rng = np.random.default_rng(11)
    for fmt in INT_FMTS:
        qmax = QMAX[fmt]
        for G in (1, 2, 3, 5, 8):
            n = 40 * G + 3
            x = (rng.standard_normal(n) * rng.choice([1e-3, 1.0, 300.0])).astype(np.float32)
            # plant exact ties: values that divide to k + 0.5
            x[:4] = np.float32([qmax, 0.5, -1.5, 2.5]) if qmax >= 3 else np.float32([1.0, 0.5, -0.5, 0.25])
            codes, scales = orc.quantize_blockwise(x, "f32", G, fmt)
            c = fields(codes, n, BITS[fmt])
            for k in range(scales.size):
                blk = x[k * G:(k + 1) * G]
                a = np.float32(np.abs(blk).max())
                s = np.float32(a / np.float32(qmax))
                assert scales[k].view(np.uint32) == s.view(np.uint32), (fmt, G, k)
                assert (c[k * G:(k + 1) * G] == brute_int_codes(blk, s, qmax)).all(), (fmt, G, k)


def pin_int_codes_torch(orc):
    """Bigger blocks: codes equal torch.round (half-even) of the float32
    quotient, clamped; scales equal torch's float32 absmax / qmax."""
    rng = np.random.default_rng(12)
    for fmt in INT_FMTS:
        qmax = QMAX[fmt]
        for G in (32, 256, 1024):
            n = 3 * G + 17
            x = (rng.standard_normal(n) * 0.02).astype(np.float32)
            codes, scales = orc.quantize_blockwise(x, "f32", G, fmt)
            t = torch.from_numpy(x)
            pad = torch.zeros(scales.size * G - n)
            blocks = torch.cat([t, pad]).view(-1, G)
            s = blocks.abs().amax(1) / qmax
            q = torch.round(blocks / s[:, None]).clamp(-qmax, qmax).reshape(-1)[:n]
            assert (scales == s.numpy()).all(), fmt
            assert (fields(codes, n, BITS[fmt]) == q.numpy().astype(np.int64)).all(), (fmt, G)


def pin_int_codes_near_ties(orc):
    """Quotients on and next to exact half-integers, with scales whose
    reciprocal is inexact (odd integers): the code must follow the true
    binary32 quotient (torch's IEEE division, then torch.round half-even), not
    x times a rounded reciprocal."""
    for fmt in INT_FMTS:
        qmax = QMAX[fmt]
        xs, ss = [], []
        for sv in range(3, 200, 2):
            s = np.float32(sv)
            k = np.arange(-qmax, qmax, dtype=np.float32)
            x = (s * (k + np.float32(0.5))).astype(np.float32)
            near = nudge(np.abs(x).view(np.uint32), (-1, 0, 1))
            near = np.concatenate([near, -near])
            G = near.size + 1
            blk = np.concatenate([np.float32([s * qmax]), near])    # block max -> scale exactly s
            xs.append(blk)
            ss.append(G)
        for blk, G in zip(xs, ss):
            codes, scales = orc.quantize_blockwise(blk, "f32", G, fmt)
            t = torch.from_numpy(blk)
            sc = torch.tensor(scales[0])
            want = torch.round(t / sc).clamp(-qmax, qmax).numpy().astype(np.int64)
            assert (fields(codes, blk.size, BITS[fmt]) == want).all(), (fmt, G)


def pin_e4m3_quantize(orc):
    """E4M3 blocks: scale = absmax/448, codes = brute-force nearest E4M3 of the
    binary32 quotient; the zero block gives scale +0 and codes 0x00."""
    rng = np.random.default_rng(13)
    G = 128
    n = 5 * G + 9
    x = (rng.standard_normal(n) * 5e-4).astype(np.float32)
    x[G:2 * G] = 0.0
    x[G + 3] = -0.0
    x[2 * G + 1] = -0.0
    codes, scales = orc.quantize_blockwise(x, "f32", G, "e4m3")
    for k in range(scales.size):
        blk = x[k * G:(k + 1) * G]
        s = np.float32(np.float32(np.abs(blk).max()) / np.float32(448))
        assert scales[k] == s
        if s == 0:
            assert (codes[k * G:(k + 1) * G] == 0).all() and not np.signbit(scales[k])
        else:
            want = brute_e4m3((blk / s).astype(np.float32))
            assert (codes[k * G:(k + 1) * G] == want).all(), k
    assert codes[2 * G + 1] == 0x80          # -0 in a non-zero block keeps its sign


def pin_absmax_maps_to_qmax(orc):
    """The element attaining the block maximum gets code +-qmax."""
    rng = np.random.default_rng(14)
    for fmt in INT_FMTS + ["e4m3"]:
        for G in (32, 512):
            n = 6 * G
            x = (rng.standard_normal(n) * 0.01).astype(np.float32)
            x[::G] = -np.abs(x[::G]) * 50          # the first element of each block is the extreme, negative
            x[G + 5] = 0.9                          # block 1: a positive extreme instead
            codes, scales = orc.quantize_blockwise(x, "f32", G, fmt)
            for k in range(n // G):
                blk = x[k * G:(k + 1) * G]
                i = int(np.argmax(np.abs(blk)))
                if fmt == "e4m3":
                    c = codes[k * G + i]
                    assert c == (0xFE if blk[i] < 0 else 0x7E), (fmt, G, k, c)
                else:
                    c = fields(codes, n, BITS[fmt])[k * G + i]
                    assert c == (-QMAX[fmt] if blk[i] < 0 else QMAX[fmt]), (fmt, G, k, c)


def pin_roundtrip_bound(orc):
    """|x - fl(c*s)| <= s/2 + qmax*s*2^-22 (INT); <= half the E4M3 spacing at
    |q|, times s, plus the same slack (E4M3); fp16/bf16 outputs add half an ulp."""
    rng = np.random.default_rng(15)
    for dt in ("f16", "bf16", "f32"):
        for fmt in INT_FMTS + ["e4m3"]:
            G = 64
            n = 8 * G + 13
            x32 = (rng.standard_normal(n) * 0.02).astype(np.float32)
            x = {"f16": x32.astype(np.float16), "bf16": f32_to_bf16_torch(x32), "f32": x32}[dt]
            xv = widen(x, dt).astype(np.float64)
            codes, scales = orc.quantize_blockwise(x, dt, G, fmt)
            y = orc.dequantize_blockwise(codes, scales, fmt, n, G, "f32").astype(np.float64)
            s = np.repeat(scales.astype(np.float64), G)[:n]
            qmax = QMAX[fmt]
            if fmt == "e4m3":
                q = np.abs(xv / np.where(s == 0, 1, s))
                e = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
                spacing = 2.0 ** (e - 3)
                bound = s * spacing / 2 + qmax * s * 2.0 ** -22
            else:
                bound = s / 2 + qmax * s * 2.0 ** -22
            err = np.abs(xv - y)
            assert (err <= bound).all(), (dt, fmt, float((err - bound).max()))
            # the 16-bit output adds at most half an ulp of that format
            if dt != "f32":
                y16 = widen(orc.dequantize_blockwise(codes, scales, fmt, n, G, dt), dt).astype(np.float64)
                ulp = np.abs(y) * (2.0 ** -11 if dt == "f16" else 2.0 ** -8) + 2.0 ** -24
                assert (np.abs(y16 - y) <= ulp).all(), (dt, fmt)


def pin_bitstream_layout(orc):
    """With a scale of exactly 1 (block max = qmax), every integer input is its
    own code: the packed stream must equal np.packbits of the LSB-first
    two's-complement fields."""
    rng = np.random.default_rng(16)
    for fmt in INT_FMTS:
        b, qmax = BITS[fmt], QMAX[fmt]
        G = 32
        n = 7 * G + 11
        c = rng.integers(-qmax, qmax + 1, n)
        c[::G] = qmax                                  # every block holds qmax -> s = 1
        codes, scales = orc.quantize_blockwise(c.astype(np.float32), "f32", G, fmt)
        assert (scales == 1.0).all()
        want = pack_fields(c, b)
        assert codes.size == want.size and (codes == want).all(), fmt
        # 4-tuples of codes pack and unpack exactly (6-bit: 3 bytes per 4 codes)
        tup = rng.integers(-qmax, qmax + 1, (50_000, 4))
        if b <= 4:      # small formats: every 4-tuple
            allc = np.arange(-qmax, qmax + 1)
            tup = np.stack(np.meshgrid(*[allc] * 4, indexing="ij"), -1).reshape(-1, 4)
        blocks = np.concatenate([tup, np.full((tup.shape[0], 1), qmax)], 1).reshape(-1)
        codes2, sc2 = orc.quantize_blockwise(blocks.astype(np.float32), "f32", 5, fmt)
        assert (sc2 == 1.0).all()
        assert (fields(codes2, blocks.size, b) == blocks).all(), fmt
        y = orc.dequantize_blockwise(codes2, sc2, fmt, blocks.size, 5, "f32")
        assert (y == blocks).all(), fmt


def pin_pack8_is_int8(orc):
    """8-bit packing is the plain INT8 quantizer, byte for byte."""
    x = (np.random.default_rng(17).standard_normal(5000) * 0.02).astype(np.float32)
    a, sa = orc.pack_subbyte(x, "f32", 8, 256)
    b, sb = orc.quantize_blockwise(x, "f32", 256, "int8")
    assert (a == b).all() and (sa == sb).all()
    assert (a.view(np.int8).astype(np.int64) == fields(a, x.size, 8)).all()


def pin_dequant_casts(orc):
    """Dequantize = one binary32 product, then the library's RNE cast."""
    rng = np.random.default_rng(18)
    for fmt in INT_FMTS + ["e4m3"]:
        G = 128
        n = 4 * G + 1
        x = (rng.standard_normal(n) * 0.02).astype(np.float32)
        x[:G] *= np.float32(1e-6)                       # small block: fp16 subnormal outputs
        codes, scales = orc.quantize_blockwise(x, "f32", G, fmt)
        if fmt == "e4m3":
            val = e4m3_table()[codes[:n]]
        else:
            val = fields(codes, n, BITS[fmt]).astype(np.float32)
        prod = (val * np.repeat(scales, G)[:n]).astype(np.float32)
        assert (orc.dequantize_blockwise(codes, scales, fmt, n, G, "f32") == prod).all()
        assert (orc.dequantize_blockwise(codes, scales, fmt, n, G, "f16").view(np.uint16)
                == prod.astype(np.float16).view(np.uint16)).all(), fmt
        assert (orc.dequantize_blockwise(codes, scales, fmt, n, G, "bf16")
                == f32_to_bf16_torch(prod)).all(), fmt


def _slices(orc, rng, n_slices, L, G, fmt, stride_pad=16):
    """Quantize n_slices random fp32 slices (different magnitudes) and lay them
    out in one buffer with a 16-byte-aligned stride."""
    cb = orc.code_bytes(L, fmt)
    stride = ((cb + 15) // 16) * 16 + stride_pad
    nb = orc.n_blocks(L, G)
    sstride = nb + 3
    buf = np.zeros(stride * n_slices, np.uint8)
    sc = np.zeros(sstride * n_slices, np.float32)
    for j in range(n_slices):
        x = (rng.laplace(0, 1e-3 * (1 + j), L)).astype(np.float32)
        c, s = orc.quantize_blockwise(x, "f32", G, fmt)
        buf[j * stride: j * stride + cb] = c
        sc[j * sstride: j * sstride + nb] = s
    return buf, stride, sc, sstride


def _decoded(orc, buf, stride, sc, sstride, n_slices, L, G, fmt):
    """Per-slice dequantized values d_j = value(c_j) * s_j (exact in fp64)."""
    d = []
    for j in range(n_slices):
        cb = orc.code_bytes(L, fmt)
        c = buf[j * stride: j * stride + cb]
        val = e4m3_table()[c[:L]] if fmt == "e4m3" else fields(c, L, BITS[fmt])
        s = np.repeat(sc[j * sstride: j * sstride + orc.n_blocks(L, G)], G)[:L]
        d.append(np.asarray(val, np.float64) * s.astype(np.float64))
    return d


def pin_reduce_n1(orc):
    """N = 1: the reduce is exactly requantize(dequantize to fp32)."""
    rng = np.random.default_rng(19)
    for fin, fout in [("int4", "int4"), ("e4m3", "e4m3"), ("int8", "int2"), ("int2", "int8")]:
        G, L = 64, 5 * 64 + 7
        buf, stride, sc, ss = _slices(orc, rng, 1, L, G, fin)
        if fin == "e4m3":
            buf[3] = 0x80                                   # a -0 code keeps its sign
        co, so, su = orc.dequant_reduce_requant(buf, stride, sc, ss, 1, L, G, fin, fout, want_sum=True)
        d = orc.dequantize_blockwise(buf, sc, fin, L, G, "f32")
        assert (su.view(np.uint32) == d.view(np.uint32)).all(), (fin, fout)
        c2, s2 = orc.quantize_blockwise(d, "f32", G, fout)
        assert (co == c2).all() and (so == s2).all(), (fin, fout)


def pin_reduce_fma_chain(orc):
    """N = 2, 3: each step of the sum is one rounding of the exact
    acc + c*s (an fmaf), checked with exact rationals."""
    rng = np.random.default_rng(20)
    for fin in ("int2", "int4", "e4m3"):
        G, L = 32, 32 * 3
        for N in (2, 3):
            buf, stride, sc, ss = _slices(orc, rng, N, L, G, fin)
            _, _, su = orc.dequant_reduce_requant(buf, stride, sc, ss, N, L, G, fin, "int4", want_sum=True)
            for i in range(0, L, 7):
                acc = Fraction(0)
                for j in range(N):
                    cb = orc.code_bytes(L, fin)
                    c = buf[j * stride: j * stride + cb]
                    val = float(e4m3_table()[c[i]]) if fin == "e4m3" else int(fields(c, L, BITS[fin])[i])
                    s = float(sc[j * ss + i // G])
                    acc = Fraction(float(f32_round_exact(acc + Fraction(val) * Fraction(s))))
                assert float(acc) == float(su[i]), (fin, N, i)


def pin_reduce_error_bound(orc):
    """N = 8 with per-slice scales: the fp32 sum is within gamma_N * sum|d_j|
    of the exact sum (recursive summation bound), and the requantized output
    obeys the round-trip bound on that sum."""
    rng = np.random.default_rng(21)
    for fin, fout, G in [("int4", "int4", 512), ("e4m3", "e4m3", 128), ("int8", "int8", 256)]:
        N, L = 8, 3 * G + 160
        buf, stride, sc, ss = _slices(orc, rng, N, L, G, fin)
        co, so, su = orc.dequant_reduce_requant(buf, stride, sc, ss, N, L, G, fin, fout, want_sum=True)
        d = _decoded(orc, buf, stride, sc, ss, N, L, G, fin)
        exact = np.sum(d, axis=0)
        mag = np.sum(np.abs(d), axis=0)
        u = 2.0 ** -24
        gamma = N * u / (1 - N * u)
        assert (np.abs(su.astype(np.float64) - exact) <= gamma * mag + 1e-45).all(), (fin, fout)
        y = orc.dequantize_blockwise(co, so, fout, L, G, "f32").astype(np.float64)
        s = np.repeat(so.astype(np.float64), G)[:L]
        if fout == "e4m3":
            q = np.abs(su / np.where(s == 0, 1, s))
            bound = s * 2.0 ** (np.floor(np.log2(np.maximum(q, 2.0 ** -6))) - 4) + 448 * s * 2.0 ** -22
        else:
            bound = s / 2 + QMAX[fout] * s * 2.0 ** -22
        assert (np.abs(su - y) <= bound).all(), (fin, fout)


def pin_accum_step0(orc):
    """From the all-zero state (s = 0, codes 0x00), one accumulate step equals
    quantizing the micro-batch gradient to E4M3 directly."""
    rng = np.random.default_rng(22)
    G = 128
    n = 9 * G + 40
    g = f32_to_bf16_torch((rng.standard_normal(n) * 5e-4).astype(np.float32))
    g[g == 0x8000] = 0                                   # no -0 entries (0 + -0 = +0)
    st_c, st_s = orc.fp8_accum_requant(np.zeros(n, np.uint8), np.zeros(orc.n_blocks(n, G), np.float32),
                                       g, "bf16", G)
    qc, qs = orc.quantize_blockwise(g, "bf16", G, "e4m3")
    assert (st_c == qc).all() and (st_s == qs).all()


def pin_accum_exact(orc):
    """Where every intermediate is exactly representable the state must hold
    the exact running sum: state values and integer gradients with a block
    maximum of 448 keep the scale at exactly 1."""
    G = 32
    tab = e4m3_table()
    n = 4 * G
    rng = np.random.default_rng(23)
    ints = rng.integers(-16, 17, n).astype(np.float32)
    ints[::G] = 448.0
    st_c, st_s = orc.quantize_blockwise(ints, "f32", G, "e4m3")
    assert (st_s == 1.0).all() and (tab[st_c] == ints).all()
    g = rng.integers(-8, 9, n).astype(np.float32)
    g[::G] = 0.0
    st_c2, st_s2 = orc.fp8_accum_requant(st_c, st_s, f32_to_bf16_torch(g), "bf16", G)
    assert (st_s2 == 1.0).all()
    want = brute_e4m3((ints + g).astype(np.float32))
    assert (st_c2 == want).all()


def pin_accum_library(orc):
    """General case against torch-CPU library conversions for every rounding
    step: float8 decode, float32 product, bf16 cast, float32 add, bf16 cast,
    float32 absmax/448, float32 quotient, float8 cast."""
    rng = np.random.default_rng(24)
    G = 128
    n = 6 * G + 50
    nb = orc.n_blocks(n, G)
    st_c = np.zeros(n, np.uint8)
    st_s = np.zeros(nb, np.float32)
    for m in range(4):
        g = f32_to_bf16_torch((rng.standard_normal(n) * 5e-4 * (1 + m)).astype(np.float32))
        st_c_new, st_s_new = orc.fp8_accum_requant(st_c, st_s, g, "bf16", G)
        e = torch.from_numpy(st_c.copy()).view(torch.float8_e4m3fn).float()
        s = torch.from_numpy(np.repeat(st_s, G)[:n].copy())
        d = (e * s).to(torch.bfloat16).float()
        t = (d + torch.from_numpy(bf16_to_f32(g).copy())).to(torch.bfloat16).float()
        pad = torch.zeros(nb * G - n)
        blocks = torch.cat([t, pad]).view(nb, G)
        sc = blocks.abs().amax(1) / 448.0
        q = (blocks / torch.where(sc == 0, torch.ones_like(sc), sc)[:, None]).reshape(-1)[:n]
        code = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
        code[np.repeat((sc == 0).numpy(), G)[:n]] = 0
        assert (st_s_new == sc.numpy()).all(), m
        assert (st_c_new == code).all(), m
        st_c, st_s = st_c_new, st_s_new


def simulate_two_hop(slices_of, grads, K, N, C):
    """The two-hop qgZ exchange on K*N virtual ranks in plain float64 numpy.

    grads[a][i] is the bucket of GPU i on node a (K*N*C values).  slices_of(g)
    returns the N send slices (an (N, K*C) array) a GPU prepares from its own
    bucket.  Hop 1: GPU (a, j) sums slice j of every GPU of node a.  Hop 2: GPU
    (a, j) sends piece b of that sum to GPU (b, j), which sums what it receives.
    Returns final[r] for global rank r = b*N + j (C values each)."""
    hop1 = {}
    for a in range(K):
        send = [np.asarray(slices_of(grads[a][i]), np.float64) for i in range(N)]
        for j in range(N):
            hop1[a, j] = sum(send[i][j] for i in range(N))
    final = {}
    for b in range(K):
        for j in range(N):
            final[b * N + j] = sum(hop1[a, j][b * C:(b + 1) * C] for a in range(K))
    return final


def pin_reorder_two_hop(orc):
    """After the reordering, the two hops leave on rank r exactly the sum over
    all ranks of chunk r -- the requirement the reordering exists for [ZPP
    "Tensor-slice reordering fixes incorrect gradient placement"].  Integer-
    valued data keeps every sum exact.  The same exchange without reordering
    misplaces chunks (so the simulation can tell)."""
    rng = np.random.default_rng(31)
    for K, N, C in [(1, 1, 3), (1, 4, 2), (2, 2, 5), (2, 4, 3), (3, 8, 2), (4, 8, 1), (2, 3, 4)]:
        n = K * N * C
        grads = [[rng.integers(-100, 100, n).astype(np.float32) for _ in range(N)] for _ in range(K)]
        total = sum(g.astype(np.float64) for row in grads for g in row)
        final = simulate_two_hop(lambda g: orc.reorder_slices(g, "f32", K, N).reshape(N, K * C),
                                 grads, K, N, C)
        for r in range(K * N):
            assert np.array_equal(final[r], total[r * C:(r + 1) * C]), (K, N, C, r)
        if K > 1 and N > 1:
            plain = simulate_two_hop(lambda g: g.reshape(N, K * C), grads, K, N, C)
            assert any(not np.array_equal(plain[r], total[r * C:(r + 1) * C]) for r in range(K * N))


def pin_reorder_quantize_layout(orc):
    """The fused sender = the reordering, then an independent blockwise
    quantization of every slice, written at the N-slice strides."""
    rng = np.random.default_rng(32)
    for K, N, C, G, fmt in [(2, 4, 40, 32, "int4"), (3, 2, 104, 64, "int8"), (1, 3, 72, 32, "e4m3")]:
        x = (rng.standard_normal(K * N * C) * 0.01).astype(np.float16)
        codes, cs, scales, ss = orc.reorder_quantize(x, "f16", K, N, G, fmt)
        y = orc.reorder_slices(x, "f16", K, N).reshape(N, K * C)
        L = K * C
        for j in range(N):
            wc, ws = orc.quantize_blockwise(y[j], "f16", G, fmt)
            assert np.array_equal(codes[j * cs:j * cs + wc.size], wc), (K, N, j)
            assert np.array_equal(scales[j * ss:j * ss + ws.size], ws), (K, N, j)
            assert np.array_equal(y[j][:C], x[j * C:(j + 1) * C])      # slice j starts with chunk j
        assert cs >= orc.code_bytes(L, fmt) and cs % 16 == 0


AQUAVIT_LEVELS = [(b, G) for b in (2, 4, 6, 8) for G in (32, 64, 128, 256, 512, 1024)]


def pin_aquavit_schedule(orc):
    """The ascending schedule realized by granularity modulation starts at the
    2-bit/G=1024 level (2.03 bpw) and ends at 6-bit/G=32 (7.00 bpw), as [AQV]
    Table 1 / Section 5.1 print; in between the level is non-decreasing and is,
    by brute force over all 24 (b, G) levels, the one nearest the target."""
    fig = golden_figures()
    T = 1000
    b0, G0 = orc.aquavit_level(0, T)
    b1, G1 = orc.aquavit_level(T, T)
    assert f"{b0 + 32 / G0:.2f}" == fig["bpw.b2.G1024"] and (b0, G0) == (2, 1024)
    assert f"{b1 + 32 / G1:.2f}" == fig["bpw.b6.G32"] and (b1, G1) == (6, 32)
    prev = 0.0
    for t in range(T + 1):
        b, G = orc.aquavit_level(t, T)
        bpw = b + 32 / G
        target = orc.aquavit_target(t, T)
        best = min(abs(bb + 32 / gg - target) for bb, gg in AQUAVIT_LEVELS)
        assert abs(bpw - target) == best, t
        assert bpw >= prev, t
        prev = bpw
    assert orc.aquavit_target(0, T) < 2.03125 < 7.0 - 0.02 < orc.aquavit_target(T, T) < 7.0


def pin_records_layout(orc):
    """Metadata interleaving: the record stream is, block by block, the block's
    fp32 scale then its codes -- assembled here with numpy from the separate
    codes and scales -- and has exactly payload_bytes(n, b, G) bytes."""
    rng = np.random.default_rng(33)
    for b, G, n in [(2, 1024, 3 * 1024 + 77), (6, 32, 40 * 32 + 5), (4, 64, 64 * 9), (8, 32, 31)]:
        x = f32_to_bf16_torch((rng.standard_normal(n) * 0.015).astype(np.float32))
        rec = orc.pack_records(x, "bf16", b, G)
        codes, scales = orc.pack_subbyte(x, "bf16", b, G)
        want = []
        for k in range(scales.size):
            lo = k * G * b // 8
            hi = min(lo + G * b // 8, codes.size)
            want += [scales[k:k + 1].view(np.uint8), codes[lo:hi]]
        want = np.concatenate(want)
        assert rec.size == orc.payload_bytes(n, b, G) == want.size
        assert np.array_equal(rec, want), (b, G, n)
        y = orc.unpack_records(rec, n, b, G, "bf16")
        assert np.array_equal(y, orc.unpack_subbyte(codes, scales, n, b, G, "bf16")), (b, G, n)


ALL_PINS = [pin_bpw_table, pin_volume_figures, pin_f16_rounding, pin_bf16_rounding,
            pin_e4m3_decode, pin_e4m3_encode, pin_int_codes_bruteforce, pin_int_codes_torch,
            pin_int_codes_near_ties, pin_e4m3_quantize, pin_absmax_maps_to_qmax, pin_roundtrip_bound,
            pin_bitstream_layout, pin_pack8_is_int8, pin_dequant_casts, pin_reduce_n1,
            pin_reduce_fma_chain, pin_reduce_error_bound, pin_accum_step0, pin_accum_exact,
            pin_accum_library, pin_reorder_two_hop, pin_reorder_quantize_layout,
            pin_aquavit_schedule, pin_records_layout]
