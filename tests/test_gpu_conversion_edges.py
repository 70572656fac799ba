"""GPU parity on the rounding edges of the hardware conversions, byte for byte
against the CPU oracle, through the library's entry points.

The kernels encode E4M3 with the gfx950 converter (after an exact quotient),
decode E4M3 with its inverse, and narrow fp32 to bf16/fp16 with the packed
converters.  Random data reaches an E4M3 midpoint about once in 2^20 elements,
so these tests put the quotients there on purpose:

  * blocks whose absmax is exactly 448 have the scale 448/448 = 1, so the
    quotient of every element is the element itself: every finite E4M3 value,
    every midpoint between neighbours (ties to even mantissa, including the
    subnormal tie 2^-10), each of them 1..3 ulps either side, both signs, and
    signed zeros -- in quantize (fp32, bf16, fp16 input), in the FP8
    accumulate from the zero state, and in the E4M3-output reduce, whose fp32
    sums are built to land on the same values exactly;
  * blocks whose scale is subnormal, where the quotient passes 448 (the
    saturation band): fp32 input m * 2^-149 under the scale 2^-149, bf16
    gradients made of subnormals, reduce sums of a few times 2^-149;
  * dequantize products c * s that land on bf16 and fp16 ties, subnormal fp16
    ties and the fp16 overflow threshold 65520;
  * the tiny qwZ round trip (1,048,576 fp16 ~ N(0, 0.02) from seed 0, INT8,
    G = 256) exactly as specified.

Format facts used to build the inputs: OCP E4M3FN has a 4-bit exponent (bias 7)
and a 3-bit mantissa, subnormals m * 2^-9, largest finite value 448 (AGoQ,
Section 2.B, names FP8; E4M3 is the reading taken for it)."""
import numpy as np
import pytest
import torch

import oracle
import qcp_synthetic as S
import quantized_collective_payloads_amd as qcp
from tests.gpu_util import assert_same_bytes, cast_host, require_gpu, to_gpu, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def e4m3_positive_values() -> np.ndarray:
    """Every positive finite E4M3FN value, ascending, from the format definition."""
    v = [m * 2.0 ** -9 for m in range(1, 8)]
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue                    # S.1111.111 is NaN
            v.append(2.0 ** (e - 7) * (1 + m / 8))
    return np.array(v, np.float64)


def ulp_neighbours(v32: np.ndarray, k: int) -> np.ndarray:
    """v and the values 1..k ulps either side of it, in the precision of v32."""
    out = [v32]
    up, down = v32.copy(), v32.copy()
    for _ in range(k):
        up = np.nextafter(up, np.array(np.inf, v32.dtype))
        down = np.nextafter(down, np.array(-np.inf, v32.dtype))
        out += [up, down]
    return np.concatenate(out)


def edge_targets(dtype: str) -> np.ndarray:
    """E4M3 values and midpoints, +-0..3 ulps of the input type, both signs, and
    +-0, limited to |v| <= 448; as float32 holding values exact in `dtype`."""
    pos = e4m3_positive_values()
    mids = (np.concatenate([[0.0], pos[:-1]]) + pos) / 2       # 2^-10 is the first
    base = np.concatenate([pos, mids])
    npdt = {"f32": np.float32, "f16": np.float16}.get(dtype)
    if npdt is not None:
        near = ulp_neighbours(base.astype(npdt), 3).astype(np.float32)
    else:                                       # bf16: step the 16-bit patterns
        b = cast_host(base.astype(np.float32), "bf16").astype(np.int32)
        near = np.concatenate([b + d for d in range(-3, 4)]).astype(np.uint32) << 16
        near = near.view(np.float32)
    near = near[(near > 0) & (near <= 448)]
    v = np.unique(near)
    v = np.concatenate([v, -v, np.array([0.0, -0.0], np.float32)])
    return v.astype(np.float32)


def blocks_with_absmax_448(vals: np.ndarray, G: int, seed: int) -> np.ndarray:
    """Lay vals out in blocks of G with one element of magnitude 448 each (at a
    varying position, alternating sign), so every block's scale is exactly 1."""
    rng = np.random.default_rng(seed)
    vals = vals[rng.permutation(vals.size)]
    per = G - 1
    nblk = -(-vals.size // per)
    vals = np.concatenate([vals, np.zeros(nblk * per - vals.size, np.float32)])
    out = np.empty(nblk * G, np.float32)
    for k in range(nblk):
        blk = list(vals[k * per:(k + 1) * per])
        blk.insert(int(rng.integers(0, G)), np.float32(448.0 if k % 2 == 0 else -448.0))
        out[k * G:(k + 1) * G] = blk
    return out


@pytest.mark.parametrize("G", [32, 128, 1024])
@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_e4m3_encoder_on_ties_and_neighbours(dt, G):
    vals = edge_targets(dt)
    x32 = blocks_with_absmax_448(vals, G, 11 + G)
    xh = cast_host(x32, dt)
    assert np.array_equal(oracle_values(xh, dt).view(np.uint32), x32.view(np.uint32)), "exact in dt"
    codes, scales = qcp.quantize_blockwise(to_gpu(xh, dt), G, "e4m3")
    wc, ws = oracle.quantize_blockwise(xh, dt, G, "e4m3")
    assert np.all(ws == 1.0), "every block's scale is 448/448 = 1"
    assert_same_bytes(to_host(scales), ws, f"E4M3 scales {dt} G={G}")
    assert_same_bytes(to_host(codes), wc, f"E4M3 codes of ties and neighbours {dt} G={G}")
    # the inputs really sit on midpoints: some codes round up, some down, to even
    assert (wc == 0x80).any() and (wc == 0x00).any()


def oracle_values(xh: np.ndarray, dt: str) -> np.ndarray:
    """The float32 values of host data of type dt (all exact)."""
    if dt == "bf16":
        return (xh.astype(np.uint32) << 16).view(np.float32)
    return xh.astype(np.float32)


@pytest.mark.parametrize("G", [32, 128])
def test_e4m3_saturation_band_under_subnormal_scales(G):
    """fp32 blocks of m * 2^-149 whose absmax M * 2^-149 gives the scale 2^-149
    (M in (224, 672)) or 2^-148 (M in [672, 1120)): the quotients are m or m/2,
    up to 671, so everything above 448 saturates to +-448 (0x7E / 0xFE)."""
    rng = np.random.default_rng(5 + G)
    blocks = []
    for k in range(96):
        M = int(rng.integers(225, 1120))
        m = rng.integers(0, M + 1, G).astype(np.int64)
        m[rng.integers(0, G)] = M                                   # the absmax element
        sign = np.where(rng.random(G) < 0.5, -1, 1)
        blocks.append((sign * m).astype(np.float64) * 2.0 ** -149)
    # and a few with M = 224, where M/448 = 1/2 rounds to a zero scale (a zero block)
    blocks.append(np.full(G, 224 * 2.0 ** -149))
    x32 = np.concatenate(blocks).astype(np.float32)
    codes, scales = qcp.quantize_blockwise(to_gpu(x32), G, "e4m3")
    wc, ws = oracle.quantize_blockwise(x32, "f32", G, "e4m3")
    assert ((wc & 0x7F) == 0x7E).sum() > G, "the saturation band is exercised"
    assert ws[-1] == 0.0
    assert_same_bytes(to_host(scales), ws, f"subnormal scales G={G}")
    assert_same_bytes(to_host(codes), wc, f"saturating E4M3 codes G={G}")


def test_fp8_accumulate_from_zero_on_ties_and_neighbours():
    """Step 0 from the zero state quantizes the bf16 gradient itself: blocks of
    G = 128 whose absmax is 448 put every t on an E4M3 value, midpoint or
    neighbour; then a second step adds the same gradient again."""
    G = 128
    g32 = blocks_with_absmax_448(edge_targets("bf16"), G, 3)
    gh = cast_host(g32, "bf16")
    n = gh.size
    st_c, st_s = torch.zeros(n, dtype=torch.uint8, device="cuda"), torch.zeros(n // G, device="cuda")
    wc, ws = np.zeros(n, np.uint8), np.zeros(n // G, np.float32)
    gd = to_gpu(gh, "bf16")
    for step in range(2):
        qcp.fp8_accum_requant(st_c, st_s, gd, G)
        wc, ws = oracle.fp8_accum_requant(wc, ws, gh, "bf16", G)
        if step == 0:
            assert np.all(ws == 1.0)
        assert_same_bytes(to_host(st_s), ws, f"FP8 state scales after step {step}")
        assert_same_bytes(to_host(st_c), wc, f"FP8 state codes after step {step}")


def test_fp8_accumulate_with_subnormal_gradients():
    """bf16 gradients made of subnormals m * 2^-133: the block scale absmax/448
    is an fp32 subnormal with few significant bits, and the quotient of the
    absmax element lands just above 448 (the converter must saturate)."""
    G = 128
    rng = np.random.default_rng(17)
    m = rng.integers(-127, 128, 64 * G)
    m[::G] = np.where(rng.random(64) < 0.5, 127, -127)
    m[G * 7::G * 9] = rng.integers(1, 127, m[G * 7::G * 9].size)    # smaller absmax too
    bits = np.where(m < 0, 0x8000 | (-m), m).astype(np.uint16)      # bf16 subnormal patterns
    n = bits.size
    st_c, st_s = torch.zeros(n, dtype=torch.uint8, device="cuda"), torch.zeros(n // G, device="cuda")
    qcp.fp8_accum_requant(st_c, st_s, to_gpu(bits, "bf16"), G)
    wc, ws = oracle.fp8_accum_requant(np.zeros(n, np.uint8), np.zeros(n // G, np.float32), bits,
                                      "bf16", G)
    assert np.all(ws < 2.0 ** -126) and np.all(ws > 0)
    assert_same_bytes(to_host(st_s), ws, "FP8 state scales (subnormal)")
    assert_same_bytes(to_host(st_c), wc, "FP8 state codes (subnormal)")


def int_digits(q: np.ndarray, scales: np.ndarray, cmax: int) -> np.ndarray:
    """Codes c_j (|c_j| <= cmax) with sum_j c_j * scales[j] == q exactly, taken
    greedily from the largest scale down (each partial sum is q rounded to a
    multiple of that scale, so it is exact in fp32 when q is)."""
    r = q.astype(np.float64)
    out = []
    for s in scales:
        c = np.rint(r / s)
        assert np.all(np.abs(c) <= cmax)
        out.append(c.astype(np.int64))
        r = r - c * s
    assert np.all(r == 0), "targets not representable with these slice scales"
    return np.stack(out)


def pack_int_codes(c: np.ndarray, b: int) -> np.ndarray:
    """LSB-first b-bit two's-complement fields (the payload layout)."""
    f = (c & ((1 << b) - 1)).astype(np.uint64)
    bits = ((f[:, None] >> np.arange(b, dtype=np.uint64)) & 1).astype(np.uint8).reshape(-1)
    return np.packbits(bits, bitorder="little")


@pytest.mark.parametrize("fmt_in,G", [("int8", 32), ("int8", 128), ("int4", 128), ("int4", 512)])
def test_e4m3_reduce_output_on_ties_and_neighbours(fmt_in, G):
    """8 slices whose fmaf chain sums to exactly the targets, with 448 once per
    block so the output scale is 1: the E4M3 codes of the sums are those of the
    targets.  INT8 digits reach every E4M3 value, midpoint and fp32 neighbour;
    INT4 digits (and the 8-slice INT4 kernel it selects) reach the values and
    midpoints from 2^-10 up, and neighbours 2^-15 apart."""
    N = 8
    if fmt_in == "int8":
        sc = [2.0 ** (2 - 7 * j) for j in range(N)]          # 4, 2^-5, ..., 2^-47
        targets = edge_targets("f32")
        cmax = 127
    else:
        sc = [2.0 ** (6 - 3 * j) for j in range(N)]          # 64, 8, ..., 2^-15
        t = np.concatenate([e4m3_positive_values(), (np.concatenate([[0.0], e4m3_positive_values()[:-1]])
                                                     + e4m3_positive_values()) / 2])
        t = t[t >= 2.0 ** -10]
        t = np.concatenate([t + d * 2.0 ** -15 for d in range(-3, 4)])
        t = t[(t > 0) & (t <= 448)]
        targets = np.unique(t.astype(np.float32))
        targets = np.concatenate([targets, -targets, np.zeros(1, np.float32)])
        cmax = 7
    targets = np.tile(targets[np.abs(targets) <= 448], 3)     # several groups of blocks
    q = blocks_with_absmax_448(targets, G, 29 + G)
    L = q.size
    digits = int_digits(q, sc, cmax)                          # (N, L)
    b = 8 if fmt_in == "int8" else 4
    cs, ss = oracle.slice_layout(L, G, fmt_in)
    nb = oracle.n_blocks(L, G)
    codes = np.zeros(N * cs, np.uint8)
    scales = np.zeros(N * ss, np.float32)
    for j in range(N):
        codes[j * cs:j * cs + oracle.code_bytes(L, fmt_in)] = pack_int_codes(digits[j], b)
        scales[j * ss:j * ss + nb] = np.float32(sc[j])
    wc, ws, wsum = oracle.dequant_reduce_requant(codes, cs, scales, ss, N, L, G, fmt_in, "e4m3",
                                                 want_sum=True)
    assert np.array_equal(wsum[q != 0], q[q != 0]) and np.all(ws == 1.0)
    co, so = qcp.dequant_reduce_requant(to_gpu(codes), cs, to_gpu(scales), ss, N, L, G, fmt_in,
                                        "e4m3")
    assert_same_bytes(to_host(so), ws, f"reduce E4M3 scales {fmt_in} G={G}")
    assert_same_bytes(to_host(co), wc, f"reduce E4M3 codes {fmt_in} G={G}")
    co, so, su = qcp.dequant_reduce_requant(to_gpu(codes), cs, to_gpu(scales), ss, N, L, G, fmt_in,
                                            "e4m3", want_sum=True)
    assert_same_bytes(to_host(su), wsum, f"reduce fp32 sums {fmt_in} G={G}")
    assert_same_bytes(to_host(co), wc, f"reduce E4M3 codes (with sums) {fmt_in} G={G}")


def test_e4m3_reduce_output_with_subnormal_sums():
    """Sums k * 2^-149 (two INT8 slices with the subnormal scales 2^-142 and
    2^-149): the output scale is 2^-149 or 2^-148, and quotients above 448
    saturate."""
    G, N = 128, 2
    rng = np.random.default_rng(23)
    k = rng.integers(-1100, 1101, 48 * G)
    for blk in range(48):
        k[blk * G + int(rng.integers(0, G))] = int(rng.integers(225, 1100))
    c0 = np.rint(k / 128).astype(np.int64)
    c1 = k - 128 * c0
    L = k.size
    cs, ss = oracle.slice_layout(L, G, "int8")
    codes = np.zeros(N * cs, np.uint8)
    codes[:L] = c0.astype(np.int8).view(np.uint8)
    codes[cs:cs + L] = c1.astype(np.int8).view(np.uint8)
    scales = np.zeros(N * ss, np.float32)
    scales[:ss] = np.float32(2.0 ** -142)
    scales[ss:] = np.float32(2.0 ** -149)
    wc, ws, wsum = oracle.dequant_reduce_requant(codes, cs, scales, ss, N, L, G, "int8", "e4m3",
                                                 want_sum=True)
    assert np.array_equal(wsum.astype(np.float64), k * 2.0 ** -149)
    assert ((wc & 0x7F) == 0x7E).sum() > 48
    co, so = qcp.dequant_reduce_requant(to_gpu(codes), cs, to_gpu(scales), ss, N, L, G, "int8",
                                        "e4m3")
    assert_same_bytes(to_host(so), ws, "reduce E4M3 scales (subnormal sums)")
    assert_same_bytes(to_host(co), wc, "reduce E4M3 codes (subnormal sums)")


def scales_with_low_bits(rng, n, low_bits: int, pattern: int, emin: int, emax: int) -> np.ndarray:
    """fp32 scales whose low `low_bits` bits are `pattern`, random above them,
    with exponents in [emin, emax]."""
    e = rng.integers(emin, emax + 1, n)
    mant = rng.integers(0, 1 << 23, n).astype(np.uint32)
    mant = (mant & ~np.uint32((1 << low_bits) - 1)) | np.uint32(pattern)
    return (((e + 127).astype(np.uint32) << 23) | mant).view(np.float32)


@pytest.mark.parametrize("fmt", ["int8", "e4m3"])
@pytest.mark.parametrize("yt", ["bf16", "f16"])
def test_dequantize_products_on_output_ties(fmt, yt):
    """fl(c * s) on ties of the output type: for codes +-2^k the product is s
    itself scaled, so scales whose low bits are exactly half an output ulp
    (bf16: 0x8000 of 16 bits; fp16: 0x1000 of 13 bits), and 1..3 ulps either
    side, give ties and near-ties; fp16 also gets subnormal ties
    (2m+1) * 2^-25 and scales around the overflow threshold 65520."""
    G = 256
    rng = np.random.default_rng(41 if yt == "bf16" else 43)
    if fmt == "int8":
        block = np.concatenate([np.arange(-127, 128), [64]]).astype(np.int8).view(np.uint8)
        cmax = 127.0
    else:
        codes_all = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)   # no NaN
        block = np.concatenate([codes_all, codes_all[:2]])
        cmax = 448.0
    sc = []
    if yt == "bf16":
        for d in range(-3, 4):
            sc.append(scales_with_low_bits(rng, 16, 16, 0x8000 + d, -60, 60))
    else:
        top = int(np.floor(np.log2(65504 / cmax)))
        for d in range(-3, 4):
            sc.append(scales_with_low_bits(rng, 16, 13, 0x1000 + d, -14, top))
        sc.append(((2 * rng.integers(0, 1 << 9, 16) + 1) * 2.0 ** -25).astype(np.float32))
        edge = np.float32(65520.0 / (64 if fmt == "int8" else 256))
        sc.append(np.array([edge, np.nextafter(edge, np.float32(0)), np.nextafter(edge, np.float32(1e9)),
                            np.float32(65504.0 / (64 if fmt == "int8" else 256))], np.float32))
    sc = np.concatenate(sc).astype(np.float32)
    codes = np.tile(block, sc.size)
    for k in range(sc.size):                     # shuffle each block's codes
        codes[k * G:(k + 1) * G] = codes[k * G:(k + 1) * G][rng.permutation(G)]
    n = codes.size
    y = qcp.dequantize_blockwise(to_gpu(codes), to_gpu(sc), fmt, n, G,
                                 torch.bfloat16 if yt == "bf16" else torch.float16)
    want = oracle.dequantize_blockwise(codes, sc, fmt, n, G, yt)
    assert_same_bytes(to_host(y), want, f"dequantize {fmt} -> {yt} on output ties")
    if yt == "f16":
        assert ((want.view(np.uint16) & 0x7FFF) == 0x7C00).any(), "the overflow threshold is exercised"


def test_tiny_qwz_round_trip_exact_config():
    """1,048,576 fp16 values ~ N(0, 0.02) from seed 0, INT8 with G = 256 (4096
    scales), then dequantized to fp16: codes, scales and values byte for byte."""
    x = S.host_tiny_roundtrip()
    assert x.dtype == np.float16 and x.size == 1 << 20
    c, s = qcp.quantize_blockwise(to_gpu(x), 256, "int8")
    wc, ws = oracle.quantize_blockwise(x, "f16", 256, "int8")
    assert ws.size == 4096
    assert_same_bytes(to_host(c), wc, "qwZ tiny codes")
    assert_same_bytes(to_host(s), ws, "qwZ tiny scales")
    y = qcp.dequantize_blockwise(c, s, "int8", x.size, 256, torch.float16)
    assert_same_bytes(to_host(y), oracle.dequantize_blockwise(wc, ws, "int8", x.size, 256, "f16"),
                      "qwZ tiny round trip")
