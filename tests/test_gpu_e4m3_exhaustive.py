"""The E4M3 encoder on every input value it can meet at scale 1, byte for byte
against the CPU oracle, through the library's entry points.

A block whose absmax is exactly 448 has the scale 448/448 = 1, and the quotient
of each of its elements is the element itself, so such blocks put the gfx950
converter (after the exact quotient) on any chosen fp32 value.  Here the other
31 elements of each block of 32 run through every bit pattern of magnitude at
most 448 -- every float32 (2 x 1,138,753,537 values, zeros and subnormals
included), every bfloat16 and every float16 -- with both signs.  The encoding
rule is OCP E4M3FN, nearest value, ties to even mantissa, saturating at 448
with the sign of zero kept (AGoQ, Section 2.B, names FP8; E4M3 is the reading
taken for it).  The FP8 accumulate is checked the same way on every bfloat16
gradient value: from the zero state its first step quantizes the gradient
itself."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import quantized_collective_payloads_amd as qcp
from tests.gpu_util import assert_same_bytes, require_gpu, to_gpu, to_host

pytestmark = pytest.mark.gpu

G = 32
PER = G - 1                                  # swept values per block
MAX_BITS_448 = 0x43E00000                    # float32 bits of 448.0
N_PARTS = 8                                  # the fp32 sweep, in parts of ~285M values
CHUNK = 1 << 25                              # values per launch
THREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def blocks_of(vals32: np.ndarray) -> np.ndarray:
    """Blocks of G: 448 first, then PER of vals (zero-padded at the end)."""
    nb = -(-vals32.size // PER)
    padded = np.zeros(nb * PER, np.float32)
    padded[:vals32.size] = vals32
    out = np.empty((nb, G), np.float32)
    out[:, 0] = 448.0
    out[:, 1:] = padded.reshape(nb, PER)
    return out.reshape(-1)


def oracle_codes(x32: np.ndarray):
    """Oracle E4M3 codes and scales of x32 (whole blocks), on THREADS threads:
    the blocks are independent, so the result is the one-call result."""
    nb = x32.size // G
    cuts = [nb * t // THREADS * G for t in range(THREADS + 1)]
    parts = [x32[cuts[t]:cuts[t + 1]] for t in range(THREADS)]
    with ThreadPoolExecutor(THREADS) as ex:
        res = list(ex.map(lambda a: oracle.quantize_blockwise(a, "f32", G, "e4m3"), parts))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def check_fp32_patterns(lo: int, hi: int, sign: int):
    """Bit patterns lo .. hi-1 (magnitudes), with the sign bit `sign`."""
    for a in range(lo, hi, CHUNK):
        b = min(hi, a + CHUNK)
        vals = (np.arange(a, b, dtype=np.uint32) | np.uint32(sign << 31)).view(np.float32)
        x = blocks_of(vals)
        codes, scales = qcp.quantize_blockwise(to_gpu(x), G, "e4m3")
        wc, ws = oracle_codes(x)
        assert np.all(ws == 1.0)
        assert_same_bytes(to_host(scales), ws, f"scales, patterns {a:#x}..{b:#x} sign {sign}")
        assert_same_bytes(to_host(codes), wc, f"E4M3 codes, patterns {a:#x}..{b:#x} sign {sign}")


@pytest.mark.parametrize("part", range(N_PARTS))
def test_e4m3_encoder_every_fp32_up_to_448(part):
    total = MAX_BITS_448 + 1
    lo, hi = total * part // N_PARTS, total * (part + 1) // N_PARTS
    for sign in (0, 1):
        check_fp32_patterns(lo, hi, sign)


def every_16bit_value_up_to_448(dt: str) -> np.ndarray:
    """Every finite value of dt with magnitude <= 448, both signs, as float32."""
    p = np.arange(1 << 16, dtype=np.uint32)
    if dt == "bf16":
        v = (p << 16).view(np.float32)
    else:
        v = p.astype(np.uint16).view(np.float16).astype(np.float32)
    return v[np.isfinite(v) & (np.abs(v) <= 448.0)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_e4m3_encoder_every_16bit_value_up_to_448(dt):
    v = every_16bit_value_up_to_448(dt)
    x32 = blocks_of(v)
    if dt == "bf16":
        xh = (x32.view(np.uint32) >> 16).astype(np.uint16)
    else:
        xh = x32.astype(np.float16)
    codes, scales = qcp.quantize_blockwise(to_gpu(xh, dt), G, "e4m3")
    wc, ws = oracle.quantize_blockwise(xh, dt, G, "e4m3")
    assert np.all(ws == 1.0)
    assert_same_bytes(to_host(scales), ws, f"scales {dt}")
    assert_same_bytes(to_host(codes), wc, f"E4M3 codes of every {dt} value")
    assert (wc == 0x80).any() and (wc == 0xFE).any()


def test_fp8_accumulate_every_bf16_gradient_up_to_448():
    """Blocks of 128 with one gradient of magnitude 448: two accumulate steps
    from the zero state, the first of which encodes every bf16 value."""
    Ga = 128
    v = every_16bit_value_up_to_448("bf16")
    nb = -(-v.size // (Ga - 1))
    padded = np.zeros(nb * (Ga - 1), np.float32)
    padded[:v.size] = v
    g32 = np.empty((nb, Ga), np.float32)
    g32[:, 0] = -448.0
    g32[:, 1:] = padded.reshape(nb, Ga - 1)
    gh = (g32.reshape(-1).view(np.uint32) >> 16).astype(np.uint16)
    n = gh.size
    st_c = torch.zeros(n, dtype=torch.uint8, device="cuda")
    st_s = torch.zeros(n // Ga, dtype=torch.float32, device="cuda")
    wc, ws = np.zeros(n, np.uint8), np.zeros(n // Ga, np.float32)
    gd = to_gpu(gh, "bf16")
    for step in range(2):
        qcp.fp8_accum_requant(st_c, st_s, gd, Ga)
        wc, ws = oracle.fp8_accum_requant(wc, ws, gh, "bf16", Ga)
        if step == 0:
            assert np.all(ws == 1.0)
        assert_same_bytes(to_host(st_s), ws, f"FP8 state scales after step {step}")
        assert_same_bytes(to_host(st_c), wc, f"FP8 state codes after step {step}")
