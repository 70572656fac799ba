"""Seeded random sweep over every entry point against the oracle, byte for byte.

Each case draws its own sizes (ragged, up to about a million elements), block
size, formats, dtypes and value scale from one seed, so the sweep reaches
combinations the hand-picked parity cases do not (odd sizes with every G,
tiny and huge value scales, slice counts 1..12, padded strides).  Inputs are
built here with numpy; expected values come from the oracle."""
import numpy as np
import pytest
import torch

import oracle
import quantized_collective_payloads_amd as qcp
from tests.gpu_util import (DTS, FMTS, GS, TORCH_DT, assert_same_bytes, cast_host, require_gpu,
                            to_gpu, to_host)

pytestmark = pytest.mark.gpu

N_CASES = 100


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def draw_values(rng, n, dt="f32"):
    """float32 values of a random magnitude (1e-30 .. 1e4; at most 1e2 for fp16,
    so that the outliers stay finite there), some zeros and a few outliers."""
    scale = 10.0 ** rng.uniform(-30, 2 if dt == "f16" else 4)
    x = (rng.standard_normal(n) * scale).astype(np.float32)
    if n > 64:
        z = rng.integers(0, n - 32)
        x[z:z + 32] = 0.0
        x[rng.random(n) < 1e-3] *= np.float32(50.0)
    return x


def draw_size(rng, G):
    return int(rng.choice([rng.integers(1, 4 * G), rng.integers(1, 2000) * G + rng.integers(0, G),
                           rng.integers(1, 1 << 20)]))


@pytest.mark.parametrize("case", range(N_CASES))
def test_codec_random(case):
    rng = np.random.default_rng(7000 + case)
    G = int(rng.choice(GS))
    fmt = str(rng.choice(FMTS))
    dt = str(rng.choice(DTS))
    n = draw_size(rng, G)
    xh = cast_host(draw_values(rng, n, dt), dt)
    tag = f"case {case}: {dt} {fmt} G={G} n={n}"
    codes, scales = qcp.quantize_blockwise(to_gpu(xh, dt), G, fmt)
    wc, ws = oracle.quantize_blockwise(xh, dt, G, fmt)
    assert_same_bytes(to_host(scales), ws, "scales " + tag)
    assert_same_bytes(to_host(codes), wc, "codes " + tag)
    yt = str(rng.choice(DTS))
    y = qcp.dequantize_blockwise(codes, scales, fmt, n, G, TORCH_DT[yt])
    assert_same_bytes(to_host(y), oracle.dequantize_blockwise(wc, ws, fmt, n, G, yt),
                      f"dequant -> {yt} " + tag)


@pytest.mark.parametrize("case", range(N_CASES))
def test_subbyte_random(case):
    rng = np.random.default_rng(8000 + case)
    G = int(rng.choice(GS))
    b = int(rng.choice([2, 4, 6, 8]))
    n = draw_size(rng, G)
    xh = cast_host(draw_values(rng, n), "bf16")
    tag = f"case {case}: b={b} G={G} n={n}"
    pk, ps = qcp.pack_subbyte(to_gpu(xh, "bf16"), b, G)
    wp, ws = oracle.pack_subbyte(xh, "bf16", b, G)
    assert_same_bytes(to_host(ps), ws, "scales " + tag)
    assert_same_bytes(to_host(pk), wp, "packed " + tag)
    y = qcp.unpack_subbyte(pk, ps, n, b, G, torch.bfloat16)
    assert_same_bytes(to_host(y), oracle.unpack_subbyte(wp, ws, n, b, G, "bf16"), "unpacked " + tag)
    rec = qcp.pack_subbyte_records(to_gpu(xh, "bf16"), b, G)
    assert_same_bytes(to_host(rec), oracle.pack_records(xh, "bf16", b, G), "records " + tag)


@pytest.mark.parametrize("case", range(N_CASES))
def test_reduce_random(case):
    rng = np.random.default_rng(9000 + case)
    G = int(rng.choice(GS))
    fin, fout = str(rng.choice(FMTS)), str(rng.choice(FMTS))
    N = int(rng.integers(1, 13))
    L = min(draw_size(rng, G), 200_000)
    cb = oracle.code_bytes(L, fin)
    stride = (cb + 15) // 16 * 16 + 16 * int(rng.integers(0, 3))
    nb = oracle.n_blocks(L, G)
    ss = (nb + 3) // 4 * 4 + 4 * int(rng.integers(0, 3))
    buf = np.zeros(N * stride, np.uint8)
    sc = np.zeros(N * ss, np.float32)
    for j in range(N):
        c, s = oracle.quantize_blockwise(draw_values(rng, L), "f32", G, fin)
        buf[j * stride:j * stride + cb] = c
        sc[j * ss:j * ss + nb] = s
    want_sum = bool(rng.integers(0, 2))
    tag = f"case {case}: {fin}->{fout} G={G} N={N} L={L} sums={want_sum}"
    out = qcp.dequant_reduce_requant(to_gpu(buf), stride, to_gpu(sc), ss, N, L, G, fin, fout,
                                     want_sum=want_sum)
    want = oracle.dequant_reduce_requant(buf, stride, sc, ss, N, L, G, fin, fout, want_sum=want_sum)
    assert_same_bytes(to_host(out[1]), want[1], "scales " + tag)
    assert_same_bytes(to_host(out[0]), want[0], "codes " + tag)
    if want_sum:
        assert_same_bytes(to_host(out[2]), want[2], "sums " + tag)


@pytest.mark.parametrize("case", range(N_CASES // 2))
def test_fp8_accumulate_random(case):
    rng = np.random.default_rng(9500 + case)
    G = int(rng.choice(GS))
    gt = str(rng.choice(DTS))
    n = draw_size(rng, G)
    sc_dev = torch.zeros(oracle.n_blocks(n, G), dtype=torch.float32, device="cuda")
    st_dev = torch.zeros(n, dtype=torch.uint8, device="cuda")
    oc, os_ = np.zeros(n, np.uint8), np.zeros(oracle.n_blocks(n, G), np.float32)
    for step in range(int(rng.integers(1, 5))):
        gh = cast_host(draw_values(rng, n, gt), gt)
        qcp.fp8_accum_requant(st_dev, sc_dev, to_gpu(gh, gt), G)
        oc, os_ = oracle.fp8_accum_requant(oc, os_, gh, gt, G)
        tag = f"case {case}: {gt} G={G} n={n} step {step}"
        assert_same_bytes(to_host(sc_dev), os_, "state scales " + tag)
        assert_same_bytes(to_host(st_dev), oc, "state codes " + tag)
