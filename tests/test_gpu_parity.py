"""GPU parity: every kernel against the CPU oracle, byte for byte, on seeded
inputs at sizes the oracle finishes in seconds.  Sizes span many waves and
workgroups and include ragged tails (n not a multiple of 8 or of G), a single
element, short blocks, zero blocks and signed zeros."""
import numpy as np
import pytest
import torch

import oracle
import quantized_collective_payloads_amd as qcp
from tests.gpu_util import (DTS, FMTS, GS, TORCH_DT, assert_same_bytes, cast_host, require_gpu,
                            to_gpu, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def sizes_for(G):
    return [1, 7, G - 1, G, G + 9, 64 * G + 3, 300 * G + 8 * 5 + 1]


def sample_input(n, dt, seed, G):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * 0.02).astype(np.float32)
    if n > 4 * G:
        x[rng.random(n) < 0.001] = 0.4
        x[G:2 * G] = 0.0                 # a zero block
        x[2 * G + 3] = -0.0              # a signed zero inside a non-zero block
        x[3 * G:4 * G] *= np.float32(1e-3)
    return cast_host(x, dt)


@pytest.mark.parametrize("G", GS)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dt", DTS)
def test_quantize_matches_oracle(dt, fmt, G):
    for i, n in enumerate(sizes_for(G)):
        xh = sample_input(n, dt, 100 + i, G)
        codes, scales = qcp.quantize_blockwise(to_gpu(xh, dt), G, fmt)
        wc, ws = oracle.quantize_blockwise(xh, dt, G, fmt)
        assert_same_bytes(to_host(scales), ws, f"scales {dt} {fmt} G={G} n={n}")
        assert_same_bytes(to_host(codes), wc, f"codes {dt} {fmt} G={G} n={n}")


@pytest.mark.parametrize("G", GS)
@pytest.mark.parametrize("fmt", FMTS)
def test_dequantize_matches_oracle(fmt, G):
    for i, n in enumerate(sizes_for(G)):
        xh = sample_input(n, "f32", 200 + i, G)
        ch, sh = oracle.quantize_blockwise(xh, "f32", G, fmt)
        cd, sd = to_gpu(ch), to_gpu(sh)
        for yt in DTS:
            y = qcp.dequantize_blockwise(cd, sd, fmt, n, G, TORCH_DT[yt])
            assert_same_bytes(to_host(y), oracle.dequantize_blockwise(ch, sh, fmt, n, G, yt),
                              f"dequant {fmt} G={G} n={n} -> {yt}")


@pytest.mark.parametrize("b", [2, 4, 6, 8])
def test_pack_unpack_are_the_int_codecs(b):
    G = 128
    n = 50 * G + 5
    xh = sample_input(n, "bf16", 300 + b, G)
    x = to_gpu(xh, "bf16")
    p, s = qcp.pack_subbyte(x, b, G)
    c, s2 = qcp.quantize_blockwise(x, G, f"int{b}")
    assert torch.equal(p, c) and torch.equal(s, s2)
    wp, ws = oracle.pack_subbyte(xh, "bf16", b, G)
    assert_same_bytes(to_host(p), wp, "packed")
    y = qcp.unpack_subbyte(p, s, n, b, G, torch.bfloat16)
    assert_same_bytes(to_host(y), oracle.unpack_subbyte(wp, ws, n, b, G, "bf16"), "unpacked")


def make_slices(n_slices, L, G, fmt, seed, stride_pad=0):
    """N peer slices quantized by the oracle, laid out in one buffer."""
    rng = np.random.default_rng(seed)
    cb = oracle.code_bytes(L, fmt)
    stride = (cb + 15) // 16 * 16 + stride_pad
    nb = oracle.n_blocks(L, G)
    sstride = (nb + 3) // 4 * 4
    buf = np.zeros(stride * n_slices, np.uint8)
    sc = np.zeros(sstride * n_slices, np.float32)
    for j in range(n_slices):
        x = rng.laplace(0, 1e-3 * (1 + 0.3 * j), L).astype(np.float32).astype(np.float16)
        if L > 3 * G:
            x[G:2 * G] = 0                          # a block of zeros in every slice
        c, s = oracle.quantize_blockwise(x, "f16", G, fmt)
        buf[j * stride:j * stride + cb] = c
        sc[j * sstride:j * sstride + nb] = s
    return buf, stride, sc, sstride


def random_int4_slices(n_slices, L, G, seed):
    """N peer slices of uniformly random INT4 codes in [-7, 7] with random
    positive scales (a block of zeros with scale 0 in every slice): any codes
    and scales are valid reduce inputs, and this is far quicker to make at
    tens of millions of elements than quantizing data."""
    rng = np.random.default_rng(seed)
    cb = oracle.code_bytes(L, "int4")
    stride = (cb + 15) // 16 * 16
    nb = oracle.n_blocks(L, G)
    ss = (nb + 3) // 4 * 4
    buf = np.frombuffer(rng.bytes(n_slices * stride), np.uint8).reshape(n_slices, stride).copy()
    buf[(buf & 0x0F) == 0x08] &= 0xF0              # code -8 is outside [-7, 7]: make it 0
    buf[(buf & 0xF0) == 0x80] &= 0x0F
    buf[:, cb:] = 0
    if L % 2:
        buf[:, cb - 1] &= 0x0F                     # the last byte's high nibble is padding
    sc = (rng.uniform(0.5, 2.0, (n_slices, ss)) * (1e-3 / 7)).astype(np.float32)
    buf[:, G // 2:G] = 0                           # block 1 of every slice: zeros, scale 0
    sc[:, 1] = 0
    return buf.reshape(-1), stride, sc.reshape(-1), ss


REDUCE_CASES = [(fi, fo) for fi in FMTS for fo in FMTS]


@pytest.mark.parametrize("G", GS)
@pytest.mark.parametrize("fin,fout", REDUCE_CASES)
def test_reduce_matches_oracle(fin, fout, G):
    for N, L in [(1, G + 7), (3, 40 * G + 1), (8, 70 * G + 160)]:
        buf, stride, sc, ss = make_slices(N, L, G, fin, seed=G + N)
        co, so, su = qcp.dequant_reduce_requant(to_gpu(buf), stride, to_gpu(sc), ss, N, L, G,
                                                fin, fout, want_sum=True)
        wc, ws, wsum = oracle.dequant_reduce_requant(buf, stride, sc, ss, N, L, G, fin, fout,
                                                     want_sum=True)
        tag = f"{fin}->{fout} G={G} N={N} L={L}"
        assert_same_bytes(to_host(su), wsum, "sums " + tag)
        assert_same_bytes(to_host(so), ws, "scales " + tag)
        assert_same_bytes(to_host(co), wc, "codes " + tag)


def test_reduce_without_sum_and_with_padded_stride():
    G, N, L = 512, 8, 123 * 512 + 160
    buf, stride, sc, ss = make_slices(N, L, G, "int4", seed=9, stride_pad=48)
    co, so = qcp.dequant_reduce_requant(to_gpu(buf), stride, to_gpu(sc), ss, N, L, G, "int4", "int4")
    wc, ws = oracle.dequant_reduce_requant(buf, stride, sc, ss, N, L, G, "int4", "int4")
    assert_same_bytes(to_host(co), wc, "codes")
    assert_same_bytes(to_host(so), ws, "scales")


@pytest.mark.parametrize("G", GS)
@pytest.mark.parametrize("gt", DTS)
def test_fp8_accumulate_matches_oracle(gt, G):
    for n in (1, G + 5, 97 * G + 33):
        rng = np.random.default_rng(G + n)
        st_c = np.zeros(n, np.uint8)
        st_s = np.zeros(oracle.n_blocks(n, G), np.float32)
        dc, ds = to_gpu(st_c), to_gpu(st_s)
        for m in range(4):
            g = cast_host((rng.standard_normal(n) * 5e-4 * (1 + m)).astype(np.float32), gt)
            qcp.fp8_accum_requant(dc, ds, to_gpu(g, gt), G)
            st_c, st_s = oracle.fp8_accum_requant(st_c, st_s, g, gt, G)
            assert_same_bytes(to_host(ds), st_s, f"scales {gt} G={G} n={n} step {m}")
            assert_same_bytes(to_host(dc), st_c, f"codes {gt} G={G} n={n} step {m}")


def test_zero_length_is_a_noop():
    x = torch.zeros(0, dtype=torch.bfloat16, device="cuda")
    c, s = qcp.quantize_blockwise(x, 256, "int8")
    assert c.numel() == 0 and s.numel() == 0
    y = qcp.dequantize_blockwise(c, s, "int8", 0, 256)
    assert y.numel() == 0


def check_reduce(buf, stride, sc, ss, N, L, G, fin, fout, tag):
    co, so, su = qcp.dequant_reduce_requant(to_gpu(buf), stride, to_gpu(sc), ss, N, L, G,
                                            fin, fout, want_sum=True)
    wc, ws, wsum = oracle.dequant_reduce_requant(buf, stride, sc, ss, N, L, G, fin, fout,
                                                 want_sum=True)
    assert_same_bytes(to_host(su), wsum, "sums " + tag)
    assert_same_bytes(to_host(so), ws, "scales " + tag)
    assert_same_bytes(to_host(co), wc, "codes " + tag)


# INT4 input with exactly 8 slices and no fp32 sums runs its own kernel, one
# wave per group of 1024 elements (64 lanes x 16 codes), over many groups; the
# short last group takes the kernel's exact routine.  With fp32 sums, or
# another slice count, the general kernel runs.
@pytest.mark.parametrize("G,N,fout", [(512, 8, "int4"), (32, 8, "int8"), (128, 8, "e4m3"),
                                      (32, 5, "int8"), (256, 2, "e4m3")])
def test_reduce_int4x8_many_groups(G, N, fout):
    L = (2048 * 4096 * 2 if N == 8 else 2048 * 2048) + 2048 * 3 + G + 17
    buf, stride, sc, ss = random_int4_slices(N, L, G, seed=31 + N)
    tag = f"int4->{fout} G={G} N={N} L={L}"
    check_reduce(buf, stride, sc, ss, N, L, G, "int4", fout, tag)
    co, so = qcp.dequant_reduce_requant(to_gpu(buf), stride, to_gpu(sc), ss, N, L, G, "int4", fout)
    wc, ws = oracle.dequant_reduce_requant(buf, stride, sc, ss, N, L, G, "int4", fout)
    assert_same_bytes(to_host(so), ws, "scales without sums " + tag)
    assert_same_bytes(to_host(co), wc, "codes without sums " + tag)


# INT8 and E4M3 input with exactly 8 slices and no fp32 sums (the AGoQ local
# reduce), over many groups of blocks, with and without a ragged end.
@pytest.mark.parametrize("G", [32, 64, 128, 256])
@pytest.mark.parametrize("fout", FMTS)
@pytest.mark.parametrize("fin", ["int8", "e4m3"])
def test_reduce_eight_wide_slices(fin, fout, G):
    N = 8
    BPW = 64 // (G // 16)                              # blocks per wave
    for L in (2 * BPW * G * 37, 2 * BPW * G * 37 + 3 * G + 40):
        buf, stride, sc, ss = make_slices(N, L, G, fin, seed=300 + G)
        co, so = qcp.dequant_reduce_requant(to_gpu(buf), stride, to_gpu(sc), ss, N, L, G, fin, fout)
        wc, ws = oracle.dequant_reduce_requant(buf, stride, sc, ss, N, L, G, fin, fout)
        tag = f"{fin}->{fout} G={G} L={L}"
        assert_same_bytes(to_host(so), ws, "scales " + tag)
        assert_same_bytes(to_host(co), wc, "codes " + tag)


@pytest.mark.parametrize("fin", ["int4", "int8", "e4m3"])
def test_reduce_more_than_eight_slices(fin):
    G, N, L = 128, 12, 600 * 128 + 77
    buf, stride, sc, ss = make_slices(N, L, G, fin, seed=77)
    check_reduce(buf, stride, sc, ss, N, L, G, fin, "int4", f"{fin}->int4 N={N}")


@pytest.mark.parametrize("N", [2, 7, 9, 16, 17, 63, 64])
@pytest.mark.parametrize("fin", FMTS)
def test_reduce_slice_counts_up_to_the_limit(fin, N):
    """Slice counts around the general kernel's batches of 8 loads, up to the
    64 slices the entry point accepts, with and without the fp32 sums (INT4 at
    8 slices without sums is the 8-slice INT4 kernel's case, tested apart)."""
    G = 256
    L = 30 * G + 100
    buf, stride, sc, ss = make_slices(N, L, G, fin, seed=500 + N)
    fout = "e4m3" if fin == "int6" else "int4"
    check_reduce(buf, stride, sc, ss, N, L, G, fin, fout, f"{fin}->{fout} N={N}")
    co, so = qcp.dequant_reduce_requant(to_gpu(buf), stride, to_gpu(sc), ss, N, L, G, fin, fout)
    wc, ws = oracle.dequant_reduce_requant(buf, stride, sc, ss, N, L, G, fin, fout)
    assert_same_bytes(to_host(so), ws, f"scales without sums {fin} N={N}")
    assert_same_bytes(to_host(co), wc, f"codes without sums {fin} N={N}")


@pytest.mark.parametrize("fin,fout", [("int4", "int4"), ("int4", "e4m3"), ("int8", "int8"),
                                      ("e4m3", "int6"), ("int2", "e4m3")])
def test_reduce_extreme_scales(fin, fout):
    """Scales outside the range the fast quotient covers: huge (code*scale needs
    the exact product path for INT4), tiny normal and subnormal; sums stay finite."""
    G, N = 64, 8
    L = 2048 * 40 + 5
    buf, stride, sc, ss = make_slices(N, L, G, fin, seed=5)
    nb = oracle.n_blocks(L, G)
    sc = sc.copy()
    # largest code times the huge scale stays below the float32 maximum
    big = np.float32(2.0 ** {"int2": 124, "int4": 124, "int8": 120, "e4m3": 118}[fin])
    for k in range(0, nb, 97):                 # one slice huge, the rest ordinary
        sc[k] = big
    for k in range(13, nb, 89):                # every slice tiny normal
        sc[np.arange(N) * ss + k] = np.float32(2.0 ** -100)
    for k in range(29, nb, 71):                # every slice subnormal
        sc[np.arange(N) * ss + k] = np.float32(3e-42)
    for k in range(41, nb, 113):               # mixed subnormal and normal
        sc[k] = np.float32(1e-44)
    check_reduce(buf, stride, sc, ss, N, L, G, fin, fout, f"{fin}->{fout} extreme scales")


# (nodes, GPUs per node, chunk length C, G): chunks that blocks straddle,
# chunks shorter than a block, and, in the last two, chunks shorter than the
# distance between one lane's vectors in a full block (64 elements at G = 256,
# 256 at G = 1024), so that a lane's vectors come from several chunks
REORDER_CASES = [(2, 4, 1000, 256), (3, 8, 40 * 64 + 24, 64), (4, 8, 8, 32), (1, 3, 5 * 128, 128),
                 (2, 2, 65536 + 8, 1024), (5, 1, 336, 512), (16, 2, 40, 256), (12, 2, 200, 1024)]


@pytest.mark.parametrize("K,N,C,G", REORDER_CASES)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dt", DTS)
def test_reorder_quantize_matches_oracle(dt, fmt, K, N, C, G):
    n = K * N * C
    xh = sample_input(n, dt, 500 + K * N + C % 97, G)
    codes, cs, scales, ss = qcp.reorder_quantize(to_gpu(xh, dt), K, N, G, fmt)
    wc, wcs, ws, wss = oracle.reorder_quantize(xh, dt, K, N, G, fmt)
    L = n // N
    cb, nb = oracle.code_bytes(L, fmt), oracle.n_blocks(L, G)
    assert cs >= cb and cs % 16 == 0 and ss >= nb and ss % 4 == 0
    ch, sh = to_host(codes), to_host(scales)
    for j in range(N):      # each side's own slice strides
        tag = f"{dt} {fmt} K={K} N={N} C={C} G={G} slice {j}"
        assert_same_bytes(sh[j * ss:j * ss + nb], ws[j * wss:j * wss + nb], "scales " + tag)
        assert_same_bytes(ch[j * cs:j * cs + cb], wc[j * wcs:j * wcs + cb], "codes " + tag)


def test_reorder_then_reduce_is_the_intra_node_hop():
    """N virtual GPUs of one node each reorder+quantize their bucket; the slices
    GPU j receives, reduced by dequant_reduce_requant, equal the oracle's."""
    K, N, C, G = 2, 4, 3 * 512 + 64, 512
    n = K * N * C
    rng = np.random.default_rng(77)
    sent = []
    for i in range(N):
        x = rng.laplace(0, 1e-3, n).astype(np.float32).astype(np.float16)
        sent.append((x, qcp.reorder_quantize(to_gpu(x), K, N, G, "int4")))
    L = n // N
    for j in range(N):
        cs, ss = sent[0][1][1], sent[0][1][3]
        buf = torch.stack([c[j * cs:(j + 1) * cs] for _, (c, _, _, _) in sent]).reshape(-1)
        sca = torch.stack([s[j * ss:(j + 1) * ss] for _, (_, _, s, _) in sent]).reshape(-1)
        co, so = qcp.dequant_reduce_requant(buf, cs, sca, ss, N, L, G, "int4", "int4")
        host = [oracle.reorder_quantize(x, "f16", K, N, G, "int4") for x, _ in sent]
        wcs, wss = host[0][1], host[0][3]
        hb = np.concatenate([h[0][j * wcs:(j + 1) * wcs] for h in host])
        hs = np.concatenate([h[2][j * wss:(j + 1) * wss] for h in host])
        wc, ws = oracle.dequant_reduce_requant(hb, wcs, hs, wss, N, L, G, "int4", "int4")
        assert_same_bytes(to_host(co), wc, f"hop-1 codes on GPU {j}")
        assert_same_bytes(to_host(so), ws, f"hop-1 scales on GPU {j}")


@pytest.mark.parametrize("G", GS)
@pytest.mark.parametrize("b", [2, 4, 6, 8])
def test_records_match_oracle(b, G):
    for i, n in enumerate(sizes_for(G)):
        for dt in DTS:
            xh = sample_input(n, dt, 700 + i + b, G)
            rec = qcp.pack_subbyte_records(to_gpu(xh, dt), b, G)
            want = oracle.pack_records(xh, dt, b, G)
            assert_same_bytes(to_host(rec), want, f"records {dt} b={b} G={G} n={n}")
        for yt in DTS:
            y = qcp.unpack_subbyte_records(to_gpu(want), n, b, G, TORCH_DT[yt])
            assert_same_bytes(to_host(y), oracle.unpack_records(want, n, b, G, yt),
                              f"unpacked records b={b} G={G} n={n} -> {yt}")
