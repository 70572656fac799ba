"""GPU parity past 32-bit offsets: tensors of more than 2^31 elements, and
reduce slices whose byte offsets pass 2^31.

Every index in the kernels is 64-bit; these tests check it where a 32-bit
index would wrap.  As in the full-size tests, the GPU runs on the whole
tensor and the oracle on sampled blocks: the blocks around element 2^31, a
random sample, and the short last block."""
import numpy as np
import pytest
import torch

import oracle
import qcp_synthetic as S
import quantized_collective_payloads_amd as qcp
from tests.gpu_util import assert_same_bytes, require_gpu, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

BIG = (1 << 31) + 3 * (1 << 20) + 37        # not a multiple of 8 or of G


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


def log(msg):
    print(msg, flush=True)


def blocks_to_check(full, G, seed):
    """Full blocks around element 2^31, a random sample and the last full block."""
    k31 = (1 << 31) // G
    rng = np.random.default_rng(seed)
    ks = np.concatenate([np.arange(k31 - 3, k31 + 3), rng.choice(full, 200, replace=False), [0, full - 1]])
    return np.unique(ks[(ks >= 0) & (ks < full)]).astype(np.int64)


def gather_blocks(t, G, ks):
    idx = torch.from_numpy(ks).to(t.device)
    return t[: (t.numel() // G) * G].view(-1, G).index_select(0, idx).reshape(-1)


def test_quantize_dequantize_past_2_31_elements():
    G, fmt = 64, "int4"
    x = S.device_normal(BIG, 0.02, S.seed_for(9, 1), torch.bfloat16)
    codes, scales = qcp.quantize_blockwise(x, G, fmt)
    y = qcp.dequantize_blockwise(codes, scales, fmt, BIG, G, torch.bfloat16)
    torch.cuda.synchronize()
    log(f"quantize/dequantize n={BIG}: GPU done")
    full = BIG // G
    ks = blocks_to_check(full, G, 91)
    xh = to_host(gather_blocks(x, G, ks))
    wc, ws = oracle.quantize_blockwise(xh, "bf16", G, fmt)
    got_c = codes[: full * G // 2].view(full, G // 2).index_select(0, torch.from_numpy(ks).cuda())
    assert_same_bytes(got_c.reshape(-1).cpu().numpy(), wc, "codes (sampled blocks)")
    assert_same_bytes(scales.cpu().numpy()[ks], ws, "scales (sampled blocks)")
    wy = oracle.dequantize_blockwise(wc, ws, fmt, ks.size * G, G, "bf16")
    assert_same_bytes(to_host(gather_blocks(y, G, ks)), wy, "dequantized (sampled blocks)")
    # the short last block (37 elements)
    tail = BIG - full * G
    xt = to_host(x[full * G:])
    tc, tsc = oracle.quantize_blockwise(xt, "bf16", G, fmt)
    assert_same_bytes(codes[full * G // 2:].cpu().numpy(), tc, "codes (short last block)")
    assert_same_bytes(scales[full:].cpu().numpy(), tsc, "scale (short last block)")
    assert_same_bytes(to_host(y[full * G:]), oracle.dequantize_blockwise(tc, tsc, fmt, tail, G, "bf16"),
                      "dequantized (short last block)")


def test_fp8_accumulate_past_2_31_elements():
    G = 128
    g = S.device_normal(BIG, 5e-4, S.seed_for(9, 2), torch.bfloat16)
    st_c = torch.zeros(BIG, dtype=torch.uint8, device="cuda")
    st_s = torch.zeros(oracle.n_blocks(BIG, G), dtype=torch.float32, device="cuda")
    qcp.fp8_accum_requant(st_c, st_s, g, G)
    qcp.fp8_accum_requant(st_c, st_s, g, G)
    torch.cuda.synchronize()
    log(f"FP8 accumulate n={BIG}: GPU done")
    full = BIG // G
    ks = blocks_to_check(full, G, 92)
    gh = to_host(gather_blocks(g, G, ks))
    oc = np.zeros(ks.size * G, np.uint8)
    os_ = np.zeros(ks.size, np.float32)
    for _ in range(2):
        oc, os_ = oracle.fp8_accum_requant(oc, os_, gh, "bf16", G)
    got = st_c[: full * G].view(full, G).index_select(0, torch.from_numpy(ks).cuda())
    assert_same_bytes(got.reshape(-1).cpu().numpy(), oc, "state codes (sampled blocks)")
    assert_same_bytes(st_s.cpu().numpy()[ks], os_, "state scales (sampled blocks)")
    tail = BIG - full * G
    gt = to_host(g[full * G:])
    tc, ts = np.zeros(tail, np.uint8), np.zeros(1, np.float32)
    for _ in range(2):
        tc, ts = oracle.fp8_accum_requant(tc, ts, gt, "bf16", G)
    assert_same_bytes(st_c[full * G:].cpu().numpy(), tc, "state codes (short last block)")
    assert_same_bytes(st_s[full:].cpu().numpy(), ts, "state scale (short last block)")


def test_reduce_slices_past_2_31_bytes():
    """8 INT4 slices of 6.4e8 + 160 codes (320 MB each): the seventh crosses
    byte 2^31 of the buffer and the eighth starts past it.  Run without fp32
    sums (the 8-slice INT4 kernel) and with them (the general one)."""
    N, G = 8, 512
    L = 640_000_000 + 160
    cb = oracle.code_bytes(L, "int4")
    stride = (cb + 15) // 16 * 16
    nb = oracle.n_blocks(L, G)
    ss = (nb + 3) // 4 * 4
    assert 6 * stride < (1 << 31) < 7 * stride
    gen = torch.Generator(device="cuda")
    gen.manual_seed(S.seed_for(9, 3))
    nib = torch.randint(-7, 8, (N, 2 * stride), generator=gen, device="cuda", dtype=torch.int16)
    nib = (nib & 0xF).to(torch.uint8)
    buf = nib[:, 0::2] | (nib[:, 1::2] << 4)
    del nib
    buf[:, cb:] = 0
    sc = (torch.rand((N, ss), generator=gen, device="cuda") * 1.5 + 0.5) * (1e-3 / 7)
    buf, sc = buf.reshape(-1).contiguous(), sc.reshape(-1).contiguous()
    co, so = qcp.dequant_reduce_requant(buf, stride, sc, ss, N, L, G, "int4", "int4")
    co2, so2, su = qcp.dequant_reduce_requant(buf, stride, sc, ss, N, L, G, "int4", "int4",
                                              want_sum=True)
    torch.cuda.synchronize()
    log(f"reduce 8 x {L} INT4: GPU done")
    assert torch.equal(co, co2) and torch.equal(so.view(torch.int32), so2.view(torch.int32))
    full = L // G
    bpb = G // 2
    rng = np.random.default_rng(93)
    ks = np.unique(np.concatenate([rng.choice(full, 200, replace=False), [0, full - 1]])).astype(np.int64)
    kd = torch.from_numpy(ks).cuda()
    bufv = buf.view(N, stride)
    mini = torch.stack([bufv[j, : full * bpb].view(full, bpb).index_select(0, kd).reshape(-1)
                        for j in range(N)]).cpu().numpy()
    msc = sc.view(N, ss)[:, :full].index_select(1, kd).cpu().numpy()
    wc, ws, wsum = oracle.dequant_reduce_requant(mini.reshape(-1), mini.shape[1], msc.reshape(-1),
                                                 msc.shape[1], N, ks.size * G, G, "int4", "int4",
                                                 want_sum=True)
    got_c = co[: full * bpb].view(full, bpb).index_select(0, kd).reshape(-1).cpu().numpy()
    assert_same_bytes(got_c, wc, "codes (sampled blocks)")
    assert_same_bytes(so.cpu().numpy()[ks], ws, "scales (sampled blocks)")
    got_s = su[: full * G].view(full, G).index_select(0, kd).reshape(-1).cpu().numpy()
    assert_same_bytes(got_s, wsum, "fp32 sums (sampled blocks)")
    # the short last block (160 elements)
    tb = cb - full * bpb
    mt = bufv[:, full * bpb: cb].cpu().numpy()
    mts = sc.view(N, ss)[:, full].cpu().numpy()
    wc, ws = oracle.dequant_reduce_requant(mt.reshape(-1), tb, mts, 1, N, L - full * G, G, "int4", "int4")
    assert_same_bytes(co[full * bpb:].cpu().numpy(), wc, "codes (short last block)")
    assert_same_bytes(so[full:].cpu().numpy(), ws, "scale (short last block)")


def test_reorder_quantize_slices_past_2_31_elements():
    """The qgZ sender with 2 nodes x 2 GPUs on 2^32 + 2^21 + 64 fp16 elements:
    each slice holds 2^31 + 2^20 + 32 elements (chunks of 2^30 + 2^19 + 16), so
    slice offsets, chunk indices and source indices all pass 2^31."""
    K, N, G, fmt = 2, 2, 512, "int4"
    n = (1 << 32) + (1 << 21) + 64
    L, C = n // N, n // (K * N)
    assert L > (1 << 31) and C % 8 == 0
    x = S.device_normal(n, 1e-3, S.seed_for(9, 4), torch.float16)
    codes, cs, scales, ss = qcp.reorder_quantize(x, K, N, G, fmt)
    torch.cuda.synchronize()
    log(f"reorder_quantize n={n}: GPU done")
    full = L // G
    for j in range(N):
        ks = blocks_to_check(full, G, 94 + j)
        e = (ks[:, None] * G + np.arange(G)[None, :]).reshape(-1)        # elements of slice j
        src = (e // C * N + j) * C + e % C                               # where they live in x
        xh = to_host(x[torch.from_numpy(src).cuda()]).view(np.float16)
        wc, ws = oracle.quantize_blockwise(xh, "f16", G, fmt)
        got = codes[j * cs:j * cs + full * G // 2].view(full, G // 2).index_select(0, torch.from_numpy(ks).cuda())
        assert_same_bytes(got.reshape(-1).cpu().numpy(), wc, f"codes, slice {j} (sampled blocks)")
        assert_same_bytes(scales[j * ss:j * ss + full].cpu().numpy()[ks], ws, f"scales, slice {j} (sampled blocks)")
        # the short last block (32 elements)
        et = np.arange(full * G, L)
        xt = to_host(x[torch.from_numpy((et // C * N + j) * C + et % C).cuda()]).view(np.float16)
        tc, tsc = oracle.quantize_blockwise(xt, "f16", G, fmt)
        nbytes = oracle.code_bytes(L, fmt)
        assert_same_bytes(codes[j * cs + full * G // 2:j * cs + nbytes].cpu().numpy(), tc,
                          f"codes, slice {j} (short last block)")
        assert_same_bytes(scales[j * ss + full:j * ss + full + 1].cpu().numpy(), tsc,
                          f"scale, slice {j} (short last block)")
