"""GPU parity at the benchmark's full sizes, with the same calls bench.py times.

The oracle is far too slow for whole tensors of hundreds of millions of
elements, but every output block depends only on the same block of the inputs
(and, for the reduce, on that block of each slice).  So each test runs the
GPU on the full tensor and the oracle on a random sample of blocks (plus the
first and the last), gathered into a small tensor, and compares those blocks
byte for byte.  Properties that hold at any size (code ranges, finite
non-negative scales) are checked on the whole GPU output.

Inputs come from qcp_synthetic's device generators; the qgZ slices are then
quantized by the oracle on the host, so no oracle input ever comes from the HIP
path."""
import numpy as np
import pytest
import torch

import oracle
import qcp_synthetic as S
import quantized_collective_payloads_amd as qcp
from tests.gpu_util import assert_same_bytes, require_gpu, to_gpu, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

SAMPLE = 1500


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


def sample_blocks(nb, seed):
    rng = np.random.default_rng(seed)
    ks = rng.choice(nb, size=min(SAMPLE, nb), replace=False)
    return np.unique(np.concatenate([ks, [0, nb - 1]])).astype(np.int64)


def host_blocks(t, G, ks):
    """Blocks ks (all full) of a 1-D 16-bit device tensor, as host data."""
    idx = torch.from_numpy(ks).to(t.device)
    return to_host(t[: (t.numel() // G) * G].view(-1, G).index_select(0, idx).reshape(-1))


def byte_blocks(t, nbytes, ks):
    idx = torch.from_numpy(ks).to(t.device)
    return t[: (t.numel() // nbytes) * nbytes].view(-1, nbytes).index_select(0, idx).reshape(-1).cpu().numpy()


def check_scales(s):
    assert torch.isfinite(s).all() and (s >= 0).all()


def log(msg):
    print(msg, flush=True)


def test_qwz_llama8b_layer_fullsize():
    G = 256
    x = S.device_llama8b_layer("cuda")
    n = x.numel()
    nb = n // G
    codes, scales = qcp.quantize_blockwise(x, G, "int8")
    y = qcp.dequantize_blockwise(codes, scales, "int8", n, G, torch.bfloat16)
    torch.cuda.synchronize()
    log(f"qwZ n={n}: GPU done")
    check_scales(scales)
    assert not (codes == 0x80).any()                       # INT8 codes stay in [-127, 127]
    ks = sample_blocks(nb, 21)
    xh = host_blocks(x, G, ks)
    wc, ws = oracle.quantize_blockwise(xh, "bf16", G, "int8")
    assert_same_bytes(byte_blocks(codes, G, ks), wc, "qwZ codes (sampled blocks)")
    assert_same_bytes(scales.cpu().numpy()[ks], ws, "qwZ scales (sampled blocks)")
    wy = oracle.dequantize_blockwise(wc, ws, "int8", ks.size * G, G, "bf16")
    assert_same_bytes(host_blocks(y, G, ks), wy, "qwZ dequantized (sampled blocks)")


@pytest.mark.parametrize("bits,G", S.AQUAVIT_SWEEP)
def test_aquavit_mlp70b_fullsize(bits, G):
    w = S.device_mlp70b(device="cuda")
    n = w.numel()
    nb = n // G
    pk, ps = qcp.pack_subbyte(w, bits, G)
    y = qcp.unpack_subbyte(pk, ps, n, bits, G, torch.bfloat16)
    torch.cuda.synchronize()
    log(f"Aquavit b={bits} G={G}: GPU done")
    check_scales(ps)
    assert pk.numel() * 8 + ps.numel() * 32 == n * bits + nb * 32          # bpw = b + 32/G
    ks = sample_blocks(nb, 40 + bits * G)
    xh = host_blocks(w, G, ks)
    wp, ws = oracle.pack_subbyte(xh, "bf16", bits, G)
    assert_same_bytes(byte_blocks(pk, G * bits // 8, ks), wp, f"packed b={bits} G={G}")
    assert_same_bytes(ps.cpu().numpy()[ks], ws, f"scales b={bits} G={G}")
    wy = oracle.unpack_subbyte(wp, ws, ks.size * G, bits, G, "bf16")
    assert_same_bytes(host_blocks(y, G, ks), wy, f"unpacked b={bits} G={G}")
    # the interleaved-metadata layout: record k = [scale k][codes of block k]
    rec = qcp.pack_subbyte_records(w, bits, G).view(nb, 4 + G * bits // 8)
    assert torch.equal(rec[:, :4], ps.view(torch.uint8).view(nb, 4))
    assert torch.equal(rec[:, 4:], pk.view(nb, G * bits // 8))
    y2 = qcp.unpack_subbyte_records(rec.view(-1), n, bits, G, torch.bfloat16)
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16))


def test_qgz_reduce_fullsize():
    N, L, G = S.QGZ_SLICES, S.QGZ_SLICE_LEN, 512
    cb = oracle.code_bytes(L, "int4")
    stride = (cb + 15) // 16 * 16
    nb = oracle.n_blocks(L, G)
    sstride = (nb + 3) // 4 * 4
    buf = np.zeros(N * stride, np.uint8)
    sc = np.zeros(N * sstride, np.float32)
    for j, gd in enumerate(S.device_qgz_slices_fp16(L, N, "cuda")):
        g = to_host(gd).view(np.float16)
        del gd
        c, s = oracle.quantize_blockwise(g, "f16", G, "int4")
        buf[j * stride:j * stride + cb] = c
        sc[j * sstride:j * sstride + nb] = s
        log(f"qgZ slice {j} quantized by the oracle")
    co, so = qcp.dequant_reduce_requant(to_gpu(buf), stride, to_gpu(sc), sstride, N, L, G,
                                        "int4", "int4")
    torch.cuda.synchronize()
    log("qgZ: GPU done")
    check_scales(so)
    nib = torch.stack([co & 0x0F, co >> 4])
    assert not (nib == 8).any()                            # INT4 codes stay in [-7, 7]
    co_h, so_h = co.cpu().numpy(), so.cpu().numpy()
    bpb = G // 2                                           # bytes per full block
    full = L // G
    ks = sample_blocks(full, 3)
    # sampled full blocks: each slice's block k, side by side, as an N-slice problem
    mini = np.stack([buf[j * stride:j * stride + full * bpb].reshape(full, bpb)[ks].reshape(-1)
                     for j in range(N)])
    msc = np.stack([sc[j * sstride:j * sstride + full][ks] for j in range(N)])
    wc, ws = oracle.dequant_reduce_requant(mini.reshape(-1), mini.shape[1], msc.reshape(-1),
                                           msc.shape[1], N, ks.size * G, G, "int4", "int4")
    assert_same_bytes(co_h[:full * bpb].reshape(full, bpb)[ks].reshape(-1), wc, "qgZ codes (sampled)")
    assert_same_bytes(so_h[ks], ws, "qgZ scales (sampled)")
    # the short last block (160 elements)
    tail = L - full * G
    tb = oracle.code_bytes(tail, "int4")
    mini = np.stack([buf[j * stride + full * bpb:j * stride + full * bpb + tb] for j in range(N)])
    msc = np.array([sc[j * sstride + full] for j in range(N)], np.float32)
    wc, ws = oracle.dequant_reduce_requant(mini.reshape(-1), tb, msc, 1, N, tail, G, "int4", "int4")
    assert_same_bytes(co_h[full * bpb:], wc, "qgZ codes (short last block)")
    assert_same_bytes(so_h[full:], ws, "qgZ scale (short last block)")


def test_agoq_accumulate_and_reduce_fullsize():
    G, Ns = 128, 8
    grads = S.device_agoq_grads(device="cuda")
    n = grads[0].numel()
    st_c = torch.zeros(n, dtype=torch.uint8, device="cuda")
    st_s = torch.zeros(n // G, dtype=torch.float32, device="cuda")
    for g in grads:
        qcp.fp8_accum_requant(st_c, st_s, g, G)
    Ls = n // Ns
    rc, rs = qcp.dequant_reduce_requant(st_c, Ls, st_s, Ls // G, Ns, Ls, G, "e4m3", "e4m3")
    torch.cuda.synchronize()
    log("AGoQ: GPU done")
    check_scales(st_s)
    check_scales(rs)
    assert not ((st_c & 0x7F) == 0x7F).any() and not ((rc & 0x7F) == 0x7F).any()   # no NaN bytes
    nbs = Ls // G                                          # blocks per slice
    ks = sample_blocks(nbs, 5)
    kb = (np.arange(Ns)[:, None] * nbs + ks[None, :]).reshape(-1)   # block k of every slice
    oc = np.zeros(kb.size * G, np.uint8)
    os_ = np.zeros(kb.size, np.float32)
    for m, g in enumerate(grads):
        oc, os_ = oracle.fp8_accum_requant(oc, os_, host_blocks(g, G, kb), "bf16", G)
    assert_same_bytes(byte_blocks(st_c, G, kb), oc, "AGoQ state codes (sampled)")
    assert_same_bytes(st_s.cpu().numpy()[kb], os_, "AGoQ state scales (sampled)")
    m_len = ks.size * G
    wc, ws = oracle.dequant_reduce_requant(oc, m_len, os_, ks.size, Ns, m_len, G, "e4m3", "e4m3")
    assert_same_bytes(byte_blocks(rc, G, ks), wc, "AGoQ reduce codes (sampled)")
    assert_same_bytes(rs.cpu().numpy()[ks], ws, "AGoQ reduce scales (sampled)")


def test_qgz_reorder_quantize_fullsize():
    """The qgZ sender on one rank's 5e8-element fp16 bucket (Laplace(0, 1e-3)),
    4 nodes x 8 GPUs: 8 send slices of 62,500,000, INT4, G = 512."""
    K, N, G = S.QGZ_NODES, S.QGZ_SLICES, 512
    n = S.QGZ_BUCKET
    x = S.device_qgz_bucket(n)
    codes, cs, scales, ss = qcp.reorder_quantize(x, K, N, G, "int4")
    torch.cuda.synchronize()
    log("qgZ sender: GPU done")
    L, C = n // N, n // (K * N)
    nb = oracle.n_blocks(L, G)
    full = L // G
    check_scales(scales.view(N, ss)[:, :nb])
    rng = np.random.default_rng(8)
    for j in (0, 3, N - 1):
        ks = np.unique(np.concatenate([rng.choice(full, 300, replace=False), [0, full - 1]]))
        e = (ks[:, None] * G + np.arange(G)[None, :]).reshape(-1)          # elements of slice j
        src = (e // C * N + j) * C + e % C                                  # where they live in x
        xh = to_host(x[torch.from_numpy(src).cuda()]).view(np.float16)
        wc, ws = oracle.quantize_blockwise(xh, "f16", G, "int4")
        got = codes[j * cs:j * cs + full * G // 2].view(full, G // 2)[torch.from_numpy(ks).cuda()]
        assert_same_bytes(got.reshape(-1).cpu().numpy(), wc, f"sender codes, slice {j} (sampled)")
        assert_same_bytes(scales[j * ss:j * ss + full].cpu().numpy()[ks], ws,
                          f"sender scales, slice {j} (sampled)")
