"""The library on the caller's streams and inside HIP graphs: every entry point
enqueues on the stream it is given (torch's current stream in the binding),
allocates nothing and issues no memset, so a captured sequence of calls
replays to the same bytes.  Replays are checked one by one against the eager
results, with eager work and synchronizations between them."""
import numpy as np
import pytest
import torch

import quantized_collective_payloads_amd as qcp
from tests.gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def inputs(seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = (torch.randn(1 << 20, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    grad = (torch.randn(1 << 20, generator=g, device="cuda") * 5e-4).to(torch.bfloat16)
    return x, grad


def run_chain(x, grad, out):
    """quantize -> dequantize, pack -> unpack, 8-slice reduce, 2 FP8 accumulates."""
    c, s, y, pk, ps, yy, rc, rs, st_c, st_s = out
    qcp.quantize_blockwise(x, 256, "int8", c, s)
    qcp.dequantize_blockwise(c, s, "int8", x.numel(), 256, torch.bfloat16, y)
    qcp.pack_subbyte(x, 6, 32, pk, ps)
    qcp.unpack_subbyte(pk, ps, x.numel(), 6, 32, torch.bfloat16, yy)
    L = x.numel() // 8
    qcp.dequant_reduce_requant(c, L, s, L // 256, 8, L, 256, "int8", "int4", False, rc, rs)
    for _ in range(2):
        qcp.fp8_accum_requant(st_c, st_s, grad, 128)


def buffers(n):
    z = lambda k, dt: torch.zeros(k, dtype=dt, device="cuda")
    L = n // 8
    return (z(n, torch.uint8), z(n // 256, torch.float32), z(n, torch.bfloat16),
            z(n * 6 // 8, torch.uint8), z(n // 32, torch.float32), z(n, torch.bfloat16),
            z(L // 2, torch.uint8), z(L // 256, torch.float32),
            z(n, torch.uint8), z(n // 128, torch.float32))


def snapshot(out):
    return [t.view(torch.uint8).clone() if t.dtype != torch.bfloat16 else t.view(torch.int16).clone()
            for t in out]


def test_side_stream_gives_the_same_bytes():
    x, grad = inputs(1)
    ref = buffers(x.numel())
    run_chain(x, grad, ref)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    out = buffers(x.numel())
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_chain(x, grad, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for a, b in zip(snapshot(ref), snapshot(out)):
        assert torch.equal(a, b)


def test_results_are_deterministic():
    x, grad = inputs(2)
    runs = []
    for _ in range(3):
        out = buffers(x.numel())
        run_chain(x, grad, out)
        torch.cuda.synchronize()
        runs.append(snapshot(out))
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)


def test_graph_capture_replays_match_eager():
    x, grad = inputs(3)
    n = x.numel()
    eager = buffers(n)
    run_chain(x, grad, eager)                       # state after 2 accumulates
    torch.cuda.synchronize()
    want = snapshot(eager)

    out = buffers(n)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):                 # warm-up outside the capture
        run_chain(x, grad, buffers(n))
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_chain(x, grad, out)
    for rep in range(4):
        out[8].zero_()                              # FP8 state back to empty
        out[9].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot(out)
        for i, (a, b) in enumerate(zip(want, got)):
            assert torch.equal(a, b), (rep, i)
        # eager work between replays
        _ = (x.float() * 2).sum().item()
