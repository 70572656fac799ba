"""The qgZ reduce-scatter protocols on virtual ranks (two-hop, one-hop
all-to-all, ring with requantization at every hop), run with the library's
kernels on one GPU, against the same protocols restated with the CPU oracle
(tests/protocol_sim.py): every rank's fp32 result byte for byte."""
import numpy as np
import pytest
import torch

from quantized_collective_payloads_amd import protocols as Q
from tests import protocol_sim as P
from tests.gpu_util import assert_same_bytes, require_gpu, to_gpu, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def buckets(K, N, C, seed):
    rng = np.random.default_rng(seed)
    return [rng.laplace(0, 1e-3 * (1 + 0.1 * r), K * N * C).astype(np.float32).astype(np.float16)
            for r in range(K * N)]


@pytest.mark.parametrize("K,N,C,G,fmt", [(2, 4, 1024, 512, "int4"), (3, 2, 256, 128, "int8"),
                                         (1, 4, 512, 32, "int4"), (2, 2, 2048, 256, "e4m3")])
def test_protocols_match_oracle(K, N, C, G, fmt):
    bk = buckets(K, N, C, 10 * K + N)
    dev = [to_gpu(b) for b in bk]
    cases = [("two_hop", Q.two_hop(dev, K, N, G, fmt), P.two_hop(bk, K, N, G, fmt)),
             ("one_hop", Q.one_hop(dev, G, fmt), P.one_hop(bk, G, fmt))]
    if K * N > 1:
        cases.append(("ring", Q.ring(dev, G, fmt), P.ring(bk, G, fmt)))
    for name, got, want in cases:
        for r in range(K * N):
            assert_same_bytes(to_host(got[r]), want[r], f"{name} rank {r} K={K} N={N} {fmt}")


def test_two_hop_beats_the_ring():
    """Fewer sequential quantizations, less error: the ring's W-1 requantizing
    hops against qgZ's two quantizations ([ZPP] "QGZ keeps reductions in full
    precision ...")."""
    K, N, C, G = 2, 8, 2048, 512
    bk = buckets(K, N, C, 5)
    dev = [to_gpu(b) for b in bk]
    exact = sum(b.astype(np.float64) for b in bk)

    def rmse(out):
        e = np.concatenate([to_host(out[r]).astype(np.float64) - exact[r * C:(r + 1) * C]
                            for r in range(K * N)])
        return float(np.sqrt((e ** 2).mean()))
    r_ring, r_two, r_one = rmse(Q.ring(dev, G)), rmse(Q.two_hop(dev, K, N, G)), rmse(Q.one_hop(dev, G))
    assert r_one < r_two < r_ring, (r_one, r_two, r_ring)
    assert Q.quantization_steps("ring", K, N) == K * N - 1
    assert Q.quantization_steps("two_hop", K, N) == 2
