"""Host-side accounting of the qgZ protocols against the volumes the pages
print ([ZPP] "Two-hop communication prevents QGZ traffic from multiplying
across GPUs"; tests/golden/pages_figures.txt): a one-hop all-to-all sends
N x M/4 across nodes per node, the two-hop protocol M/(4N) per GPU, in units of
the 16-bit model size M (2M bytes).  The pages' figures ignore the scales and
the chunks that stay on a GPU's own node, so they are the large-K, large-G
limit of the exact byte counts."""
import pytest

from quantized_collective_payloads_amd import protocols as Q
from tests.oracle_pins import golden_figures


def test_cross_node_volumes_match_the_pages():
    fig = golden_figures()
    K, N, G, C = 64, 8, 1024, 1 << 16
    M = K * N * C
    two = Q.cross_node_bytes_per_gpu("two_hop", M, K, N, G) / (2 * M)
    one_node = N * Q.cross_node_bytes_per_gpu("one_hop", M, K, N, G) / (2 * M)
    assert two == pytest.approx(float(fig["qgz.cross_node_per_gpu.N8"]), rel=0.025)
    assert one_node == pytest.approx(float(fig["onehop.cross_node.N8"]), rel=0.025)


@pytest.mark.parametrize("K,N", [(2, 8), (4, 8), (16, 4), (3, 5)])
def test_one_hop_sends_n_times_the_two_hop_volume(K, N):
    M, G = K * N * 4096, 512
    assert (Q.cross_node_bytes_per_gpu("one_hop", M, K, N, G) ==
            N * Q.cross_node_bytes_per_gpu("two_hop", M, K, N, G))


def test_single_node_sends_nothing_across_nodes():
    for p in ("one_hop", "two_hop", "ring"):
        assert Q.cross_node_bytes_per_gpu(p, 8 * 4096, 1, 8, 512) == 0
