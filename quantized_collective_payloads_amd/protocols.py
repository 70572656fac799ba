"""qgZ gradient reduce-scatter protocols on virtual ranks held in one GPU's HBM.

[ZPP] "Quantized LLM Training at Scale with ZeRO++":
  * "QGZ keeps reductions in full precision while sending quantized gradients":
    the ring reduce-scatter it replaces dequantizes, adds and requantizes at
    every hop, so a contribution goes through about one quantization per GPU
    (W-1 here); the one-hop all-to-all needs one, the two-hop protocol two.
  * "Two-hop communication prevents QGZ traffic from multiplying across GPUs":
    a one-hop all-to-all sends N x M/4 across nodes per node; the two-hop
    protocol (intra-node all-to-all and reduce, then inter-node) sends M/(4N)
    per GPU.
  * "Tensor-slice reordering fixes incorrect gradient placement".

Every protocol takes the W = K*N ranks' buckets (rank r = node*N + gpu, each a
1-D GPU tensor of M elements, M = W*C) and returns, for every rank r, the fp32
sums of chunk r over all ranks -- the reduce-scatter result, which the last
reduce leaves in full precision.  All arithmetic runs in the library's kernels
(quantize_blockwise, reorder_quantize, dequant_reduce_requant); the exchanges
between virtual ranks are device-to-device copies standing in for the
collectives.  Blocks restart at every chunk boundary as long as C is a
multiple of G, which these functions require (each chunk is then a whole
number of blocks and can be forwarded with its own scales).
"""
from __future__ import annotations

import torch

from . import (code_bytes, dequant_reduce_requant, n_blocks, quantize_blockwise,
               reorder_quantize, slice_layout)


def _chunk_len(buckets, n_ranks, G, fmt):
    M = buckets[0].numel()
    if M % n_ranks:
        raise ValueError("bucket size must be a multiple of the number of ranks")
    C = M // n_ranks
    if C % G:
        raise ValueError("each chunk must be a whole number of blocks")
    return C


def _stack(parts, stride, dtype, dev):
    """Copy payload parts into one N-slice receive buffer at `stride` elements."""
    buf = torch.zeros(stride * len(parts), dtype=dtype, device=dev)
    for i, p in enumerate(parts):
        buf[i * stride:i * stride + p.numel()].copy_(p)
    return buf


def two_hop(buckets, n_nodes: int, gpus_per_node: int, G: int = 512, fmt: str = "int4"):
    """qgZ: reorder+quantize, intra-node all-to-all + reduce, inter-node
    all-to-all + reduce."""
    K, N = n_nodes, gpus_per_node
    W = K * N
    C = _chunk_len(buckets, W, G, fmt)
    dev = buckets[0].device
    cb, nb = code_bytes(C, fmt), n_blocks(C, G)
    sent = [reorder_quantize(b, K, N, G, fmt) for b in buckets]        # per rank: N slices
    # hop 1: GPU j of node a reduces slice j of every GPU of its node (K chunks)
    hop1 = {}
    for a in range(K):
        for j in range(N):
            cs, ss = sent[a * N][1], sent[a * N][3]
            codes = _stack([sent[a * N + i][0][j * cs:(j + 1) * cs] for i in range(N)], cs,
                           torch.uint8, dev)
            scales = _stack([sent[a * N + i][2][j * ss:(j + 1) * ss] for i in range(N)], ss,
                            torch.float32, dev)
            hop1[a, j] = dequant_reduce_requant(codes, cs, scales, ss, N, K * C, G, fmt, fmt)
    # hop 2: GPU j of node b reduces piece b of hop 1 from GPU j of every node
    out = [None] * W
    cs2, ss2 = slice_layout(C, G, fmt)
    for b in range(K):
        for j in range(N):
            codes = _stack([hop1[a, j][0][b * cb:(b + 1) * cb] for a in range(K)], cs2,
                           torch.uint8, dev)
            scales = _stack([hop1[a, j][1][b * nb:(b + 1) * nb] for a in range(K)], ss2,
                            torch.float32, dev)
            out[b * N + j] = dequant_reduce_requant(codes, cs2, scales, ss2, K, C, G, fmt, fmt,
                                                    want_sum=True)[2]
    return out


def one_hop(buckets, G: int = 512, fmt: str = "int4"):
    """One all-to-all over all W ranks: every rank quantizes its bucket and
    sends chunk c to rank c, which reduces the W pieces."""
    W = len(buckets)
    C = _chunk_len(buckets, W, G, fmt)
    dev = buckets[0].device
    cb, nb = code_bytes(C, fmt), n_blocks(C, G)
    sent = [quantize_blockwise(b, G, fmt) for b in buckets]
    cs, ss = slice_layout(C, G, fmt)
    out = []
    for c in range(W):
        codes = _stack([s[0][c * cb:(c + 1) * cb] for s in sent], cs, torch.uint8, dev)
        scales = _stack([s[1][c * nb:(c + 1) * nb] for s in sent], ss, torch.float32, dev)
        out.append(dequant_reduce_requant(codes, cs, scales, ss, W, C, G, fmt, fmt,
                                          want_sum=True)[2])
    return out


def ring(buckets, G: int = 512, fmt: str = "int4"):
    """The ring reduce-scatter with quantized hops that qgZ replaces: the
    partial sum of chunk c starts at rank c+1 and passes through ranks c+2, ...,
    c (mod W); each receiver dequantizes it, adds its own contribution and
    requantizes (every contribution enters quantized, as it would be sent)."""
    W = len(buckets)
    if W < 2:
        raise ValueError("a ring needs at least two ranks")
    C = _chunk_len(buckets, W, G, fmt)
    dev = buckets[0].device
    cb, nb = code_bytes(C, fmt), n_blocks(C, G)
    own = [quantize_blockwise(b, G, fmt) for b in buckets]
    cs, ss = slice_layout(C, G, fmt)
    out = [None] * W
    for c in range(W):
        first = (c + 1) % W
        part = (own[first][0][c * cb:(c + 1) * cb], own[first][1][c * nb:(c + 1) * nb])
        for h in range(2, W + 1):
            m = (c + h) % W
            codes = _stack([part[0], own[m][0][c * cb:(c + 1) * cb]], cs, torch.uint8, dev)
            scales = _stack([part[1], own[m][1][c * nb:(c + 1) * nb]], ss, torch.float32, dev)
            part = dequant_reduce_requant(codes, cs, scales, ss, 2, C, G, fmt, fmt,
                                          want_sum=(h == W))
        out[c] = part[2]
    return out


def quantization_steps(protocol: str, n_nodes: int, gpus_per_node: int) -> int:
    """Quantizations in sequence on the longest path of a contribution to the
    final sum (the sender's own included; the final sum stays fp32): the ring
    requantizes at every one of its W-1 hops but the last."""
    W = n_nodes * gpus_per_node
    return {"ring": W - 1, "one_hop": 1, "two_hop": 2}[protocol]


def cross_node_bytes_per_gpu(protocol: str, M: int, n_nodes: int, gpus_per_node: int,
                             G: int = 512, fmt: str = "int4") -> int:
    """Payload bytes (codes + scales) the busiest GPU sends to other nodes in
    one reduce-scatter of an M-element bucket (ranks numbered node-major)."""
    K, N = n_nodes, gpus_per_node
    W = K * N
    C = M // W
    chunk = code_bytes(C, fmt) + 4 * n_blocks(C, G)
    if protocol == "one_hop":          # every chunk owned by a rank of another node
        return (W - N) * chunk
    if protocol == "two_hop":          # after hop 1: one chunk to each other node
        return (K - 1) * chunk
    if protocol == "ring":             # the last GPU of a node forwards W-1 chunks to the next node
        return (W - 1) * chunk if K > 1 else 0
    raise ValueError(protocol)
