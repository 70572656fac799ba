"""The qgZ reduce-scatter protocols on virtual ranks, restated on the host with
the CPU oracle (test infrastructure): the expected values for the GPU
simulation in quantized_collective_payloads_amd/protocols.py.  Written
separately from it -- plain numpy slicing for the exchanges, oracle functions
for every arithmetic step.  buckets[r] is rank r's fp16 bucket (rank r = node*N
+ gpu); each function returns rank r's fp32 sums of chunk r."""
import numpy as np

import oracle


def _reduce(payloads, C, G, fmt, want_sum):
    """payloads: list of (codes, scales) of C-element pieces -> oracle reduce."""
    cs, ss = oracle.slice_layout(C, G, fmt)
    codes = np.zeros(cs * len(payloads), np.uint8)
    scales = np.zeros(ss * len(payloads), np.float32)
    for i, (c, s) in enumerate(payloads):
        codes[i * cs:i * cs + c.size] = c
        scales[i * ss:i * ss + s.size] = s
    return oracle.dequant_reduce_requant(codes, cs, scales, ss, len(payloads), C, G, fmt, fmt,
                                         want_sum=want_sum)


def two_hop(buckets, K, N, G, fmt):
    W = K * N
    C = buckets[0].size // W
    L = K * C
    cb, nb = oracle.code_bytes(C, fmt), oracle.n_blocks(C, G)
    sent = [oracle.reorder_quantize(b, "f16", K, N, G, fmt) for b in buckets]
    lb, lnb = oracle.code_bytes(L, fmt), oracle.n_blocks(L, G)
    hop1 = {}
    for a in range(K):
        for j in range(N):
            pieces = []
            for i in range(N):
                codes, cs, scales, ss = sent[a * N + i]
                pieces.append((codes[j * cs:j * cs + lb], scales[j * ss:j * ss + lnb]))
            hop1[a, j] = _reduce(pieces, L, G, fmt, False)
    out = [None] * W
    for b in range(K):
        for j in range(N):
            pieces = [(hop1[a, j][0][b * cb:(b + 1) * cb], hop1[a, j][1][b * nb:(b + 1) * nb])
                      for a in range(K)]
            out[b * N + j] = _reduce(pieces, C, G, fmt, True)[2]
    return out


def one_hop(buckets, G, fmt):
    W = len(buckets)
    C = buckets[0].size // W
    cb, nb = oracle.code_bytes(C, fmt), oracle.n_blocks(C, G)
    sent = [oracle.quantize_blockwise(b, "f16", G, fmt) for b in buckets]
    return [_reduce([(c[r * cb:(r + 1) * cb], s[r * nb:(r + 1) * nb]) for c, s in sent],
                    C, G, fmt, True)[2] for r in range(W)]


def ring(buckets, G, fmt):
    W = len(buckets)
    C = buckets[0].size // W
    cb, nb = oracle.code_bytes(C, fmt), oracle.n_blocks(C, G)
    own = [oracle.quantize_blockwise(b, "f16", G, fmt) for b in buckets]
    out = []
    for c in range(W):
        m = (c + 1) % W
        part = (own[m][0][c * cb:(c + 1) * cb], own[m][1][c * nb:(c + 1) * nb])
        for h in range(2, W + 1):
            m = (c + h) % W
            mine = (own[m][0][c * cb:(c + 1) * cb], own[m][1][c * nb:(c + 1) * nb])
            part = _reduce([part, mine], C, G, fmt, h == W)
        out.append(part[2])
    return out
