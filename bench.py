#!/usr/bin/env python3
"""Throughput of the quantized-payload hot path on one MI355X.

One step is one pass of every row of the hot path, each at its workload's
full size, inputs resident in HBM before timing starts:
  qwZ      quantize INT8 (G=256) + dequantize to bf16 of a Llama-3-8B-shaped
           decoder layer, 218,103,808 bf16 values;
  qgZ      dequant -> fp32 sum -> requant INT4 (G=512) of the 8 slices one rank
           receives from a 5e8-element gradient bucket, 8 x 62,500,000;
  Aquavit  sub-byte pack + unpack of an 8192x28672 bf16 weight at
           (b,G) = (2,1024) (4,256) (4,64) (6,128) (6,32) (8,32);
  AGoQ     4 FP8 (E4M3, G=128) main-gradient accumulates of a 369,098,752-element
           70B-shaped layer, then the 8-slice fp32 local reduce of that state.
value = algorithmic bytes of the step (inputs + outputs of every kernel, never a
dense fp32 intermediate) / wall time of the step, in GB/s.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]

Prints one JSON line.  Per-kernel durations are measured with HIP events on the
stream the kernels run on, in the step and, for every step kernel, alone after
a 1 GiB read that leaves the caches holding unrelated data (median, min, max);
`roofline` describes the kernel with the largest share of the step;
`copy_ceiling` is a plain 1 GiB device-to-device copy and `stream_ceilings` torch's
elementwise add (2:1 read:write) and a fill (writes only) under the same
protocol; `tiny_roundtrip` is the
1,048,576-element qwZ round trip (launch-bound, reported outside the step);
`cpu_baseline` times the CPU oracle single-threaded on a 1/8 sample of the same
workload (about 10-30 s of host time).

    python bench.py --summarize-counters DIR [DIR ...] --bench-log FILE [--traffic-out FILE]

summarizes rocprofv3 --pmc runs of one bench.py command (their output
directories and the output of one of them): per kernel and context (warm, or
cold after the cache flush), the mean of every counter, and with the
request-size counters the HBM bytes per launch against the algorithmic bytes.
"""
from __future__ import annotations

import argparse
import functools
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "quantize / dequant-reduce-requant GB/s on 1 MI355X; % of HBM peak"
HBM_PEAK_GBS = 8000.0               # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(HERE, "profiles", "hbm_traffic.json")
CSRC = os.path.join(HERE, "quantized_collective_payloads_amd", "csrc")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# algorithmic bytes (inputs + outputs a kernel must move)
# ---------------------------------------------------------------------------

def nblk(n, G):
    return (n + G - 1) // G


def bytes_codec(n, in_bytes_per_elem, bits, G):
    """quantize (16-bit in, codes + scales out) or its inverse: same bytes."""
    return n * in_bytes_per_elem + (n * bits + 7) // 8 + 4 * nblk(n, G)


def bytes_reduce(N, L, bits_in, bits_out, G):
    slice_in = (L * bits_in + 7) // 8 + 4 * nblk(L, G)
    return N * slice_in + (L * bits_out + 7) // 8 + 4 * nblk(L, G)


def bytes_accum(n, G, grad_bytes=2):
    return n * (1 + 1 + grad_bytes) + 8 * nblk(n, G)


# ---------------------------------------------------------------------------
# the GPU step
# ---------------------------------------------------------------------------

class Step:
    """Allocates every row's inputs/outputs once, then runs the hot path."""

    def __init__(self, torch, qcp, S, n_states=1, extras=True):
        self.torch, self.qcp = torch, qcp
        dev = "cuda"
        bf16 = torch.bfloat16
        self.launches = []          # (row, kernel label, bytes, callable)

        # qwZ: Llama-3-8B-shaped decoder layer
        x = S.device_llama8b_layer(dev)
        n = x.numel()
        c = torch.empty(n, dtype=torch.uint8, device=dev)
        s = torch.empty(nblk(n, 256), dtype=torch.float32, device=dev)
        y = torch.empty(n, dtype=bf16, device=dev)
        b = bytes_codec(n, 2, 8, 256)
        self.launches.append(("qwZ", "quantize_blockwise(bf16->int8,G=256)", b,
                              functools.partial(qcp.quantize_blockwise, x, 256, "int8", c, s)))
        self.launches.append(("qwZ", "dequantize_blockwise(int8->bf16,G=256)", b,
                              functools.partial(qcp.dequantize_blockwise, c, s, "int8", n, 256,
                                                bf16, y)))
        self.qwz = (x, c, s, y)

        # qgZ: 8 received INT4 slices of 62.5M (quantized from Laplace fp16 by the
        # library's own encoder; input preparation, not timed)
        N, L, G = S.QGZ_SLICES, S.QGZ_SLICE_LEN, 512
        cb = (L * 4 + 7) // 8
        nb = nblk(L, G)
        stride, sstride = qcp.slice_layout(L, G, "int4")      # receive buffer: 256-byte slices
        slices = torch.zeros(N * stride, dtype=torch.uint8, device=dev)
        sscales = torch.zeros(N * sstride, dtype=torch.float32, device=dev)
        for j, g in enumerate(S.device_qgz_slices_fp16(L, N, dev)):
            qcp.quantize_blockwise(g, G, "int4", slices[j * stride:j * stride + cb],
                                   sscales[j * sstride:j * sstride + nb])
            del g
        qc = torch.empty(cb, dtype=torch.uint8, device=dev)
        qs = torch.empty(nb, dtype=torch.float32, device=dev)
        self.launches.append(("qgZ", "dequant_reduce_requant(8xint4->int4,G=512)",
                              bytes_reduce(N, L, 4, 4, G),
                              functools.partial(qcp.dequant_reduce_requant, slices, stride, sscales,
                                                sstride, N, L, G, "int4", "int4", False, qc, qs)))
        self.qgz = (slices, sscales, qc, qs)

        # Aquavit granularity sweep on a 70B MLP weight
        w = S.device_mlp70b(device=dev)
        nw = w.numel()
        self.aqv = [w]
        for bits, G in S.AQUAVIT_SWEEP:
            pk = torch.empty((nw * bits + 7) // 8, dtype=torch.uint8, device=dev)
            ps = torch.empty(nblk(nw, G), dtype=torch.float32, device=dev)
            yy = torch.empty(nw, dtype=bf16, device=dev)
            bb = bytes_codec(nw, 2, bits, G)
            self.launches.append(("Aquavit", f"pack_subbyte(bf16->int{bits},G={G})", bb,
                                  functools.partial(qcp.pack_subbyte, w, bits, G, pk, ps)))
            self.launches.append(("Aquavit", f"unpack_subbyte(int{bits}->bf16,G={G})", bb,
                                  functools.partial(qcp.unpack_subbyte, pk, ps, nw, bits, G, bf16,
                                                    yy)))
            self.aqv += [pk, ps, yy]

        # AGoQ: FP8 main-gradient accumulation over 4 micro-batches + local reduce.
        # Every step starts from the all-zero state, as the workload does: each
        # step takes the next of n_states pre-zeroed states (one per step the
        # timed regions run), so no zeroing happens inside the step.
        grads = S.device_agoq_grads(device=dev)
        na = grads[0].numel()
        G = 128
        self.states = [(torch.zeros(na, dtype=torch.uint8, device=dev),
                        torch.zeros(nblk(na, G), dtype=torch.float32, device=dev))
                       for _ in range(n_states)]
        self.cur = 0

        def accum(m, G=G):
            st_c, st_s = self.states[self.cur]
            qcp.fp8_accum_requant(st_c, st_s, grads[m], G)

        for m in range(len(grads)):
            self.launches.append(("AGoQ", f"fp8_accum_requant(bf16->e4m3,G=128) micro-batch {m}",
                                  bytes_accum(na, G), functools.partial(accum, m)))
        Ns = 8
        Ls = na // Ns
        rc = torch.empty(Ls, dtype=torch.uint8, device=dev)
        rs = torch.empty(nblk(Ls, G), dtype=torch.float32, device=dev)

        def local_reduce(G=G, Ns=Ns, Ls=Ls):
            st_c, st_s = self.states[self.cur]
            qcp.dequant_reduce_requant(st_c, Ls, st_s, Ls // G, Ns, Ls, G, "e4m3", "e4m3", False,
                                       rc, rs)

        self.launches.append(("AGoQ", "dequant_reduce_requant(8xe4m3->e4m3,G=128)",
                              bytes_reduce(Ns, Ls, 8, 8, G), local_reduce))
        self.agoq = (grads, rc, rs)
        self.bytes_per_step = sum(l[2] for l in self.launches)

        self.extra = []
        if extras:
            self._build_extra_rows(torch, qcp, S, dev, w, nw)
        torch.cuda.synchronize()

    def _build_extra_rows(self, torch, qcp, S, dev, w, nw):
        bf16 = torch.bfloat16
        # Rows beyond the step (timed on their own, not part of `value`):
        # the qgZ sender -- tensor-slice reordering fused with the INT4
        # quantization of one rank's 5e8-element bucket, 4 nodes x 8 GPUs.
        xb = S.device_qgz_bucket(device=dev)
        K, Nn, G = S.QGZ_NODES, S.QGZ_SLICES, 512
        Lb = xb.numel() // Nn
        cs, ss = qcp.slice_layout(Lb, G, "int4")
        sc_ = torch.empty(cs * Nn, dtype=torch.uint8, device=dev)
        ssc = torch.empty(ss * Nn, dtype=torch.float32, device=dev)
        self.extra.append(("qgZ sender", f"reorder_quantize(fp16->int4,G=512,{K}x{Nn})",
                           xb.numel() * 2 + Nn * ((Lb * 4 + 7) // 8 + 4 * nblk(Lb, G)),
                           functools.partial(qcp.reorder_quantize, xb, K, Nn, G, "int4", sc_, cs,
                                             ssc, ss)))
        self.sender = (xb, sc_, ssc)
        # qgZ stress variant: 8 received slices of a whole 5e8-element bucket each
        # (every peer's INT4 payload at bucket size), quantized by the library's
        # encoder as above (input preparation, not timed)
        LB, GB = S.QGZ_BUCKET, 512
        cbb, sbb = qcp.slice_layout(LB, GB, "int4")
        nbb = nblk(LB, GB)
        vb_c = torch.zeros(Nn * cbb, dtype=torch.uint8, device=dev)
        vb_s = torch.zeros(Nn * sbb, dtype=torch.float32, device=dev)
        for j in range(Nn):
            gj = S.device_laplace(LB, 1e-3, S.seed_for(3, 300 + j), torch.float16, dev)
            qcp.quantize_blockwise(gj, GB, "int4", vb_c[j * cbb:j * cbb + (LB * 4 + 7) // 8],
                                   vb_s[j * sbb:j * sbb + nbb])
            del gj
        vb_oc = torch.empty((LB * 4 + 7) // 8, dtype=torch.uint8, device=dev)
        vb_os = torch.empty(nbb, dtype=torch.float32, device=dev)
        self.extra.append(("qgZ variant B", f"dequant_reduce_requant(8xint4->int4,G=512,8x{LB})",
                           bytes_reduce(Nn, LB, 4, 4, GB),
                           functools.partial(qcp.dequant_reduce_requant, vb_c, cbb, vb_s, sbb, Nn, LB,
                                             GB, "int4", "int4", False, vb_oc, vb_os)))
        self.variant_b = (vb_c, vb_s, vb_oc, vb_os)
        # Aquavit payload with interleaved metadata ([scale][codes] per block) at the
        # schedule's two ends, on the same 8192x28672 weight
        for bits, G in ((2, 1024), (6, 32)):
            rec = torch.empty(qcp.payload_bytes(nw, bits, G), dtype=torch.uint8, device=dev)
            yr = torch.empty(nw, dtype=bf16, device=dev)
            bb = bytes_codec(nw, 2, bits, G)
            self.extra.append(("Aquavit records", f"pack_subbyte_records(bf16->int{bits},G={G})",
                               bb, functools.partial(qcp.pack_subbyte_records, w, bits, G, rec)))
            self.extra.append(("Aquavit records", f"unpack_subbyte_records(int{bits}->bf16,G={G})",
                               bb, functools.partial(qcp.unpack_subbyte_records, rec, nw, bits, G,
                                                     bf16, yr)))
            self.sender += (rec, yr)

    def run(self, events=None):
        if events is None:
            for _, _, _, fn in self.launches:
                fn()
        else:
            for i, (_, _, _, fn) in enumerate(self.launches):
                events[i][0].record()
                fn()
                events[i][1].record()
        self.cur = (self.cur + 1) % len(self.states)


# ---------------------------------------------------------------------------
# CPU oracle baseline on a 1/8 sample
# ---------------------------------------------------------------------------

def cpu_baseline(S, frac_div=8):
    import numpy as np
    import oracle

    timings = []       # (bytes, seconds)

    def timed(bytes_, fn, *a):
        t0 = time.perf_counter()
        out = fn(*a)
        timings.append((bytes_, time.perf_counter() - t0))
        return out

    # qwZ
    x = S.host_llama8b_layer(scale_down=frac_div)
    n = x.size
    c, s = timed(bytes_codec(n, 2, 8, 256), oracle.quantize_blockwise, x, "bf16", 256, "int8")
    timed(bytes_codec(n, 2, 8, 256), oracle.dequantize_blockwise, c, s, "int8", n, 256, "bf16")
    # qgZ (inputs quantized by the oracle, untimed)
    N, L, G = S.QGZ_SLICES, S.QGZ_SLICE_LEN // frac_div, 512
    cb = oracle.code_bytes(L, "int4")
    stride = (cb + 15) // 16 * 16
    nb = oracle.n_blocks(L, G)
    ss = (nb + 3) // 4 * 4
    buf = np.zeros(N * stride, np.uint8)
    sc = np.zeros(N * ss, np.float32)
    for j, g in enumerate(S.host_qgz_slices_fp16(L, N)):
        cc, s2 = oracle.quantize_blockwise(g, "f16", G, "int4")
        buf[j * stride:j * stride + cb] = cc
        sc[j * ss:j * ss + nb] = s2
    timed(bytes_reduce(N, L, 4, 4, G), oracle.dequant_reduce_requant, buf, stride, sc, ss, N, L,
          G, "int4", "int4")
    # Aquavit
    w = S.host_mlp70b(S.MLP70B_N // frac_div)
    nw = w.size
    for bits, G in S.AQUAVIT_SWEEP:
        pk, ps = timed(bytes_codec(nw, 2, bits, G), oracle.pack_subbyte, w, "bf16", bits, G)
        timed(bytes_codec(nw, 2, bits, G), oracle.unpack_subbyte, pk, ps, nw, bits, G, "bf16")
    # AGoQ
    na = S.AGOQ_LAYER_N // frac_div
    G = 128
    st_c = np.zeros(na, np.uint8)
    st_s = np.zeros(oracle.n_blocks(na, G), np.float32)
    for g in S.host_agoq_grads(na):
        st_c, st_s = timed(bytes_accum(na, G), oracle.fp8_accum_requant, st_c, st_s, g, "bf16", G)
    Ls = na // 8
    timed(bytes_reduce(8, Ls, 8, 8, G), oracle.dequant_reduce_requant, st_c, Ls, st_s, Ls // G, 8,
          Ls, G, "e4m3", "e4m3")
    tot_b = sum(b for b, _ in timings)
    tot_s = sum(t for _, t in timings)
    return {"value": round(tot_b / tot_s / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": (f"every row at 1/{frac_div} of its elements (same recipes, seeds and "
                       f"block sizes): {tot_b / 1e9:.2f} GB of algorithmic traffic in "
                       f"{tot_s:.1f} s on one host thread; host has {os.cpu_count()} CPUs")}


# ---------------------------------------------------------------------------
# qgZ protocols on 2 nodes x 8 virtual GPUs in this GPU's HBM
# ---------------------------------------------------------------------------

def qgz_protocols(torch, qcp, S, K=2, N=8, C=512 * 512, G=512):
    """Error against the exact (fp64) reduce-scatter, quantizations in
    sequence, cross-node bytes of the busiest GPU and wall time of the whole
    simulated exchange, for the two-hop, one-hop and ring protocols."""
    from quantized_collective_payloads_amd import protocols as Q
    W = K * N
    M = W * C
    buckets = [S.device_laplace(M, 1e-3, S.seed_for(3, 200 + r), torch.float16) for r in range(W)]
    exact = torch.zeros(M, dtype=torch.float64, device="cuda")
    for b in buckets:
        exact += b.double()
    res = {"nodes": K, "gpus_per_node": N, "bucket_elements": M, "format": "int4", "G": G}
    runs = {"two_hop": lambda: Q.two_hop(buckets, K, N, G), "one_hop": lambda: Q.one_hop(buckets, G),
            "ring": lambda: Q.ring(buckets, G)}
    for name, fn in runs.items():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        out = fn()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        err = torch.cat([out[r].double() - exact[r * C:(r + 1) * C] for r in range(W)])
        res[name] = {"rmse": float(err.pow(2).mean().sqrt()),
                     "quantization_steps": Q.quantization_steps(name, K, N),
                     "cross_node_bytes_per_gpu": Q.cross_node_bytes_per_gpu(name, M, K, N, G),
                     "simulated_exchange_ms": round(wall * 1e3, 2)}
    res["signal_rms"] = float(exact.pow(2).mean().sqrt())
    return res


def add_extras(out, torch, qcp, S):
    """The protocol comparison and the Aquavit schedule summary."""
    out["qgz_protocols"] = qgz_protocols(torch, qcp, S)
    T = 1000
    levels = [qcp.aquavit_level(t, T) for t in range(T)]
    out["aquavit_schedule"] = {
        "steps": T, "a": 0.9, "c": 5.0,
        "first": {"b": levels[0][0], "G": levels[0][1]},
        "last": {"b": qcp.aquavit_level(T, T)[0], "G": qcp.aquavit_level(T, T)[1]},
        "mean_bpw": round(sum(b + 32 / G for b, G in levels) / T, 4),
        "mean_bpw_unsnapped": round(sum(qcp.aquavit_target(t, T) for t in range(T)) / T, 4)}


def host_info(torch):
    """Host model, core count and library versions (context for cpu_baseline)."""
    import platform
    import subprocess

    import numpy as np
    model = platform.processor() or "unknown"
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    rocm = None
    for f in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(f):
            with open(f) as fh:
                rocm = fh.read().strip()
            break
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "numpy": np.__version__,
            "torch": torch.__version__, "torch_hip": getattr(torch.version, "hip", None),
            "rocm": rocm, "gpu": torch.cuda.get_device_name(0)}


class ColdTimer:
    """One launch timed alone with HIP events on the current stream, after a
    1 GiB read of an unrelated buffer: the read writes back dirty lines and
    leaves the caches (L2 and the 256 MB Infinity Cache) holding clean,
    unrelated data, so the kernel's inputs come from HBM and no earlier write-back
    is charged to it."""

    def __init__(self, torch):
        self.torch = torch
        self.flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        self.sink = torch.empty((), dtype=torch.float32, device="cuda")

    def time(self, fn, nbytes, reps, cold=True):
        torch = self.torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        fn()
        for e0, e1 in evs:
            if cold:
                torch.sum(self.flush, dim=(0,), out=self.sink)
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
        med = us[len(us) // 2]
        return {"median_us": round(med, 2), "min_us": round(us[0], 2), "max_us": round(us[-1], 2),
                "GBps": round(nbytes / (med * 1e-6) / 1e9, 1),
                "hbm_frac": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def copy_ceiling(torch, timer, reps=20):
    """A plain 1 GiB device-to-device copy (1 GiB read + 1 GiB written)."""
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    r = timer.time(lambda: dst.copy_(src), 2 * src.numel() * 4, reps)
    del src, dst
    return {"what": "torch copy_ of 2^28 fp32 (1 GiB read + 1 GiB written), cold", **r}


def stream_ceilings(torch, timer, reps=20):
    """torch's own streams over 1 GiB tensors, cold: an elementwise add (2 GiB
    read + 1 GiB written, a 2:1 mix like the encoders') and a fill (writes
    only, the limit the decoders' 1:4-1:8 mixes approach).  Context for the
    kernels' fractions of the 8 TB/s peak, not bounds.  (torch's sum, read
    only, is left out: as a two-pass reduction it reads at about half the
    rate the encoders do.)"""
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.ones_like(a)
    c = torch.empty_like(a)
    n = a.numel() * 4
    out = {"read2_write1": {"what": "torch.add of two 2^28 fp32 (2 GiB read + 1 GiB written), cold",
                            **timer.time(lambda: torch.add(a, b, out=c), 3 * n, reps)},
           "write_only": {"what": "fill_ of 2^28 fp32 (1 GiB written), cold",
                          **timer.time(lambda: c.fill_(1.0), n, reps)}}
    del a, b, c
    return out


def tiny_roundtrip(torch, qcp, S, timer, reps=20):
    """The 1,048,576-element fp16 qwZ round trip (INT8, G=256): 3 MB per call,
    so launch- and cache-dominated; reported apart from the step and exempt
    from the bandwidth bar."""
    import numpy as np
    x = torch.from_numpy(np.ascontiguousarray(S.host_tiny_roundtrip())).cuda()
    n = x.numel()
    c = torch.empty(n, dtype=torch.uint8, device="cuda")
    s = torch.empty(nblk(n, 256), dtype=torch.float32, device="cuda")
    y = torch.empty(n, dtype=torch.float16, device="cuda")
    b = bytes_codec(n, 2, 8, 256)
    q = functools.partial(qcp.quantize_blockwise, x, 256, "int8", c, s)
    d = functools.partial(qcp.dequantize_blockwise, c, s, "int8", n, 256, torch.float16, y)
    return {"workload": "1,048,576 fp16 ~ N(0, 0.02), seed 0; INT8 G=256; dequantize to fp16",
            "bytes_per_call": b, "exempt_from_bar": True,
            "quantize": {"cold": timer.time(q, b, reps), "back_to_back": timer.time(q, b, reps, False)},
            "dequantize": {"cold": timer.time(d, b, reps), "back_to_back": timer.time(d, b, reps, False)}}


# ---------------------------------------------------------------------------
# counter summaries (rocprofv3 --pmc runs of this script)
# ---------------------------------------------------------------------------

def _library_label(name):
    import re
    m = re.search(r"qcp::(k_\w+<[^>]*>)", name)
    return m.group(1) if m else None


def load_counter_runs(dirs):
    """Dispatches of one or more rocprofv3 --pmc runs of the same command, in
    launch order: kernel name, grid, duration (ns) and the counters of every
    run merged by dispatch index (the runs must launch the same sequence)."""
    import csv
    import glob
    merged = None
    for d in dirs:
        path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        disp = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                k = int(r["Dispatch_Id"])
                e = disp.setdefault(k, {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]),
                                        "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                                        "c": {}})
                e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        seq = [disp[k] for k in sorted(disp)]
        if merged is None:
            merged = seq
            continue
        if [(e["name"], e["grid"]) for e in seq] != [(e["name"], e["grid"]) for e in merged]:
            raise SystemExit(f"{d}: not the same launch sequence as {dirs[0]}")
        for a, b in zip(merged, seq):
            a["c"].update(b["c"])
            a["ns"] += b["ns"]
    for e in merged:
        e["ns"] /= len(dirs)
    return merged


def label_dispatches(seq, bench):
    """Give each library dispatch its bench label, algorithmic bytes and
    context.  `bench` is the JSON line the profiled run printed.  The step's
    launches are found as the W + 2K repetitions (warmup + both timed regions)
    of its launch sequence.  After them come, when the run timed them, each
    step kernel alone (1 + R launches per distinct kernel, R = cold_reps) and
    each row beyond the step (1 + R launches cold, then 1 + R back to back), in
    the order the JSON line lists them; launches after those (the small round
    trip, the protocol simulation) stay unlabelled.  context = "cold" if the
    dispatch before it is the cache flush (a torch reduction), else "warm"."""
    lib = [i for i, e in enumerate(seq) if _library_label(e["name"])]
    nl, reps = len(bench["kernels"]), bench["warmup"] + 2 * bench["steps"]
    key = [(_library_label(seq[i]["name"]), seq[i]["grid"]) for i in lib]
    start = next((o for o in range(len(lib) - nl * reps + 1)
                  if all(key[o + j] == key[o + j % nl] for j in range(nl * reps))), None)
    if start is None:
        raise SystemExit("the step's launch sequence was not found in the profile")
    label = [None] * len(lib)
    steplab = []
    for j in range(nl):
        k = bench["kernels"][j]
        steplab.append((k["kernel"].split(" micro-batch")[0], k["bytes"]))
    for pos in range(start, start + nl * reps):
        label[pos] = steplab[(pos - start) % nl]
    pos = start + nl * reps
    if "cold_reps" in bench and any("cold" in k for k in bench["kernels"]):
        blocks = []
        for lab in dict.fromkeys(steplab):          # distinct step kernels, in order
            blocks.append((lab, 1 + bench["cold_reps"]))
        for r in bench.get("next_rows", []):
            blocks.append(((r["kernel"], r["bytes"]), 2 * (1 + bench["cold_reps"])))
        for lab, cnt in blocks:
            if pos + cnt > len(lib) or len(set(key[pos:pos + cnt])) != 1:
                raise SystemExit(f"unexpected launches where {lab[0]} was timed alone")
            for q in range(pos, pos + cnt):
                label[q] = lab
            pos += cnt
    for q, i in enumerate(lib):
        e = seq[i]
        e["label"], e["bytes"] = label[q] if label[q] else (None, None)
        e["template"] = key[q][0]
        prev = seq[i - 1]["name"] if i else ""
        e["context"] = "cold" if ("reduce_kernel" in prev and not _library_label(prev)) else "warm"
    return [seq[i] for i in lib]


def hbm_bytes(c):
    """Bytes the L2 exchanged with the memory fabric, from the request-size
    counters summed over the TCC channels: reads = 32*RDREQ_32B + 64*RDREQ_64B
    + 128*RDREQ_128B, writes = 32*(WRREQ - WRREQ_64B) + 64*WRREQ_64B."""
    rd = wr = None
    if "TCC_EA0_RDREQ_128B_sum" in c:
        rd = (32 * c["TCC_EA0_RDREQ_32B_sum"] + 64 * c["TCC_EA0_RDREQ_64B_sum"]
              + 128 * c["TCC_EA0_RDREQ_128B_sum"])
    if "TCC_EA0_WRREQ_64B_sum" in c:
        wr = 32 * (c["TCC_EA0_WRREQ_sum"] - c["TCC_EA0_WRREQ_64B_sum"]) + 64 * c["TCC_EA0_WRREQ_64B_sum"]
    return rd, wr


def summarize_counters(dirs, bench_log, traffic_out=None):
    """Per (kernel, context) means of every counter of the runs in `dirs`,
    printed as a markdown table; with the request-size counters present, also
    HBM read/write bytes per launch and their ratio to the algorithmic bytes,
    written to `traffic_out` with the hash of the kernel sources."""
    import collections
    with open(bench_log) as f:
        bench = [json.loads(l) for l in f if l.startswith("{")][-1]
    seq = load_counter_runs(dirs)
    lib = label_dispatches(seq, bench)
    groups = collections.OrderedDict()
    for e in lib:
        if e["label"] is None:
            continue
        g = groups.setdefault((e["label"], e["template"], e["grid"], e["context"]),
                              {"n": 0, "ns": 0.0, "c": collections.Counter(), "bytes": e["bytes"]})
        g["n"] += 1
        g["ns"] += e["ns"]
        g["c"].update(e["c"])
    calib = [e for e in seq if e["grid"] == (1 << 28) // 4 and "Mul" in e["name"]]
    rows = []
    for (label, tmpl, grid, ctx), g in groups.items():
        c = {k: v / g["n"] for k, v in g["c"].items()}
        rd, wr = hbm_bytes(c)
        row = {"kernel": label, "template": tmpl, "grid": grid, "context": ctx, "launches": g["n"],
               "avg_us": round(g["ns"] / g["n"] / 1e3, 2), "algorithmic_bytes": g["bytes"],
               "counters": {k: round(v, 1) for k, v in sorted(c.items())}}
        if rd is not None and wr is not None:
            row.update(read_bytes=round(rd), write_bytes=round(wr), hbm_bytes_per_launch=round(rd + wr),
                       traffic_over_algorithmic=round((rd + wr) / g["bytes"], 4))
        rows.append(row)
    cal = None
    if calib:
        rd, wr = hbm_bytes(calib[-1]["c"])
        cal = {"what": "torch.mul of 2^28 fp32 (1 GiB read, 1 GiB written)",
               "read_bytes": None if rd is None else round(rd), "write_bytes": None if wr is None else round(wr)}
    cols = sorted({k for r in rows for k in r["counters"]})
    print("| kernel | template | context | launches | us | " + " | ".join(cols)
          + (" | read MB | write MB | HBM MB | algorithmic MB | ratio |" if rows and "read_bytes" in rows[0] else " |"))
    print("|---|---|---|---:|---:|" + "---:|" * len(cols) + ("---:|" * 5 if rows and "read_bytes" in rows[0] else ""))
    for r in rows:
        line = (f"| {r['kernel']} | `{r['template']}` | {r['context']} | {r['launches']} | {r['avg_us']} | "
                + " | ".join(f"{r['counters'].get(k, 0):.4g}" for k in cols) + " |")
        if "read_bytes" in r:
            line += (f" {r['read_bytes'] / 1e6:.1f} | {r['write_bytes'] / 1e6:.1f} | "
                     f"{r['hbm_bytes_per_launch'] / 1e6:.1f} | {r['algorithmic_bytes'] / 1e6:.1f} | "
                     f"{r['traffic_over_algorithmic']:.3f} |")
        print(line)
    if cal:
        print(f"\ncopy calibration: {cal}")
    if traffic_out:
        with open(traffic_out, "w") as f:
            json.dump({"source_hash": kernel_source_hash(), "method": hbm_bytes.__doc__,
                       "copy_calibration": cal,
                       "kernels": [{k: v for k, v in r.items() if k != "counters"} for r in rows]},
                      f, indent=1)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rows", action="store_true", help="also print a per-kernel table to stderr")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip everything beyond the two timed regions of the step (per-kernel cold "
                         "times, rows beyond the step, copy ceiling, tiny round trip), e.g. so that "
                         "a profile holds the step's launches only")
    ap.add_argument("--cold-reps", type=int, default=20, metavar="R",
                    help="launches per kernel for the cold-cache per-kernel statistics")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one plain elementwise copy of 1 GiB (reads 1 GiB, "
                         "writes 1 GiB) whose byte counters check the counter arithmetic")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="summarize rocprofv3 --pmc runs of one bench.py command (no GPU needed)")
    ap.add_argument("--bench-log", metavar="FILE",
                    help="with --summarize-counters: the output of the profiled runs (their JSON line)")
    ap.add_argument("--traffic-out", metavar="FILE",
                    help="with --summarize-counters: write the HBM bytes per launch here as JSON")
    args = ap.parse_args()
    if args.summarize_counters:
        if not args.bench_log:
            ap.error("--summarize-counters needs --bench-log")
        summarize_counters(args.summarize_counters, args.bench_log, args.traffic_out)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import qcp_synthetic as S
    import quantized_collective_payloads_amd as qcp

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    qcp.library()
    step = Step(torch, qcp, S, n_states=args.warmup + 2 * args.steps, extras=not args.no_extras)
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    # Timed region 1: K whole steps back to back, nothing between the launches.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step.run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = step.bytes_per_step / (wall / args.steps) / 1e9

    # Timed region 2: K more steps with a pair of HIP events around every launch
    # (on the stream the library launches on) for the per-kernel durations.  The
    # event packets add about 10 us between launches, which is why region 1 has none.
    nl = len(step.launches)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(nl)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(args.steps):
        step.run(ev[k])
    torch.cuda.synchronize()
    ms_per_step_instrumented = (time.perf_counter() - t1) * 1e3 / args.steps
    per = []
    for i, (row, label, b, _) in enumerate(step.launches):
        ms = sorted(ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps))
        avg = sum(ms) / len(ms)
        per.append({"row": row, "kernel": label, "bytes": b, "avg_us": round(avg * 1e3, 2),
                    "median_us": round(ms[len(ms) // 2] * 1e3, 2),
                    "GBps": round(b / (avg * 1e-3) / 1e9, 1),
                    "hbm_frac": round(b / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    # the dominant kernel: largest total time per step, grouped by kernel instance
    groups = {}
    for p in per:
        key = p["kernel"].split(" micro-batch")[0]
        g = groups.setdefault(key, {"us": 0.0, "bytes": p["bytes"], "n": 0})
        g["us"] += p["avg_us"]
        g["n"] += 1
    dom_key, dom = max(groups.items(), key=lambda kv: kv[1]["us"])
    dom_avg_us = dom["us"] / dom["n"]
    achieved = dom["bytes"] / (dom_avg_us * 1e-6) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        kernels = tr.get("kernels")
        ent = [k for k in (kernels if isinstance(kernels, list) else [])
               if k.get("kernel") == dom_key and k["context"] == "warm" and "hbm_bytes_per_launch" in k]
        if ent and tr.get("source_hash") == kernel_source_hash():
            traffic = ent[0]["hbm_bytes_per_launch"]
    roofline = {"bound": "hbm", "kernel": dom_key, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "algorithmic_bytes_per_launch": dom["bytes"],
                "avg_launch_us": round(dom_avg_us, 2), "launches_per_step": dom["n"]}

    out = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "cold_reps": args.cold_reps,
           "ms_per_step": round(ms_per_step, 4),
           "ms_per_step_with_kernel_events": round(ms_per_step_instrumented, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic (seeded torch generators on the GPU; recipes in qcp_synthetic.py)",
           "config": {"workload": "qwZ Llama-3-8B layer (218,103,808 bf16, INT8 G=256) + "
                                  "qgZ 8x62,500,000 INT4 G=512 reduce + Aquavit 8192x28672 bf16 "
                                  "(b,G) sweep + AGoQ 369,098,752 E4M3 G=128 (4 accumulates from "
                                  "the zero state + 8-slice reduce)",
                      "bytes_per_step": step.bytes_per_step, "kernels_per_step": nl,
                      "hbm_frac_of_step": round(value / HBM_PEAK_GBS, 4)},
           "roofline": roofline, "cpu_baseline": None, "kernels": per}

    if not args.no_extras:
        timer = ColdTimer(torch)
        # every step kernel alone from a cold cache (median, min, max).  The
        # accumulates run on one of the step's states, which keeps accumulating:
        # the same work per launch (the values stay far from the slow paths).
        seen = {}
        for p, (_, _, b, fn) in zip(per, step.launches):
            key = p["kernel"].split(" micro-batch")[0]
            if key not in seen:
                seen[key] = timer.time(fn, b, args.cold_reps)
            p["cold"] = seen[key]
        # rows beyond the step (not part of `value`)
        out["next_rows"] = [{"row": row, "kernel": label, "bytes": b,
                             "cold": timer.time(fn, b, args.cold_reps),
                             "back_to_back": timer.time(fn, b, args.cold_reps, False)}
                            for row, label, b, fn in step.extra]
        out["copy_ceiling"] = copy_ceiling(torch, timer)
        out["stream_ceilings"] = stream_ceilings(torch, timer)
        out["tiny_roundtrip"] = tiny_roundtrip(torch, qcp, S, timer)
        add_extras(out, torch, qcp, S)
    out["host"] = host_info(torch)
    if args.rows:
        for p in per:
            cd = p.get("cold", {})
            print(f"{p['row']:8s} {p['kernel']:52s} step {p['avg_us']:8.2f} us {100 * p['hbm_frac']:5.1f}%"
                  + (f" | cold {cd['median_us']:8.2f} us {100 * cd['hbm_frac']:5.1f}% "
                     f"[{cd['min_us']:.1f}, {cd['max_us']:.1f}]" if cd else ""), file=sys.stderr)
        for p in out.get("next_rows", []):
            print(f"next     {p['kernel']:52s} cold {p['cold']['median_us']:8.2f} us "
                  f"{100 * p['cold']['hbm_frac']:5.1f}%", file=sys.stderr)
        if "copy_ceiling" in out:
            sc = out["stream_ceilings"]
            print(f"copy ceiling {out['copy_ceiling']['GBps']} GB/s; 2:1 add "
                  f"{sc['read2_write1']['GBps']} GB/s; "
                  f"write only {sc['write_only']['GBps']} GB/s", file=sys.stderr)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}
        del src, dst
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(S)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
