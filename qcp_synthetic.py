"""Seeded synthetic inputs for the quantized-payload hot path.

This module only draws random tensors of the shapes and value distributions of
the workloads on the pages; it holds none of the method's arithmetic (no
scaling, rounding to codes or packing).  Both the CPU oracle's tests and the HIP
path's tests and benchmark take their inputs from here.

Two generators with the same recipe:
  * ``host_*``  -- numpy PCG64 (``np.random.default_rng(seed)``) on the CPU;
  * ``device_*`` -- torch's generator on a GPU, for full-size inputs that would
    take the host too long to draw.
Casts of the drawn float32 values to float16 / bfloat16 are round-to-nearest-
even (numpy ``astype`` and torch ``.to``).  bfloat16 host data is returned as
``np.uint16`` bit patterns.

Workloads (sizes as the pages' settings give them):
  * qwZ tiny round trip: 1,048,576 fp16 ~ N(0, 0.02), seed 0.
  * qwZ forward-gather payload of one Llama-3-8B-shaped decoder layer: bf16
    4096x4096 (x2), 4096x1024 (x2), 4096x14336 (x3), N(0, 0.02), each element
    independently an outlier with probability 0.001, value +-0.4 (20 sigma).
  * qgZ local reduce of one 5e8-element gradient bucket: 8 received slices of
    62,500,000 fp16 ~ Laplace(0, 1e-3) (scale parameter 1e-3); the sender side
    reorders and quantizes one rank's whole 5e8-element bucket (4 nodes x 8 GPUs).
  * Aquavit granularity sweep on a 70B-shaped MLP weight: bf16 8192x28672
    ~ N(0, 0.015).
  * AGoQ FP8 gradients of a 70B-shaped layer: 8192x28672 + 2 x 8192x8192
    bf16 gradients ~ N(0, 5e-4), 4 independent micro-batches.
"""
from __future__ import annotations

import numpy as np

LLAMA8B_LAYER_SHAPES = [(4096, 4096), (4096, 4096), (4096, 1024), (4096, 1024),
                        (4096, 14336), (4096, 14336), (4096, 14336)]
LLAMA8B_LAYER_N = sum(r * c for r, c in LLAMA8B_LAYER_SHAPES)          # 218,103,808
QGZ_SLICES = 8
QGZ_SLICE_LEN = 62_500_000                                             # 5e8 / 8
QGZ_BUCKET = 500_000_000                                               # reduce_bucket_size 5e8
QGZ_NODES = 4                                                          # sender: 4 nodes x 8 GPUs
MLP70B_SHAPE = (8192, 28672)
MLP70B_N = MLP70B_SHAPE[0] * MLP70B_SHAPE[1]                           # 234,881,024
AGOQ_LAYER_SHAPES = [(8192, 28672), (8192, 8192), (8192, 8192)]
AGOQ_LAYER_N = sum(r * c for r, c in AGOQ_LAYER_SHAPES)                # 369,098,752
AGOQ_MICROBATCHES = 4
AQUAVIT_SWEEP = [(2, 1024), (4, 256), (4, 64), (6, 128), (6, 32), (8, 32)]

OUTLIER_P = 0.001
OUTLIER_VALUE = 0.4


def seed_for(workload: int, tensor: int = 0) -> int:
    """Seed of tensor `tensor` of workload number `workload` (1 = tiny round
    trip uses seed 0; workload k >= 2 uses 1000*k + tensor)."""
    return 0 if workload == 1 else 1000 * workload + tensor


# ----------------------------------------------------------------------------
# host (numpy) generators
# ----------------------------------------------------------------------------

def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def host_normal(n: int, sigma: float, seed: int, dtype: str) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n, dtype=np.float32) * np.float32(sigma)
    return _cast(x, dtype)


def host_normal_outliers(n: int, sigma: float, seed: int, dtype: str,
                         p: float = OUTLIER_P, value: float = OUTLIER_VALUE) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n, dtype=np.float32) * np.float32(sigma)
    hit = rng.random(n) < p
    sign = np.where(rng.random(n) < 0.5, np.float32(-1.0), np.float32(1.0))
    x = np.where(hit, sign * np.float32(value), x).astype(np.float32)
    return _cast(x, dtype)


def host_laplace(n: int, scale: float, seed: int, dtype: str) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.laplace(0.0, scale, n).astype(np.float32)
    return _cast(x, dtype)


def _cast(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x32.astype(np.float32)
    if dtype == "f16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        return _to_bf16_bits(x32)
    raise ValueError(dtype)


def host_tiny_roundtrip() -> np.ndarray:
    return host_normal(1_048_576, 0.02, seed_for(1), "f16")


def host_llama8b_layer(scale_down: int = 1) -> np.ndarray:
    """The 7 matrices of one decoder layer, flattened and concatenated in the
    order of ``LLAMA8B_LAYER_SHAPES``.  ``scale_down`` > 1 keeps every matrix's
    first rows/scale_down rows (same recipe, fewer elements)."""
    parts = []
    for t, (r, c) in enumerate(LLAMA8B_LAYER_SHAPES):
        n = (r // scale_down) * c
        parts.append(host_normal_outliers(n, 0.02, seed_for(2, t), "bf16"))
    return np.concatenate(parts)


def host_qgz_slices_fp16(slice_len: int = QGZ_SLICE_LEN, n_slices: int = QGZ_SLICES):
    """The gradient values each of the N peers quantizes before sending."""
    return [host_laplace(slice_len, 1e-3, seed_for(3, j), "f16") for j in range(n_slices)]


def host_mlp70b(n: int = MLP70B_N) -> np.ndarray:
    return host_normal(n, 0.015, seed_for(4), "bf16")


def host_agoq_grads(n: int = AGOQ_LAYER_N, microbatches: int = AGOQ_MICROBATCHES):
    return [host_normal(n, 5e-4, seed_for(5, m), "bf16") for m in range(microbatches)]


# ----------------------------------------------------------------------------
# device (torch) generators: same distributions, drawn on a GPU
# ----------------------------------------------------------------------------

def _gen(seed: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def device_normal(n: int, sigma: float, seed: int, dtype, device="cuda"):
    import torch
    g = _gen(seed, device)
    return (torch.randn(n, generator=g, device=device, dtype=torch.float32) * sigma).to(dtype)


def device_normal_outliers(n: int, sigma: float, seed: int, dtype, device="cuda",
                           p: float = OUTLIER_P, value: float = OUTLIER_VALUE):
    import torch
    g = _gen(seed, device)
    x = torch.randn(n, generator=g, device=device, dtype=torch.float32) * sigma
    hit = torch.rand(n, generator=g, device=device) < p
    sign = torch.where(torch.rand(n, generator=g, device=device) < 0.5, -1.0, 1.0)
    x = torch.where(hit, sign * value, x)
    return x.to(dtype)


def device_laplace(n: int, scale: float, seed: int, dtype, device="cuda"):
    """Laplace(0, scale) by inversion of its CDF: for u ~ U(-1/2, 1/2),
    x = -scale * sign(u) * ln(1 - 2|u|)."""
    import torch
    g = _gen(seed, device)
    u = torch.rand(n, generator=g, device=device, dtype=torch.float64) - 0.5
    x = -scale * torch.sign(u) * torch.log1p(-2.0 * u.abs())
    return x.to(torch.float32).to(dtype)


def device_llama8b_layer(device="cuda"):
    import torch
    return torch.cat([device_normal_outliers(r * c, 0.02, seed_for(2, t), torch.bfloat16, device)
                      for t, (r, c) in enumerate(LLAMA8B_LAYER_SHAPES)])


def device_qgz_slices_fp16(slice_len: int = QGZ_SLICE_LEN, n_slices: int = QGZ_SLICES,
                           device="cuda"):
    import torch
    return [device_laplace(slice_len, 1e-3, seed_for(3, j), torch.float16, device)
            for j in range(n_slices)]


def device_qgz_bucket(n: int = QGZ_BUCKET, device="cuda"):
    """One rank's fp16 gradient bucket before the qgZ sender reorders and
    quantizes it (same distribution as the slices)."""
    import torch
    return device_laplace(n, 1e-3, seed_for(3, 100), torch.float16, device)


def device_mlp70b(n: int = MLP70B_N, device="cuda"):
    import torch
    return device_normal(n, 0.015, seed_for(4), torch.bfloat16, device)


def device_agoq_grads(n: int = AGOQ_LAYER_N, microbatches: int = AGOQ_MICROBATCHES,
                      device="cuda"):
    import torch
    return [device_normal(n, 5e-4, seed_for(5, m), torch.bfloat16, device)
            for m in range(microbatches)]
