"""Helpers shared by the GPU tests: host <-> device copies and bit-level views.
Inputs always come from qcp_synthetic (or are written out here), expected
values always from the CPU oracle."""
import numpy as np
import pytest
import torch

import quantized_collective_payloads_amd as qcp

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
NP_DT = {"f16": np.float16, "bf16": np.uint16, "f32": np.float32}
FMTS = ["int2", "int4", "int6", "int8", "e4m3"]
GS = [32, 64, 128, 256, 512, 1024]
DTS = ["f16", "bf16", "f32"]


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    qcp.library()          # raises if libqcp.so is missing: no fallback


def to_gpu(a: np.ndarray, dt: str = None) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dt == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    else:
        t = torch.from_numpy(a)
    return t.cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    return a.view({1: np.uint8, 2: np.uint16, 4: np.uint32}[a.dtype.itemsize])


def assert_same_bytes(got, want, what):
    got, want = bits(np.asarray(got)), bits(np.asarray(want))
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:8]}: got {got[bad[:8]]} want {want[bad[:8]]}"


def cast_host(x32: np.ndarray, dt: str) -> np.ndarray:
    """float32 host data -> the element type dt (RNE), as the oracle takes it."""
    if dt == "f32":
        return x32.astype(np.float32)
    if dt == "f16":
        return x32.astype(np.float16)
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def host_values(dt_np: np.ndarray, dt: str) -> np.ndarray:
    if dt == "bf16":
        return (dt_np.astype(np.uint32) << 16).view(np.float32)
    return dt_np.astype(np.float32)
