"""Hardware self-test of the arithmetic shortcuts in the library's device code
(tests/hw/qcp_hw_selftest.hip): the fast reciprocal, the block scale with its
reciprocal, the Markstein quotient and the SDWA code conversions, each against
the IEEE operation it replaces -- exhaustively where the input space allows.
The GPU's own IEEE division, used as the reference there, is pinned to the
host's (numpy) on a sample first."""
import ctypes
import os

import numpy as np
import pytest
import torch

from tests.gpu_util import require_gpu

pytestmark = pytest.mark.gpu

HW_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw", "libqcp_hwtest.so")
U32P, F32P, VP = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p


@pytest.fixture(scope="module")
def hw():
    require_gpu()
    if not os.path.exists(HW_LIB):
        pytest.fail(f"{HW_LIB} is missing: build it with python -m tests.hw.build")
    lib = ctypes.CDLL(HW_LIB)
    lib.hw_recip_slots.restype = ctypes.c_int64
    lib.hw_block_scale_slots.restype = ctypes.c_int64
    lib.hw_recip_exhaustive.argtypes = [U32P, U32P, VP]
    lib.hw_block_scale_exhaustive.argtypes = [ctypes.c_int, U32P, U32P, VP]
    lib.hw_quot_sample.argtypes = [ctypes.c_uint32, ctypes.c_int64, U32P, U32P, VP]
    lib.hw_sdwa.argtypes = [F32P, VP]
    lib.hw_values.argtypes = [F32P, F32P, ctypes.c_int, F32P, F32P, F32P, F32P, VP]
    return lib


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def run_counts(fn, slots, *args):
    count = torch.full((slots,), 0xFFFFFFF, dtype=torch.int32, device="cuda")
    example = torch.zeros(slots, dtype=torch.int32, device="cuda")
    assert fn(*args, ptr(count), ptr(example), stream()) == 0
    torch.cuda.synchronize()
    c = count.cpu().numpy().astype(np.int64)
    e = example.cpu().numpy().view(np.uint32)
    return c, e


def test_gpu_ieee_division_matches_host(hw):
    rng = np.random.default_rng(3)
    n = 1 << 20
    s = (rng.random(n) * 2.0 + 0.5).astype(np.float32) * np.exp2(rng.integers(-63, 63, n)).astype(np.float32)
    x = (rng.standard_normal(n) * 100).astype(np.float32) * s
    xd, sd = torch.from_numpy(x).cuda(), torch.from_numpy(s).cuda()
    outs = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(4)]
    assert hw.hw_values(ptr(xd), ptr(sd), n, *map(ptr, outs), stream()) == 0
    q_ieee, q_fast, r_ieee, r_fast = (o.cpu().numpy() for o in outs)
    with np.errstate(all="ignore"):
        want_q = x / s
        want_r = np.float32(1.0) / s
    assert np.array_equal(q_ieee.view(np.uint32), want_q.view(np.uint32))
    assert np.array_equal(r_ieee.view(np.uint32), want_r.view(np.uint32))
    assert np.array_equal(q_fast.view(np.uint32), want_q.view(np.uint32))
    assert np.array_equal(r_fast.view(np.uint32), want_r.view(np.uint32))


def test_fast_reciprocal_is_ieee_on_its_whole_range(hw):
    c, e = run_counts(hw.hw_recip_exhaustive, hw.hw_recip_slots())
    bad = np.nonzero(c)[0]
    assert bad.size == 0, f"{c.sum()} reciprocals differ, e.g. s bits {e[bad[:4]]}"


@pytest.mark.parametrize("fmt", [2, 4, 6, 8, 0x43])
def test_block_scale_is_ieee_for_every_absmax(hw, fmt):
    c, e = run_counts(lambda *a: hw.hw_block_scale_exhaustive(fmt, *a), hw.hw_block_scale_slots())
    bad = np.nonzero(c)[0]
    assert bad.size == 0, f"{c.sum()} block scales differ, e.g. absmax bits {e[bad[:4]]}"


def test_markstein_quotient_sample(hw):
    waves = 1 << 16                      # 2^28 (x, s) pairs
    c, e = run_counts(lambda *a: hw.hw_quot_sample(12345, waves, *a), waves)
    bad = np.nonzero(c)[0]
    assert bad.size == 0, f"{c.sum()} quotients differ, e.g. counters {e[bad[:4]]}"


def test_sdwa_code_conversions(hw):
    out = torch.empty(2048, dtype=torch.float32, device="cuda")
    assert hw.hw_sdwa(ptr(out), stream()) == 0
    o = out.cpu().numpy().reshape(4, 256, 2)
    v = np.arange(256)
    sbyte = v.astype(np.uint8).view(np.int8).astype(np.float32)
    nib16 = (((v & 15) ^ 8) - 8).astype(np.float32) / 16
    for k in range(4):
        assert np.array_equal(o[k, :, 0], sbyte), f"signed byte at position {k}"
        assert np.array_equal(o[k, :, 1], nib16), f"signed low nibble / 16 at position {k}"
