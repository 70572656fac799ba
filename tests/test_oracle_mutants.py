"""Plant plausible mistakes in copies of the CPU oracle and check that the pins
catch every one (CPU only).  Each mutant is a one-line textual change to
oracle/qcp_oracle.c -- a dropped term, a wrong sign, bound or index, a wrong
rounding rule -- compiled into a temporary library; at least one pin must fail
against it.  This is the evidence that the pins constrain the oracle rather
than restate it."""
import os
import subprocess
import tempfile

import pytest

import oracle
from oracle import build as obuild
from tests import oracle_pins as P

MUTANTS = {
    "qmax_off_by_one": ("(float)((1 << (f - 1)) - 1)", "(float)(1 << (f - 1))"),
    "scale_wrong_divisor": ("return absmax / fmt_qmax(fmt);", "return absmax / (fmt_qmax(fmt) + 1.0f);"),
    "round_truncates": ("float c = nearbyintf(q);", "float c = truncf(q);"),
    "round_half_away": ("float c = nearbyintf(q);", "float c = roundf(q);"),
    "quotient_by_reciprocal": ("float q = x / s;", "float q = x * (1.0f / s);"),
    "clamp_too_tight": ("if (!(c <= qmax)) c = qmax;", "if (!(c <= qmax - 1)) c = qmax - 1;"),
    "bitstream_msb_first": ("int64_t bit = (int64_t)b * i + t;\n        if ((f >> t)",
                            "int64_t bit = (int64_t)b * i + (b - 1 - t);\n        if ((f >> t)"),
    "sign_extend_wrong": ("if (f & (1 << (b - 1))) f -= (1 << b);",
                          "if (f & (1 << (b - 1))) f -= (1 << (b - 1));"),
    "absmax_without_abs": ("if (fabsf(v[i]) > a) a = fabsf(v[i]);", "if (v[i] > a) a = v[i];"),
    "absmax_skips_last": ("block_scale(block_absmax(v + lo, len), fmt)",
                          "block_scale(block_absmax(v + lo, len > 1 ? len - 1 : len), fmt)"),
    "e4m3_saturate_drops_sign": ("if (!(a < 448.0)) return sign | 0x7e;", "if (!(a < 448.0)) return 0x7e;"),
    "e4m3_subnormal_edge": ("if (e == -6 && m < 8.0) return sign | (uint8_t)m;",
                            "if (e == -6 && m < 7.0) return sign | (uint8_t)m;"),
    "e4m3_decode_bias": ("v = ldexp(8.0 + m, e - 10);", "v = ldexp(8.0 + m, e - 11);"),
    "e4m3_zero_block_sign": ("if (s == 0.0f) return 0x00;", "if (s == 0.0f) return signbit(x) ? 0x80 : 0x00;"),
    "f16_round_half_up": ("double m = nearbyint(ldexp(a, 10 - e));", "double m = floor(ldexp(a, 10 - e) + 0.5);"),
    "f16_widen_exponent": ("v = ldexp(1024.0 + m, e - 25);", "v = ldexp(1024.0 + m, e - 24);"),
    "bf16_ties_up": ("return ((lo >> 16) & 1) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);",
                     "return (uint16_t)(hi >> 16);"),
    "reduce_mul_then_add": ("acc = fmaf(code_value(slice, i, fmt_in), s, acc);",
                            "acc = code_value(slice, i, fmt_in) * s + acc;"),
    "reduce_starts_at_plus_zero": ("float acc = -0.0f;", "float acc = 0.0f;"),
    "reduce_ignores_slice_scale": ("float s = scales_in[(int64_t)j * in_scale_stride + i / G];",
                                   "float s = scales_in[i / G];"),
    "reduce_ignores_slice_stride": ("(const uint8_t *)codes_in + (int64_t)j * in_slice_stride_bytes;",
                                    "(const uint8_t *)codes_in;"),
    "accum_unrounded_dequant": (
        "float d = bf16_value(bf16_round(e4m3_value(state_codes[i]) * state_scales[i / G]));",
        "float d = e4m3_value(state_codes[i]) * state_scales[i / G];"),
    "accum_unrounded_sum": ("t[i] = bf16_value(bf16_round(d + load_elem(grad, gt, i)));",
                            "t[i] = d + load_elem(grad, gt, i);"),
    "accum_subtracts": ("t[i] = bf16_value(bf16_round(d + load_elem(grad, gt, i)));",
                        "t[i] = bf16_value(bf16_round(d - load_elem(grad, gt, i)));"),
    "dequant_block_index": ("store_elem(y, yt, i, c * scales[i / G]);",
                            "store_elem(y, yt, i, c * scales[i / (G + 1)]);"),
    "reorder_transposed": ("(const uint8_t *)x + ((b * gpus_per_node + j) * C) * esz",
                           "(const uint8_t *)x + ((j * n_nodes + b) * C) * esz"),
    "reorder_node_order_reversed": ("(uint8_t *)y + (j * n_nodes * C + b * C) * esz",
                                    "(uint8_t *)y + (j * n_nodes * C + (n_nodes - 1 - b) * C) * esz"),
    "aquavit_a_c_swapped": ("return 8.0 - 6.0 / (a + c * (double)t / (double)T);",
                            "return 8.0 - 6.0 / (c + a * (double)t / (double)T);"),
    "aquavit_picks_from_above": ("double d = fabs(bpw - target);",
                                 "double d = bpw >= target ? bpw - target : 1e9 + target - bpw;"),
    "records_codes_first": ("memcpy(rec, &scales[k], 4);\n        memcpy(rec + 4,",
                            "memcpy(rec + (len * b + 7) / 8, &scales[k], 4);\n        memcpy(rec,"),
    "payload_floor_blocks": ("return (n * bits + 7) / 8 + 4 * ((n + G - 1) / G);",
                             "return (n * bits + 7) / 8 + 4 * (n / G);"),
}


@pytest.fixture(scope="module")
def source():
    with open(obuild.SRC, encoding="utf-8") as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) >= 1, f"mutant {name}: pattern not found in the oracle"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new, 1))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", *obuild.CFLAGS, "-o", str(lib), str(src), "-lm"], check=True)
    caught = []
    with oracle.loaded_from(str(lib)):
        for pin in P.ALL_PINS:
            try:
                pin(oracle)
            except (AssertionError, ValueError, IndexError) as e:   # a pin tripped
                caught.append(pin.__name__)
                break
    assert caught, f"no pin catches the planted mistake {name!r}"
