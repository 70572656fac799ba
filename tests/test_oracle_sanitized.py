"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): a sanitized build runs every pin and a set of ragged-size calls of each
entry point in a child process with the ASan runtime preloaded; any
out-of-bounds access, use after free, signed overflow, bad shift or misaligned
access aborts it.  A copy with one planted one-byte overflow shows that the
instrumentation is live."""
import os
import subprocess
import sys
import textwrap

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CALLS = textwrap.dedent("""
    import sys
    import numpy as np
    sys.path.insert(0, ROOT)
    import oracle
    from tests import oracle_pins as P

    def ragged(G):
        return [1, 7, G - 1, G, G + 9, 3 * G + 41]

    with oracle.loaded_from(LIB):
        for pin in P.ALL_PINS:
            pin(oracle)
        print("pins ok", len(P.ALL_PINS), flush=True)
        rng = np.random.default_rng(3)
        for G in (32, 128, 1024):
            for n in ragged(G):
                x = (rng.standard_normal(n) * 0.02).astype(np.float32)
                for dt in ("f32", "f16", "bf16"):
                    xh = x if dt == "f32" else (x.astype(np.float16) if dt == "f16" else
                                                (x.view(np.uint32) >> 16).astype(np.uint16))
                    for fmt in ("int2", "int4", "int6", "int8", "e4m3"):
                        c, s = oracle.quantize_blockwise(xh, dt, G, fmt)
                        for yt in ("f32", "f16", "bf16"):
                            oracle.dequantize_blockwise(c, s, fmt, n, G, yt)
                    for b in (2, 4, 6, 8):
                        r = oracle.pack_records(xh, dt, b, G)
                        oracle.unpack_records(r, n, b, G, "bf16")
                for N in (1, 3, 8):
                    for fi, fo in (("int4", "int4"), ("e4m3", "e4m3"), ("int6", "int2"), ("int8", "e4m3")):
                        cs, ss = oracle.slice_layout(n, G, fi)
                        codes = rng.integers(0, 256, N * cs, dtype=np.uint8)
                        scales = (rng.random(N * ss) * 1e-3).astype(np.float32)
                        oracle.dequant_reduce_requant(codes, cs, scales, ss, N, n, G, fi, fo, want_sum=True)
                st_c = np.zeros(n, np.uint8)
                st_s = np.zeros(oracle.n_blocks(n, G), np.float32)
                for _ in range(3):
                    g = (x * rng.random()).view(np.uint32) >> 16
                    st_c, st_s = oracle.fp8_accum_requant(st_c, st_s, g.astype(np.uint16), "bf16", G)
        xb = (rng.standard_normal(2 * 4 * 40) * 1e-3).astype(np.float16)
        oracle.reorder_quantize(xb, "f16", 2, 4, 32, "int4")
        for t in range(0, 101):
            oracle.aquavit_level(t, 100)
        print("calls ok", flush=True)
""")


def run_sanitized(lib, script):
    env = dict(os.environ, LD_PRELOAD=oracle_build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    code = f"ROOT = {ROOT!r}\nLIB = {lib!r}\n" + script
    return subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                          timeout=600)


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("san") / "liboracle_san.so")
    return oracle_build.build(sanitize=True, out=out)


def test_oracle_clean_under_asan_and_ubsan(sanitized_lib):
    r = run_sanitized(sanitized_lib, CALLS)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "pins ok 25" in r.stdout and "calls ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_sanitizer_catches_a_planted_overflow(tmp_path):
    src = open(oracle_build.SRC, encoding="utf-8").read()
    stmt = "memset(codes, 0, (size_t)((n * b + 7) / 8));"
    assert stmt in src
    bad = tmp_path / "qcp_oracle_bad.c"
    bad.write_text(src.replace(stmt, "memset(codes, 0, (size_t)((n * b + 7) / 8) + 1);"))
    lib = oracle_build.build(sanitize=True, out=str(tmp_path / "liboracle_bad.so"), src=str(bad))
    r = run_sanitized(lib, textwrap.dedent("""
        import sys
        import numpy as np
        sys.path.insert(0, ROOT)
        import oracle
        with oracle.loaded_from(LIB):
            oracle.quantize_blockwise(np.zeros(1000, np.float32), "f32", 128, "int4")
        print("no report", flush=True)
    """))
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stdout + r.stderr[-2000:]
