"""Host logic of bench.py (CPU only): the algorithmic byte counts, the counter
summary that turns rocprofv3 --pmc runs into per-kernel HBM bytes, and the
one-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_of_the_workloads():
    # qwZ Llama-3-8B layer, INT8 G=256: 2 B in, 1 B of code, one fp32 scale per 256
    assert bench.bytes_codec(218_103_808, 2, 8, 256) == 218_103_808 * 3 + 4 * 851_968
    # Aquavit (2,1024) and (8,32) on 8192 x 28672
    n = 8192 * 28672
    assert bench.bytes_codec(n, 2, 2, 1024) == 2 * n + n // 4 + 4 * (n // 1024) == 529_399_808
    assert bench.bytes_codec(n, 2, 8, 32) == 734_003_200
    # qgZ: 8 INT4 slices of 62.5M in, one out, fp32 scales per 512
    nb = -(-62_500_000 // 512)
    assert bench.bytes_reduce(8, 62_500_000, 4, 4, 512) == 9 * (31_250_000 + 4 * nb) == 285_644_556
    # AGoQ accumulate: state in + out, bf16 gradient, scales in + out
    assert bench.bytes_accum(369_098_752, 128) == 369_098_752 * 4 + 8 * 2_883_584 == 1_499_463_680
    # a short last block counts as a block
    assert bench.nblk(257, 256) == 2 and bench.nblk(0, 256) == 0


HDR = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
       "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
       "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
       "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write_run(d, seq, counters):
    """seq: [(kernel name, grid, duration ns)]; counters: name -> f(index) value."""
    os.makedirs(d)
    t = 1000
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HDR)
        for i, (name, grid, ns) in enumerate(seq, start=1):
            for cname, fn in counters.items():
                w.writerow([i, i, 1, 1, 1, 1, grid, 7, name, 256, 0, 0, 32, 0, 48, cname,
                            fn(i - 1), t, t + ns])
            t += ns + 500


def test_counter_summary_labels_contexts_and_bytes(tmp_path):
    enc = "void qcp::k_encode<2, 8, 256>(void const*, long, long, unsigned char*, float*)"
    dec = "void qcp::k_decode<8, 2, 256>(unsigned char const*, float const*, long, long, void*)"
    setup = "void qcp::k_encode<1, 4, 512>(void const*, long, long, unsigned char*, float*)"
    nxt = "void qcp::k_encode_reorder<1, 4, 512>(void const*, long, long, long, long, double)"
    flush = "void at::native::reduce_kernel<512, 1, at::native::ReduceOp<float> >(...)"
    mul = "void at::native::vectorized_elementwise_kernel<4, MulFunctor<float> >(...)"
    W, K, R = 1, 2, 2
    seq = [(setup, 1000, 10)] * 3
    seq += [(enc, 6_815_744, 100), (dec, 6_815_744, 90)] * (W + 2 * K)        # indexes 3..12
    # each step kernel alone: one warm launch, then R after the flush read
    seq += [(enc, 6_815_744, 100)] + [(flush, 4096, 300), (enc, 6_815_744, 95)] * R   # 13..17
    seq += [(dec, 6_815_744, 90)] + [(flush, 4096, 300), (dec, 6_815_744, 85)] * R    # 18..22
    # a row beyond the step, same kernel and grid as a step kernel: labelled by position
    seq += [(enc, 6_815_744, 100)] + [(flush, 4096, 300), (enc, 6_815_744, 95)] * R   # 23..27
    seq += [(enc, 6_815_744, 100)] * (1 + R)                                          # 28..30
    seq += [(nxt, 61_040 * 256, 200)] * 2                  # after the labelled blocks: unlabelled
    seq += [(mul, 1 << 26, 400)]
    # reads: 4 requests of 128 B, 2 of 64 B, 1 of 32 B per dispatch index i -> 672 * (i + 1) B
    rd = {"TCC_EA0_RDREQ_128B_sum": lambda i: 4 * (i + 1), "TCC_EA0_RDREQ_64B_sum": lambda i: 2 * (i + 1),
          "TCC_EA0_RDREQ_32B_sum": lambda i: i + 1, "TCC_EA0_RDREQ_sum": lambda i: 7 * (i + 1)}
    # writes: 3 requests, one of them 64 B -> 128 B per dispatch
    wr = {"TCC_EA0_WRREQ_sum": lambda i: 3, "TCC_EA0_WRREQ_64B_sum": lambda i: 1}
    _write_run(str(tmp_path / "r"), seq, rd)
    _write_run(str(tmp_path / "w"), seq, wr)
    log = tmp_path / "bench.log"
    log.write_text("noise line\n" + json.dumps({
        "warmup": W, "steps": K, "cold_reps": R,
        "kernels": [{"kernel": "quantize(x)", "bytes": 1000, "cold": {}},
                    {"kernel": "dequantize(x)", "bytes": 2000, "cold": {}}],
        "next_rows": [{"kernel": "stress(x)", "bytes": 5000}]}) + "\n")
    out = tmp_path / "traffic.json"
    bench.summarize_counters([str(tmp_path / "r"), str(tmp_path / "w")], str(log), str(out))
    rec = json.loads(out.read_text())
    assert rec["source_hash"] == bench.kernel_source_hash()
    assert rec["copy_calibration"]["write_bytes"] == 128
    assert rec["copy_calibration"]["read_bytes"] == 672 * len(seq)
    rows = {(r["kernel"], r["context"]): r for r in rec["kernels"]}
    assert set(rows) == {("quantize(x)", "warm"), ("quantize(x)", "cold"), ("dequantize(x)", "warm"),
                         ("dequantize(x)", "cold"), ("stress(x)", "warm"), ("stress(x)", "cold")}

    def mean_read(idx):
        return round(sum(672 * (i + 1) for i in idx) / len(idx))
    q = rows[("quantize(x)", "warm")]
    assert q["launches"] == 6 and q["read_bytes"] == mean_read([3, 5, 7, 9, 11, 13])
    assert q["write_bytes"] == 128 and q["algorithmic_bytes"] == 1000
    assert q["traffic_over_algorithmic"] == round(q["hbm_bytes_per_launch"] / 1000, 4)
    c = rows[("quantize(x)", "cold")]
    assert c["launches"] == 2 and c["read_bytes"] == mean_read([15, 17]) and c["avg_us"] == round(95 / 1e3, 2)
    assert rows[("dequantize(x)", "warm")]["launches"] == 6
    assert rows[("dequantize(x)", "cold")]["read_bytes"] == mean_read([20, 22])
    st = rows[("stress(x)", "warm")]
    assert st["launches"] == 4 and st["algorithmic_bytes"] == 5000
    assert st["read_bytes"] == mean_read([23, 28, 29, 30])
    assert rows[("stress(x)", "cold")]["launches"] == 2


def test_counter_runs_must_launch_the_same_sequence(tmp_path):
    a = [("void qcp::k_encode<2, 8, 256>(...)", 64, 10)]
    b = [("void qcp::k_decode<8, 2, 256>(...)", 64, 10)]
    _write_run(str(tmp_path / "a"), a, {"TCC_EA0_RDREQ_sum": lambda i: 1})
    _write_run(str(tmp_path / "b"), b, {"TCC_EA0_WRREQ_sum": lambda i: 1})
    with pytest.raises(SystemExit):
        bench.load_counter_runs([str(tmp_path / "a"), str(tmp_path / "b")])


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
