"""bench.py's host logic, on the CPU: the rocprofv3 summary (per-kernel durations, the
back-to-back dominant-kernel launches, the per-layer call sites, counter scaling by the
plain copy) on synthetic CSV files, the algorithmic byte accounting, and the refusal to
run on more than one GPU."""
import csv
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _trace(path, seq):
    """A kernel-trace CSV with the dispatches (name, microseconds) back to back."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 1000
        for name, us in seq:
            w.writerow([name, t, t + int(us * 1000)])
            t += int(us * 1000) + 500


def test_summary_of_a_kernel_trace(tmp_path):
    layer = [("void pi::(anonymous namespace)::k_hidden_b1<1, 16, 1>(...)", 5.0),
             ("void pi::(anonymous namespace)::k_pred_fc1<1, 1, 16, false, 1, 64, true>(...)", 17.0),
             ("void pi::(anonymous namespace)::k_fc2_seg<1>(...)", 8.0),
             ("pi::(anonymous namespace)::k_reduce_y(...)", 4.0)]
    seq = layer * 10 + [layer[1]] * 5          # ten layer calls, then five isolated dominant launches
    d = tmp_path / "prof"
    d.mkdir()
    _trace(d / "run_kernel_trace.csv", seq)
    out = bench.rocprof_summary([str(d)], 256)
    rows = {l.split()[0]: l.split() for l in out.splitlines() if l.startswith("k_") and l.split()[1].isdigit()}
    assert rows["k_pred_fc1"][1] == "15" and float(rows["k_pred_fc1"][2]) == pytest.approx(17.0)
    assert rows["k_hidden_b1"][1] == "10"
    # four of the five isolated launches follow another k_pred_fc1
    iso = [l for l in out.splitlines() if l.startswith("k_pred_fc1 back-to-back")][0].split()
    assert iso[2] == "4"
    # the per-layer table: ten sequences closed by the ordered sum (the isolated launches after them
    # close no layer call)
    assert "per layer call (10 layer sequences of 4 kernels)" in out
    assert any(l.split()[:2] == ["2", "k_fc2_seg"] for l in out.splitlines())
    total = [l for l in out.splitlines() if l.strip().startswith("sum")][0].split()
    assert float(total[1]) == pytest.approx(34.0)


def test_batched_layer_call_sites(tmp_path):
    """A kernel launched twice per layer (the matrix-core row-dot for the hidden layer and FC1) is
    reported at both of its sites; setup kernels before the first call are not a layer call."""
    layer = [("k_mm_rowdot16<1, false, true>(...)", 5.0), ("k_mm_finish_tr<false>(...)", 4.0),
             ("k_mm_axpy16<1, true>(...)", 16.0), ("k_list(...)", 5.0), ("k_mm_rowdot16<1, false, false>(...)", 23.0),
             ("k_mm_finish_tr<false>(...)", 4.5), ("k_mm_axpy16<1, false>(...)", 20.0), ("k_reduce(...)", 4.0)]
    d = tmp_path / "prof"
    d.mkdir()
    _trace(d / "run_kernel_trace.csv", [("k_fill_dense(...)", 30.0)] * 3 + layer * 6)
    out = bench.rocprof_summary([str(d)], 256)
    assert "per layer call (5 layer sequences of 8 kernels)" in out
    sites = [l.split() for l in out.splitlines() if l[:4].strip().isdigit() and len(l.split()) == 4]
    assert [r[1] for r in sites if r[1] == "k_mm_rowdot16"] == ["k_mm_rowdot16"] * 2
    assert float([r for r in sites if r[0] == "4"][0][2]) == pytest.approx(23.0)
    total = [l for l in out.splitlines() if l.strip().startswith("sum")][0].split()
    assert float(total[1]) == pytest.approx(81.5)


def test_counter_scaling_by_the_plain_copy(tmp_path):
    d = tmp_path / "pmc"
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for _ in range(3):     # a 256 MiB copy reads as half its bytes
            w.writerow(["__amd_rocclr_copyBuffer", "FETCH_SIZE", 128 * 1024])
        w.writerow(["__amd_rocclr_copyBuffer", "FETCH_SIZE", 10.0])    # a small copy: not the reference
        for _ in range(4):
            w.writerow(["void pi::(anonymous namespace)::k_pred_fc1<...>(...)", "FETCH_SIZE", 31000.0])
    out = bench.rocprof_summary([str(d)], 256)
    assert "scale 2.0000" in out
    line = [l for l in out.splitlines() if l.strip().startswith("k_pred_fc1")][0]
    assert f"{31000.0 * 2 * 1024 / 1e6:9.3f} MB" in line


def test_memory_side_latency_and_translation_summary(tmp_path):
    d = tmp_path / "pmc"
    d.mkdir()
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(hdr)
        # the streaming read: 1000 reads in 10 us waiting 2000 cycles each; the kernel: 400 reads in
        # 10 us waiting 1000 cycles each -> 0.2 times the reads in flight
        for disp, (k, req, lev) in enumerate([("k_read_probe", 1000, 2.0e6), ("k_pred_fc1<...>(...)", 400, 4.0e5)]):
            for c, v in (("TCC_EA0_RDREQ_sum", req), ("TCC_EA0_RDREQ_LEVEL_sum", lev),
                         ("TCP_UTCL1_REQUEST_sum", 10000), ("TCP_UTCL1_TRANSLATION_MISS_sum", 25)):
                w.writerow([disp, f"void pi::(anonymous namespace)::{k}", c, v, 1000, 11000])
    out = bench.rocprof_summary([str(d)], 256)
    line = [l for l in out.splitlines() if l.strip().startswith("k_pred_fc1") and "cycles each" in l][0]
    assert "1000 cycles each" in line and "40 per us" in line and "0.20 x the streaming read's" in line
    tl = [l for l in out.splitlines() if l.strip().startswith("k_pred_fc1") and "misses" in l][0]
    assert "(0.2500%)" in tl


def test_layer_bytes_count_what_the_method_reads():
    cfg = synth.CONFIGS["opt-30b"]
    spec = synth.layer_spec(cfg, 0)
    d, N, H = cfg.d, cfg.N, spec.H
    pred, ffn, small = bench.layer_bytes(spec, 1, 2000, 400, 512, 1000)
    assert pred == H * d * 2 + 512 * N * 2 + N * 2           # P1, the P2 rows read, c2
    assert ffn == 2000 * (d * 2 + 2) + 1000 * d * 2           # FC1 rows + b1, FC2 rows with a != 0
    # a denser read (every P2 row, every listed W2 row) is strictly more
    p2, f2, _ = bench.layer_bytes(spec, 1, 2000, 400, H, 2000)
    assert p2 > pred and f2 > ffn and small > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_digest_follows_code_not_comments():
    """The counter digest: a comment edit leaves it, a code edit changes it, and the committed
    traffic figure is the committed summary's while the code is that of the passes."""
    src = "// header\nint f(int a) {  /* two\n lines */\n  return a + 1;   // note\n}\n"
    same = "// another header\n\nint f(int a) {\n  return a + 1;\n}\n"
    other = "int f(int a) {\n  return a + 2;\n}\n"
    assert bench.code_text(src) == bench.code_text(same)
    assert bench.code_text(src) != bench.code_text(other)
    assert "return a + 1;" in bench.code_text(src) and "note" not in bench.code_text(src)
    with open(os.path.join(ROOT, bench.TRAFFIC_PROFILE)) as fh:
        recorded = [l.split(":", 1)[1].strip() for l in fh if l.startswith("kernel sources sha256: ")][-1]
    if recorded == bench.kernel_source_digest():
        assert bench.committed_traffic(bench.DOMINANT) is not None
