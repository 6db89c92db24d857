"""Host-side logic of bench.py (no GPU): the rocprofv3 summary it writes
under profiles/, the kernel-source hash that ties a summary to the sources,
the one-GPU refusal and the decode-step grouping."""
import csv
import os
import shutil
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXPAND = "void lora::expand_kernel<lora::Bf16, true>(lora::KArgs)"
SHRINK = "void lora::shrink_kernel<lora::Bf16, true>(lora::KArgs)"
APPLY = "void lora::apply_kernel<lora::Bf16, true, true>(lora::KArgs)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(at::TensorIteratorBase&)>"


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_summary_scales_counters_by_the_calibration_copy(tmp_path, capsys):
    """FETCH_SIZE reading half the calibration copy's bytes gives a scale of
    2; WRITE_SIZE reading them exactly, 1; per-launch bytes follow."""
    d = tmp_path / "prof"
    d.mkdir()
    calib_kib = bench.CALIB_BYTES / 1024
    rows = []
    disp = 0
    for name, fetch, write in ((COPY, calib_kib / 2, calib_kib), (EXPAND, 1000.0, 300.0), (EXPAND, 3000.0, 500.0),
                               (SHRINK, 700.0, 10.0), (APPLY, 4000.0, 600.0)):
        disp += 1
        rows.append([disp, name, "FETCH_SIZE", fetch])
        rows.append([disp, name, "WRITE_SIZE", write])
    _write_csv(d / "run_counter_collection.csv", ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    bench.summarize_profile([str(d)], "rocprofv3 --pmc ... (test)")
    out = capsys.readouterr().out.splitlines()
    assert out[0] == "command: rocprofv3 --pmc ... (test)"
    assert out[1] == f"kernel_source_hash: {bench.kernel_source_hash()}"
    vals = dict(l.split(": ") for l in out if ": " in l and not l.startswith(("command", "kernel_source")))
    assert float(vals["fetch_size_scale"]) == pytest.approx(2.0)
    assert float(vals["write_size_scale"]) == pytest.approx(1.0)
    assert int(vals["expand_fetch_size_bytes_per_launch"]) == 2000 * 1024 * 2
    assert int(vals["expand_write_size_bytes_per_launch"]) == 400 * 1024
    assert int(vals["expand_hbm_bytes_per_launch"]) == 2000 * 2048 + 400 * 1024
    assert int(vals["shrink_hbm_bytes_per_launch"]) == 700 * 2048 + 10 * 1024
    assert int(vals["apply_hbm_bytes_per_launch"]) == 4000 * 2048 + 600 * 1024


def test_committed_summaries_are_read_back(tmp_path, monkeypatch):
    """The bench reads per-kernel durations and HBM bytes back from summaries
    written by summarize_profile, and ignores them under another kernel hash."""
    h = bench.kernel_source_hash()
    stats = tmp_path / "stats.txt"
    stats.write_text(f"command: x\nkernel_source_hash: {h}\nkernel stats (...):\n"
                     f"    calls     avg_us     min_us     max_us   total_ms    pct  name\n"
                     f"      128      88.50      20.00     150.00     11.328  90.00  {APPLY}\n"
                     f"      128      30.00      10.00      60.00      3.840  10.00  {SHRINK}\n")
    traffic = tmp_path / "traffic.txt"
    traffic.write_text(f"command: x\nkernel_source_hash: {h}\napply_hbm_bytes_per_launch: 350000000\n"
                       f"expand_hbm_bytes_per_launch: 200000000\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "STATS_SUMMARY", "stats.txt")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", "traffic.txt")
    st = bench.load_stats(h)
    assert st[bench.APPLY_KERNEL] == 88.5 and st[bench.SHRINK_KERNEL] == 30.0
    assert bench.load_traffic(h) == {"apply": 350000000, "expand": 200000000}
    assert bench.load_stats("0" * 16) is None and bench.load_traffic("0" * 16) is None


def test_config_summaries_give_traffic_over_algorithmic(tmp_path, monkeypatch):
    """A single-workload summary pair yields each kernel's mean launch, rate
    and counter bytes over algorithmic bytes; kernels absent from both are
    left out, and summaries under another kernel hash are not used."""
    h = bench.kernel_source_hash()
    (tmp_path / "s.txt").write_text(f"command: x\nkernel_source_hash: {h}\nkernel stats (...):\n"
                                    f"    calls     avg_us     min_us     max_us   total_ms    pct  name\n"
                                    f"       20      50.00      40.00      60.00      1.000  50.00  {SHRINK}\n")
    (tmp_path / "t.txt").write_text(f"command: x\nkernel_source_hash: {h}\nshrink_hbm_bytes_per_launch: 110000000\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "CONFIG_SUMMARIES", {3: ("s.txt", "t.txt")})
    got = bench.config_rocprof(3, {"apply": 1.0, "shrink": 100e6, "expand": 1.0})
    assert set(got) == {"stats_source", "traffic_source", "shrink"}
    assert got["shrink"] == {"mean_launch_us": 50.0, "gbs": 2000.0, "algorithmic_bytes_per_launch": 100000000,
                             "hbm_bytes_per_launch": 110000000, "hbm_over_algorithmic": 1.1}
    (tmp_path / "t.txt").write_text("command: x\nkernel_source_hash: 0000000000000000\n")
    assert bench.config_rocprof(3, {"apply": 1.0, "shrink": 100e6, "expand": 1.0})["traffic_source"] is None


def test_summary_of_kernel_stats_and_mfma_counters(tmp_path, capsys):
    d = tmp_path / "prof"
    d.mkdir()
    _write_csv(d / "x_kernel_stats.csv", ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs", "Percentage"],
               [[EXPAND, 4, 240000, 60000, 50000, 70000, 60.0], [COPY, 1, 160000, 160000, 160000, 160000, 40.0]])
    _write_csv(d / "m_counter_collection.csv", ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
               [[1, EXPAND, "MfmaUtil", 3.0], [2, EXPAND, "MfmaUtil", 4.0], [1, EXPAND, "MfmaFlopsBF16", 1e9]])
    bench.summarize_profile([str(d)], "")
    out = capsys.readouterr().out
    line = [l for l in out.splitlines() if EXPAND in l and "avg_us" not in l and "Mfma" not in l
            and not l.startswith("mfma")][0].split()
    assert line[:6] == ["4", "60.00", "50.00", "70.00", "0.240", "60.00"]
    assert f"mfma_util_pct 3.5  {EXPAND}" in out
    assert f"mfma_bf16_flops_per_dispatch 1e+09  {EXPAND}" in out
    assert "lora::" in out and "neg_kernel" not in out.split("kernel stats")[1].split("counters")[0]


def test_derived_counter_ratios():
    """Per-wave instruction counts, L2 read latency, credit-stall share, reads
    in flight per channel and hit rate, from the per-dispatch counter means
    of each kernel (two dispatches of the apply kernel averaged)."""
    per = {
        (APPLY, "SQ_WAVES"): {1: 3000.0, 2: 3000.0},
        (APPLY, "SQ_INSTS_VALU"): {1: 6.0e6, 2: 12.0e6},
        (APPLY, "SQ_INSTS_SALU"): {1: 3.0e6, 2: 3.0e6},
        (APPLY, "TCP_TCC_READ_REQ_LATENCY_sum"): {1: 2.0e9},
        (APPLY, "TCP_TCC_READ_REQ_sum"): {1: 1.0e6},
        (APPLY, "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum"): {1: 50.0},
        (APPLY, "TCC_EA0_RDREQ_LEVEL_sum"): {1: 1.0e7},
        (APPLY, "TCC_CYCLE_sum"): {1: 1.0e5},
        (APPLY, "TCC_HIT_sum"): {1: 600.0},
        (APPLY, "TCC_MISS_sum"): {1: 400.0},
        ("some::other_kernel()", "SQ_WAVES"): {1: 1.0},
    }
    got = {line.split()[0]: float(line.split()[1]) for line in bench.derived_counter_lines(per)}
    assert got == {"per_wave_salu": 1000.0, "per_wave_valu": 3000.0, "l2_read_latency_cycles": 2000.0,
                   "dram_credit_stall_share": 5e-4, "dram_reads_in_flight_per_channel": 100.0, "l2_hit_rate": 0.6}


def test_counter_read_in_two_runs_is_averaged_not_added(tmp_path, capsys):
    """Dispatch ids restart in every profiled run: SQ_WAVES read in two runs
    (dispatch 1 in each) averages to its value, and per-wave ratios use it."""
    for i, ctr in enumerate(("SQ_INSTS_VALU", "SQ_INSTS_SALU")):
        d = tmp_path / f"run{i}"
        d.mkdir()
        _write_csv(d / "r_counter_collection.csv", ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
                   [[1, APPLY, "SQ_WAVES", 3000.0], [1, APPLY, ctr, 6e6 * (i + 1)]])
    bench.summarize_profile([str(tmp_path / "run0"), str(tmp_path / "run1")], "")
    out = capsys.readouterr().out
    assert f"per_wave_valu 2000  {APPLY}" in out and f"per_wave_salu 4000  {APPLY}" in out


def test_per_cu_stall_shares(tmp_path, capsys):
    """Per-CU stall counters are summed over 256 CUs and GRBM_GUI_ACTIVE over
    8 XCDs: 256 CUs each stalled half of 1000 busy cycles read as 0.5."""
    _write_csv(tmp_path / "r_counter_collection.csv", ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
               [[1, APPLY, "GRBM_GUI_ACTIVE", 8 * 1000.0], [1, APPLY, "TCP_PENDING_STALL_CYCLES", 256 * 500.0],
                [1, APPLY, "TD_TD_BUSY", 256 * 250.0]])
    bench.summarize_profile([str(tmp_path)], "")
    out = capsys.readouterr().out
    assert f"tcp_pending_stall_share 0.5  {APPLY}" in out and f"td_busy_share 0.25  {APPLY}" in out


def test_only_byte_counters_are_calibrated(tmp_path, capsys):
    """Counters other than FETCH_SIZE / WRITE_SIZE read on the calibration
    copy are reported as read, never turned into bytes."""
    d = tmp_path / "prof"
    d.mkdir()
    _write_csv(d / "c_counter_collection.csv", ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
               [[1, COPY, "TCC_CYCLE_sum", 1e6], [2, APPLY, "TCC_CYCLE_sum", 5e5],
                [1, COPY, "TCC_HIT_sum", 10.0], [2, APPLY, "TCC_HIT_sum", 3.0]])
    bench.summarize_profile([str(d)], "")
    out = capsys.readouterr().out
    assert "_scale" not in out and "bytes_per_launch" not in out
    assert "TCC_CYCLE_sum" in out


def test_kernel_hash_ignores_comments_but_not_code(tmp_path):
    for rel in bench.KERNEL_SOURCES:
        os.makedirs(tmp_path / os.path.dirname(rel), exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), tmp_path / rel)
    h0 = bench.kernel_source_hash(str(tmp_path))
    assert h0 == bench.kernel_source_hash()
    first = tmp_path / bench.KERNEL_SOURCES[0]
    text = first.read_text()
    first.write_text("// a new comment line\n/* and a block\n comment */\n" + text.replace("\n", "\n  ", 3))
    assert bench.kernel_source_hash(str(tmp_path)) == h0
    first.write_text(text + "\nstatic int lora_extra_symbol = 1;\n")
    assert bench.kernel_source_hash(str(tmp_path)) != h0


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_layer_grouping_follows_the_block_dependencies():
    names = ["q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj"]
    g = bench.groups_for(2, names, "layer")
    assert g[:4] == [[0, 1, 2], [3], [4, 5], [6]]
    assert g[4:] == [[7, 8, 9], [10], [11, 12], [13]]
    assert sorted(i for grp in g for i in grp) == list(range(14))
    a = bench.groups_for(32, names, "all")
    assert all(len(grp) <= 16 for grp in a) and sum(len(grp) for grp in a) == 224
