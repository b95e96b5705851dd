"""The benchmark's host logic that needs no GPU: more than one GPU is
refused with a message and exit status 2, and rocprofv3 counter CSVs turn
into the traffic record as stated."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for n in (2, 8):
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                            "--gpus", str(n)], capture_output=True, text=True,
                           timeout=120)
        assert p.returncode == 2
        assert f"--gpus {n} is not supported" in p.stderr
        assert "one GPU" in p.stderr
        assert p.stdout == ""


def _counter_csv(path, counter, rows):
    """A rocprofv3 counter-collection CSV with the columns the bench reads."""
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (k, v) in enumerate(rows):
            f.write(f'{i},"{k}",{counter},{v}\n')


def test_record_traffic_scales_by_the_calibration_copy(tmp_path):
    """Bytes per launch = counter KiB x 1024 x (4 GiB / the counter's reading
    for the 4 GiB copy); only the tiled step's dispatches count."""
    sys.path.insert(0, ROOT)
    import bench
    W, n = 8, 1000
    step = "void (anonymous namespace)::step_kernel<8, true, Shape<64, 1, 8>, false>(StepArgs)"
    plain = "void (anonymous namespace)::step_kernel<8, false, Shape<64, 1, 8>, false>(StepArgs)"
    pure = "void (anonymous namespace)::step_kernel<8, true, Shape<64, 1, 8>, true>(StepArgs)"
    copy = "void k_copy16(...)"
    kib = 4 << 20                       # 4 GiB in KiB
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [(copy, kib / 2), (step, 10.0), (step, 14.0), (plain, 20.0),
                  (pure, 999.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [(copy, kib), (step, 5.0), (step, 5.0), (plain, 6.0),
                  (pure, 999.0)])
    rec = bench.record_traffic(str(tmp_path / "f.csv"),
                               str(tmp_path / "w.csv"), n, W, "llama8b",
                               out_path=str(tmp_path / "t.json"))
    assert rec["copy_calibration"]["read_scale"] == 2.0
    assert rec["bytes_read_per_launch"] == 12.0 * 1024 * 2
    assert rec["bytes_written_per_launch"] == 5.0 * 1024
    assert rec["algorithmic_bytes_per_launch"] == (2 * W + 26) * n
    assert rec["plain_slices"]["bytes_read_per_launch"] == 20.0 * 1024 * 2
    assert (tmp_path / "t.json").exists()


def test_record_traffic_sums_group_launches_per_full_step(tmp_path):
    """The streaming step's record is per full step: per_step consecutive
    group dispatches summed, the sums averaged; a partial step is refused."""
    sys.path.insert(0, ROOT)
    import bench
    import pytest
    W = 16
    grp = "void (anonymous namespace)::group_step_kernel<16, true, Shape<64, 1, 16>, false>(GroupArgs)"
    copy = "void k_copy16(...)"
    kib = 4 << 20
    f = [(copy, kib)] + [(grp, v) for v in (1, 2, 3, 3, 3, 3)]
    w = [(copy, kib)] + [(grp, 1.0)] * 6
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", f)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", w)
    rec = bench.record_traffic(str(tmp_path / "f.csv"),
                               str(tmp_path / "w.csv"), 100, W, "llama70b",
                               per_step=3, out_path=str(tmp_path / "t.json"))
    assert rec["FETCH_SIZE_KiB_per_launch"] == [6, 9]
    assert rec["bytes_read_per_launch"] == 7.5 * 1024
    assert rec["bytes_written_per_launch"] == 3.0 * 1024
    with pytest.raises(SystemExit):
        bench.record_traffic(str(tmp_path / "f.csv"),
                             str(tmp_path / "w.csv"), 100, W, "llama70b",
                             per_step=4, out_path=str(tmp_path / "u.json"))


def test_record_traffic_pure_bf16_counts_only_the_pure_step(tmp_path):
    """The <workload>_bf16 record takes the pure-bf16 step's dispatches
    (kernel names ending in `true>`) and 2W + 20 algorithmic bytes."""
    sys.path.insert(0, ROOT)
    import bench
    W, n = 8, 1000
    mixed = "void (anonymous namespace)::step_kernel<8, true, Shape<64, 1, 8>, false>(StepArgs)"
    pure = "void (anonymous namespace)::step_kernel<8, true, Shape<64, 1, 8>, true>(StepArgs)"
    copy = "void k_copy16(...)"
    kib = 4 << 20
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [(copy, kib), (mixed, 99.0), (pure, 3.0), (pure, 5.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [(copy, kib), (mixed, 99.0), (pure, 2.0), (pure, 2.0)])
    rec = bench.record_traffic(str(tmp_path / "f.csv"),
                               str(tmp_path / "w.csv"), n, W, "llama8b_bf16",
                               out_path=str(tmp_path / "t.json"))
    assert rec["bytes_read_per_launch"] == 4.0 * 1024
    assert rec["bytes_written_per_launch"] == 2.0 * 1024
    assert rec["algorithmic_bytes_per_launch"] == (2 * W + 20) * n


def test_record_traffic_accumulation_per_cycle(tmp_path):
    """The <workload>_accum record sums each cycle's two accumulation
    dispatches (first and last micro-batch) against 14 B per element, and
    keeps one digest per kernel; the gather record matches the plain
    function name the profiler gives it."""
    sys.path.insert(0, ROOT)
    import bench
    first = "void (anonymous namespace)::accum_kernel<0>(AccArgs)"
    last = "void (anonymous namespace)::accum_kernel<2>(AccArgs)"
    copy = "void k_copy16(...)"
    kib = 4 << 20
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [(copy, kib), (first, 2.0), (last, 6.0), (first, 2.0),
                  (last, 6.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [(copy, kib), (first, 4.0), (last, 2.0), (first, 4.0),
                  (last, 2.0)])
    rec = bench.record_traffic(str(tmp_path / "f.csv"),
                               str(tmp_path / "w.csv"), 1024, 8,
                               "llama8b_accum", per_step=2,
                               out_path=str(tmp_path / "t.json"))
    assert rec["bytes_read_per_launch"] == 8.0 * 1024
    assert rec["bytes_written_per_launch"] == 6.0 * 1024
    assert rec["algorithmic_bytes_per_launch"] == 14 * 1024
    assert isinstance(rec["kernel_symbol"], tuple) or \
        isinstance(rec["kernel_symbol"], list)
    gather = "(anonymous namespace)::gather_kernel((anonymous namespace)::GatherArgs)"
    _counter_csv(tmp_path / "gf.csv", "FETCH_SIZE",
                 [(copy, kib), (gather, 1.0), (gather, 3.0)])
    _counter_csv(tmp_path / "gw.csv", "WRITE_SIZE",
                 [(copy, kib), (gather, 1.0), (gather, 3.0)])
    rec = bench.record_traffic(str(tmp_path / "gf.csv"),
                               str(tmp_path / "gw.csv"), 1024, 8,
                               "llama8b_zero3", per_step=2,
                               out_path=str(tmp_path / "g.json"))
    assert rec["bytes_read_per_launch"] == 4.0 * 1024
    assert rec["algorithmic_bytes_per_launch"] == 4 * 1024
    # the whole-tensor gather's segment copies, not the flat gather's
    seg = ("(anonymous namespace)::copy_segments_kernel((anonymous "
           "namespace)::CopyArgs)")
    _counter_csv(tmp_path / "sf.csv", "FETCH_SIZE",
                 [(copy, kib), (gather, 9.0), (seg, 1.0), (seg, 1.0),
                  (seg, 2.0), (seg, 2.0)])
    _counter_csv(tmp_path / "sw.csv", "WRITE_SIZE",
                 [(copy, kib), (gather, 9.0), (seg, 2.0), (seg, 2.0),
                  (seg, 1.0), (seg, 1.0)])
    rec = bench.record_traffic(str(tmp_path / "sf.csv"),
                               str(tmp_path / "sw.csv"), 1024, 8,
                               "llama8b_zero3_tensors", per_step=2,
                               out_path=str(tmp_path / "s.json"))
    assert rec["FETCH_SIZE_KiB_per_launch"] == [2.0, 4.0]
    assert rec["bytes_read_per_launch"] == 3.0 * 1024
    assert rec["bytes_written_per_launch"] == 3.0 * 1024
    assert rec["algorithmic_bytes_per_launch"] == 4 * 1024
    assert "copy_segments_kernel" in rec["kernel"]
