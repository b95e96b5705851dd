"""Every committed HBM-traffic record (profiles/traffic_*.json, written by
`bench.py --record-traffic` from rocprofv3 FETCH_SIZE / WRITE_SIZE runs) was
taken on the machine code the library builds now: its kernels' digests
equal those of the built libzs.so, so the benchmark reports its `traffic`
instead of null.  Also checks each record against its own arithmetic."""

import glob
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNELS = os.path.join(ROOT, "zero_sharded_optimizer_shard_amd",
                       "libzs.kernels.json")
RECORDS = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")))


def test_there_are_records():
    assert len(RECORDS) >= 8


@pytest.mark.parametrize("path", RECORDS, ids=os.path.basename)
def test_record_matches_the_built_kernels(path):
    if not os.path.exists(KERNELS):
        pytest.skip("library not built")
    built = json.load(open(KERNELS))
    rec = json.load(open(path))
    syms, want = rec["kernel_symbol"], rec["kernel_sha256_16"]
    if isinstance(syms, str):
        syms, want = [syms], [want]
    assert [built.get(s) for s in syms] == list(want), \
        f"{os.path.basename(path)}: counters taken on other machine code"


@pytest.mark.parametrize("path", RECORDS, ids=os.path.basename)
def test_record_arithmetic(path):
    rec = json.load(open(path))
    cal = rec["copy_calibration"]
    rs = cal["bytes_read"] / 1024 / cal["FETCH_SIZE_KiB"]
    ws = cal["bytes_written"] / 1024 / cal["WRITE_SIZE_KiB"]
    assert rs == pytest.approx(cal["read_scale"], rel=1e-12)
    assert ws == pytest.approx(cal["write_scale"], rel=1e-12)
    f, w = rec["FETCH_SIZE_KiB_per_launch"], rec["WRITE_SIZE_KiB_per_launch"]
    rd = sum(f) / len(f) * 1024 * rs
    wr = sum(w) / len(w) * 1024 * ws
    assert rd == pytest.approx(rec["bytes_read_per_launch"], rel=1e-9)
    assert wr == pytest.approx(rec["bytes_written_per_launch"], rel=1e-9)
    tot = rec["bytes_per_launch"]
    assert tot == pytest.approx(rd + wr, rel=1e-9)
    assert tot / rec["algorithmic_bytes_per_launch"] == pytest.approx(
        rec["ratio_to_algorithmic"], rel=1e-9)
    # every mode moves its algorithmic bytes within a small fraction
    assert abs(rec["ratio_to_algorithmic"] - 1) < 2e-3
