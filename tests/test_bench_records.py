"""The committed HBM traffic records (profiles/*.traffic.json) and bench.py's
lookup of them, on the CPU.

bench.py reports roofline.traffic from a record only when the record was
taken for the same launch (workload, launch mode, share plan, the
algorithmic bytes the roofline counts) and the decode kernel's sources still
hash to the record's SHA-256.  A record that the lookup cannot find leaves
traffic null in the bench line, so every committed record must be found
under its own key, and its figures must be the counters' scaled sum."""
import glob
import json
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RECORDS = sorted(glob.glob(os.path.join(ROOT, "profiles", "decode_mfma_balanced_*.traffic.json")))


def _records():
    for path in RECORDS:
        recs = json.load(open(path))
        for rec in recs if isinstance(recs, list) else [recs]:
            yield os.path.basename(path), rec


@pytest.mark.parametrize("name,rec", list(_records()),
                         ids=lambda x: x if isinstance(x, str) else f"{x['steps']}steps")
def test_record_is_found_for_its_launch(name, rec):
    assert name == f"decode_mfma_balanced_{rec['workload']}.traffic.json"
    got = bench.measured_traffic(rec["workload"], rec["partition"],
                                 rec["algorithmic_bytes_per_launch"], not rec["share_plan"])
    assert got == rec["hbm_bytes_per_launch"], (
        "the record does not match the current decode sources or its key: profile the "
        "kernel again (bench.py --traffic-record)")
    # another launch (other bytes, the other plan setting) finds nothing
    assert bench.measured_traffic(rec["workload"], rec["partition"],
                                  rec["algorithmic_bytes_per_launch"] + 1,
                                  not rec["share_plan"]) is None
    assert bench.measured_traffic(rec["workload"], rec["partition"],
                                  rec["algorithmic_bytes_per_launch"], rec["share_plan"]) is None


@pytest.mark.parametrize("name,rec", list(_records()),
                         ids=lambda x: x if isinstance(x, str) else f"{x['steps']}steps")
def test_record_figures_are_the_scaled_counters(name, rec):
    fetch = rec["fetch_size_kib_per_launch_raw"] * 1024 * rec["fetch_scale"]
    write = rec["write_size_kib_per_launch_raw"] * 1024 * rec["write_scale"]
    assert abs(fetch + write - rec["hbm_bytes_per_launch"]) <= 2048  # raw KiB rounded to 0.01
    cal = rec["copy_calibration"]
    gib_kib = (1 << 30) / 1024
    assert rec["fetch_scale"] == round(gib_kib / cal["fetch_size_kib"], 2)
    assert rec["write_scale"] == round(gib_kib / cal["write_size_kib"], 2)
    # traffic at or above the algorithmic bytes, and within 10% of them
    ratio = rec["hbm_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"]
    assert 1.0 <= ratio < 1.1, ratio
