"""Host logic of the counter summaries (no GPU): HBM bytes per launch from
FETCH_SIZE / WRITE_SIZE runs calibrated by a plain device copy, and the
kernel-source check that keeps a stale record out of the benchmark line."""
import csv
import json

from decode_megakernel_md_amd import profiling as P

FIELDS = ["Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, counter, copy_kib, mk_kib):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for v in copy_kib:
            w.writerow({"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter, "Counter_Value": v})
        for v in mk_kib:
            w.writerow({"Kernel_Name": "md_megakernel", "Counter_Name": counter, "Counter_Value": v})


def test_traffic_record_scales_by_the_copy(tmp_path):
    # the copy reads and writes 1 GiB = 1048576 KiB; a counter that reads half
    # of that for the copy counts 2 bytes per unit
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [262144.0, 262144.0], [1000.0, 3000.0])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [1048576.0], [10.0])
    rec = P.traffic_record(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "dense_27b", 1)
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["fetch_bytes"] == 2000.0 * 1024 * 2
    assert rec["write_bytes"] == 10.0 * 1024
    assert rec["bytes"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["kernel_sha256"] == P.kernel_source_hash()


def test_traffic_for_rejects_other_sources_and_workloads(tmp_path, monkeypatch):
    rec = {"workload": "dense_27b", "batch": 1, "kernel_sha256": P.kernel_source_hash(), "bytes": 5.0}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(P, "TRAFFIC_JSON", str(path))
    assert P.traffic_for("dense_27b", 1)["bytes"] == 5.0
    assert P.traffic_for("dense_27b", 8) is None
    assert P.traffic_for("hybrid_moe", 1) is None
    path.write_text(json.dumps(dict(rec, kernel_sha256="0" * 64)))
    assert P.traffic_for("dense_27b", 1) is None


def test_dispatch_gaps():
    """Idle time between back-to-back dispatches; a pause longer than 1 ms
    starts a new run and is not counted as a gap."""
    d = [(0, 100_000), (110_000, 200_000), (5_000_000, 5_000_100), (5_000_150, 5_000_300)]
    r = P.gaps(d)
    assert r["dispatches"] == 4 and r["runs"] == 2 and r["gaps"] == 2
    assert abs(r["busy_us"] - 190.25) < 1e-9
    assert abs(r["idle_us"] - 10.05) < 1e-9
    assert abs(r["max_gap_us"] - 10.0) < 1e-9


def test_traffic_records_per_workload_and_batch(tmp_path, monkeypatch):
    """Records of several (workload, batch) pairs live side by side; storing
    one replaces only the record of its own pair."""
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(P, "TRAFFIC_JSON", str(path))
    h = P.kernel_source_hash()
    P.store_traffic({"workload": "dense_27b", "batch": 1, "kernel_sha256": h, "bytes": 1.0})
    P.store_traffic({"workload": "hybrid_moe", "batch": 8, "kernel_sha256": h, "bytes": 2.0})
    P.store_traffic({"workload": "dense_27b", "batch": 1, "kernel_sha256": h, "bytes": 3.0})
    assert P.traffic_for("dense_27b", 1)["bytes"] == 3.0
    assert P.traffic_for("hybrid_moe", 8)["bytes"] == 2.0
    assert P.traffic_for("hybrid_moe", 1) is None
    assert len(json.loads(path.read_text())["records"]) == 2
