"""The rocprofv3 summariser: calibration against the 64 MiB copy, per-dispatch medians."""
import csv
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import profile_summary as P  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(path, counter, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": v})


def test_counters_are_scaled_by_the_copy(tmp_path):
    k = "void winattn::attn_decode_kernel<128, 4, 2, 256>(winattn::AttnParams)"
    copy_kib = 64 * 1024
    # FETCH_SIZE reads half of the copy; WRITE_SIZE all of it
    _write(str(tmp_path / "FETCH_SIZE" / "x_counter_collection.csv"), "FETCH_SIZE",
           [("other", 5.0), (P.COPY_KERNEL, copy_kib / 2), (k, 100.0), (k, 300.0), (k, 200.0)])
    _write(str(tmp_path / "WRITE_SIZE" / "x_counter_collection.csv"), "WRITE_SIZE",
           [(P.COPY_KERNEL, copy_kib), (k, 10.0), (k, 12.0), (k, 11.0)])
    data, (fcal, ff), (wcal, wf) = P.calibrated(str(tmp_path))
    assert ff == 2.0 and wf == 1.0
    n, fk, rb, wk, wb = data[k]
    assert n == 3 and fk == 200.0 and wk == 11.0
    assert rb == 200.0 * 1024 * 2 and wb == 11.0 * 1024
    doc = P.decode_json(str(tmp_path), str(tmp_path / "out.json"), "digest")
    assert doc["hbm_bytes_per_launch"] == int(rb + wb)
    assert doc["kernel_source_digest"] == "digest"


def test_mfma_utilisation(tmp_path):
    k = "void winattn::attn_mfma_kernel<128, false>(winattn::AttnParams)"
    path = str(tmp_path / "sq_counter_collection.csv")
    rows = []
    for inst, busy, gui in ((1000.0, 64000.0, 8000.0), (1000.0, 64000.0, 8000.0)):
        rows += [(k, "SQ_INSTS_VALU_MFMA_F32", inst), (k, "SQ_VALU_MFMA_BUSY_CYCLES", busy),
                 (k, "GRBM_GUI_ACTIVE", gui)]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i // 3, "Kernel_Name": name, "Counter_Name": c,
                        "Counter_Value": v})
    md = P.mfma_md(path, "t", {"attn_mfma_kernel": (4096.0, 2048000.0)})
    line = [ln for ln in md.splitlines() if "attn_mfma_kernel" in ln][0]
    cells = [c.strip() for c in line.split("|")]
    # busy 64000 over (8000 / 8 XCDs) x 1024 SIMDs; 1000 x 4096 flops over 2048000
    assert cells[2] == "2" and cells[6] == f"{64000 / (1000 * 1024):.3f}" and cells[7] == "2.000"
