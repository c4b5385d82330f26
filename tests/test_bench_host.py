"""Host logic of bench.py that needs no GPU.

* More than one GPU is refused with a message, before anything touches a
  GPU (every run here uses one GPU; several is a design note only).
* HBM traffic from rocprofv3 counters: FETCH_SIZE and WRITE_SIZE (KiB per
  dispatch) of the pass kernel, each scaled by what the same counter reads
  for the calibration copy of 1 GiB, the pass value being the median of its
  last eight dispatches.  Checked on synthetic counter files whose answer is
  known by construction (the copy's fetch counter reads half of its bytes,
  as it does on the device), written to a temporary file, not the committed
  record."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

GIB_KIB = float(1 << 20)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})
        w.writerow({"Kernel_Name": "void sv::k_pass<0, false, false>(sv::PassP)", "Counter_Name": "OTHER",
                    "Counter_Value": 1e12})


def test_traffic_from_counters(tmp_path, monkeypatch):
    # the copy reads 1 GiB and writes 1 GiB; its fetch counter shows half
    copy_fetch, copy_write = GIB_KIB / 2, GIB_KIB
    # pass dispatches: prefill-like outliers first, then the timed ones; the
    # median of the last eight is 13 GiB of counted fetch (6.5 GiB raw) and
    # 0.75 GiB written
    f_rows = [("void sv::k_pass<0, false, false>(sv::PassP)", 99 * GIB_KIB)] * 3
    f_rows += [("void sv::k_pass<0, false, false>(sv::PassP)", v * GIB_KIB) for v in
               (6.4, 6.5, 6.5, 6.6, 6.5, 6.3, 6.7, 6.5)]
    f_rows += [("__amd_rocclr_copyBuffer", copy_fetch), ("sv::k_accept(sv::AcceptParams)", 5.0)]
    w_rows = [("void sv::k_pass<0, false, false>(sv::PassP)", 0.75 * GIB_KIB)] * 10
    w_rows += [("__amd_rocclr_copyBuffer", copy_write)]
    fc, wc = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write(fc, "FETCH_SIZE", f_rows)
    _write(wc, "WRITE_SIZE", w_rows)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.traffic_from(str(fc), str(wc), "bench.py --traffic-from fetch.csv write.csv")
    t = json.loads(out.read_text())
    want = (13.0 + 0.75) * (1 << 30)
    assert abs(t["per_launch_bytes"]["pass"] - want) <= 1
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["pass_sources_sha256_16"] == bench.source_digest(bench.PASS_SOURCES)
