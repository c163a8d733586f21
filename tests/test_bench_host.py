"""Host-side logic of bench.py, on the CPU: the one-GPU refusal, the split of a
kernel trace into per-leg runs, and the gate that reports HBM traffic only
while the committed counter profile matches the kernel sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _trace(path, dispatches):
    cols = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"]
    with open(path, "w") as fh:
        fh.write(",".join(f'"{c}"' for c in cols) + "\n")
        t = 1000
        for i, (name, grid, us) in enumerate(dispatches):
            fh.write(f'"KERNEL_DISPATCH",{i},"{name}(int, float)",{t},{t + int(us * 1000)},{grid}\n')
            t += int(us * 1000) + 500


def test_trace_runs(tmp_path, capsys):
    # three legs: 6 launches of kernel a, 2 of a copy (below the 5-call floor),
    # 5 of kernel a at another grid, 6 of kernel a again: four runs, three shown
    d = [("void a<1>", 256, 10.0)] * 5 + [("void a<1>", 256, 14.0)] + [("copy", 64, 1.0)] * 2
    d += [("void a<1>", 512, 20.0)] * 5 + [("void a<1>", 256, 12.0)] * 6
    p = tmp_path / "trace.csv"
    _trace(p, d)
    bench.summarize_trace_runs(str(p))
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("|")]
    assert len(lines) == 3
    first = [c.strip() for c in lines[0].split("|")[1:-1]]
    assert first[0] == "0" and first[1] == "`void a<1>`" and first[2] == "256" and first[3] == "6"
    assert float(first[4]) == pytest.approx((5 * 10.0 + 14.0) / 6, abs=0.01)
    assert float(first[6]) == pytest.approx(10.0, abs=0.01)
    assert [l.split("|")[1].strip() for l in lines] == ["0", "2", "3"]
    assert lines[1].split("|")[3].strip() == "512"


def test_traffic_gate(tmp_path, monkeypatch):
    # the committed profile is read only while its source hash matches
    h = bench.kernel_source_hash()
    blob = {"kernel_source_hash": h, "hbm_bytes_per_launch": 123}
    p = tmp_path / "traffic.md"
    p.write_text("# profile\n\n```json\n" + json.dumps(blob) + "\n```\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(p))
    assert bench.load_traffic(h) == 123
    assert bench.load_traffic("0" * 16) is None
    p.write_text("no json block here")
    assert bench.load_traffic(h) is None
