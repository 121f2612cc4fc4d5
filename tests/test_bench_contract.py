"""Host-side checks of the benchmark's contract (no GPU): it refuses more than
one GPU with a JSON error line, and the HBM-traffic records under profiles/
that its roofline reads are well formed, name sources that exist, and are
used only for the kernel and the source bytes they were taken on."""
import glob
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

KERNELS = {"verify_attn_kernel", "verify_rows_kernel"}
RECORDS = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_verify_attn_*.json")))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_there_is_a_traffic_record_per_benchmark_workload():
    names = {json.load(open(p))["workload"] for p in RECORDS}
    from long_context_gqa_amd import workloads as W
    assert names == {wl.name for wl in W.WORKLOADS.values()}


@pytest.mark.parametrize("path", RECORDS, ids=[os.path.basename(p) for p in RECORDS])
def test_traffic_record_is_well_formed(path):
    rec = json.load(open(path))
    assert os.path.basename(path) == f"traffic_verify_attn_{rec['workload']}.json"
    assert rec["kernel"] in KERNELS
    for src in rec["sources"]:
        assert os.path.exists(os.path.join(ROOT, src)), src
    assert len(rec["source_sha256"]) == 64 and int(rec["source_sha256"], 16) >= 0
    assert rec["fetch_bytes_per_launch"] > 0 and rec["write_bytes_per_launch"] >= 0
    assert all(c.startswith("rocprofv3 --pmc ") and " -- python bench.py " in c for c in rec["commands"])
    # used for its own kernel while the sources hash to the record, never for another kernel
    h = hashlib.sha256()
    for src in rec["sources"]:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    want = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    got = bench.measured_traffic(path, rec["workload"], rec["kernel"])
    assert got == (want if h.hexdigest() == rec["source_sha256"] else None)
    other = (KERNELS - {rec["kernel"]}).pop()
    assert bench.measured_traffic(path, rec["workload"], other) is None


def test_a_changed_source_voids_the_record(tmp_path):
    rec = json.load(open(RECORDS[0]))
    rec["source_sha256"] = "0" * 64
    p = tmp_path / "rec.json"
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic(str(p), rec["workload"], rec["kernel"]) is None
