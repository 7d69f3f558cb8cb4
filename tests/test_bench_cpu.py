"""Host-side checks of bench.py's contract (no GPU): the single-GPU refusal,
and that committed HBM-traffic measurements are used only for the kernel
sources they were taken on."""
import copy
import hashlib
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_more_than_one_gpu_is_refused(gpus):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_vendor_comparison_refuses_low_precision_layers():
    """The vendor grouped-GEMM comparison times bf16 products only; an fp8
    workload is refused before anything touches a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "deepseek_v3_fp8",
                        "--vendor-grouped-mm"], capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "bf16" in r.stderr
    assert r.stdout == ""


def test_traffic_is_used_only_for_the_measured_sources(tmp_path):
    bench = _bench_module()
    # a private tree: one kernel source and a traffic record for it
    csrc = tmp_path / "routing_grouped_gemm_router_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = b"// kernel source\n"
    (csrc / "k.hip").write_bytes(src)
    rec = {"sources": ["k.hip"], "sha256": hashlib.sha256(src).hexdigest(),
           "bytes_per_launch": 12345}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps({"w/k": rec}))
    bench.ROOT = str(tmp_path)
    assert bench.traffic_for("w", "k") == 12345
    assert bench.traffic_for("w", "other") is None
    # the source changes after the measurement: the figure is no longer used
    (csrc / "k.hip").write_bytes(src + b"// changed\n")
    assert bench.traffic_for("w", "k") is None
    # a record for a different source text
    stale = copy.deepcopy(rec)
    stale["sha256"] = "0" * 64
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps({"w/k": stale}))
    (csrc / "k.hip").write_bytes(src)
    assert bench.traffic_for("w", "k") is None


def test_committed_traffic_records_are_well_formed():
    path = os.path.join(ROOT, "profiles", "traffic.json")
    recs = json.load(open(path))
    assert recs, "no traffic records"
    for key, rec in recs.items():
        workload, kernel = key.split("/")
        assert workload and kernel
        assert rec["bytes_per_launch"] > 0
        assert len(rec["sha256"]) == 64
        for s in rec["sources"]:
            assert os.path.exists(os.path.join(ROOT, "routing_grouped_gemm_router_amd", "csrc", s)), s
