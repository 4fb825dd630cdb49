"""Host-side checks of bench.py's contract (no GPU): the one-GPU refusal,
and that the HBM traffic it reports comes only from a counter summary taken
on the same kernel source, workload and history path."""

import importlib.util
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True, text=True,
                       env=dict(os.environ, **env), timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line


def test_traffic_only_from_a_matching_counter_summary(tmp_path, monkeypatch):
    bench = _bench()
    src = tmp_path / "segment_causal_dit_amd" / "csrc"
    src.mkdir(parents=True)
    shutil.copy(os.path.join(ROOT, "segment_causal_dit_amd", "csrc", "attn.hip"), src / "attn.hip")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    cfg = bench.workloads.CONFIGS["c4"]
    path = bench.history_path(cfg)
    summary = {"workload": "c4", "attn_source_sha": bench.attn_source_hash(), "history_path": path,
               "hbm_bytes_per_launch": 1.5e10}
    out = tmp_path / "profiles" / "attn_c4_counters.json"
    out.write_text(json.dumps(summary))
    assert bench.measured_traffic(cfg, path) == 1.5e10
    assert bench.measured_traffic(cfg, "int8 cache") is None            # another history path
    out.write_text(json.dumps(dict(summary, attn_source_sha="0" * 16)))
    assert bench.measured_traffic(cfg, path) is None                    # taken on another kernel
    (src / "attn.hip").write_text("// changed\n")
    out.write_text(json.dumps(summary))
    assert bench.measured_traffic(cfg, path) is None                    # the kernel changed since
    out.write_text("not json")
    assert bench.measured_traffic(cfg, path) is None


def test_committed_counter_summary_is_consistent():
    with open(os.path.join(ROOT, "profiles", "attn_c4_counters.json")) as f:
        s = json.load(f)
    assert s["workload"] == "c4" and s["kernel"] == "attn_kernel"
    assert s["hbm_bytes_per_launch"] == pytest.approx(s["fetch_bytes_per_launch"] + s["write_bytes_per_launch"])
    cal = s["calibration"]
    assert cal["fetch_scale"] == pytest.approx(cal["copy_bytes"] / 1024.0 / cal["fetch_kib_read"])
    assert cal["write_scale"] == pytest.approx(cal["copy_bytes"] / 1024.0 / cal["write_kib_read"])
    assert any("FETCH_SIZE" in c for c in s["commands"]) and any("WRITE_SIZE" in c for c in s["commands"])
