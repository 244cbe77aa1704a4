"""Host logic of bench.py (CPU only): the one-GPU guard, and the rule that a
committed traffic figure is used only while it was taken on the current
kernel source and workload."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _counters_file(tmp_path, path, workload, kernel_hash):
    rec = {"workload": workload, "kernel_hash": kernel_hash, "traffic_bytes_per_launch": 123456}
    f = tmp_path / f"{path}_counters.md"
    f.write_text("# summary\n\n```json\n" + json.dumps(rec, indent=1) + "\n```\n")
    return str(f)


def test_traffic_only_for_the_current_kernel_and_workload(tmp_path, monkeypatch):
    for path in ("compare", "record"):
        target = {}
        monkeypatch.setattr(bench, "counters_file", lambda w, p: target["file"])
        target["file"] = _counters_file(tmp_path, path, "corpus", bench.kernel_hash(path))
        traffic, src = bench.stored_traffic("corpus", path)
        assert traffic == 123456 and src.endswith(f"{path}_counters.md")
        assert bench.stored_traffic("stream", path) == (None, None)     # another workload
        target["file"] = _counters_file(tmp_path, path, "corpus", "0" * 16)
        assert bench.stored_traffic("corpus", path) == (None, None)     # another kernel source
        target["file"] = str(tmp_path / "missing.md")
        assert bench.stored_traffic("corpus", path) == (None, None)


def test_kernel_hash_covers_the_kernel_sources():
    h = bench.kernel_hash("compare")
    assert h == bench.kernel_hash("compare") and len(h) == 16
    assert h != bench.kernel_hash("record")
    for path in ("compare", "record"):
        for name in bench.PATHS[path]["sources"]:
            assert os.path.exists(os.path.join(ROOT, "logit_distribution_diffing_amd", "csrc", name))


def test_committed_profiles_name_their_kernel_sources():
    """Each committed counter summary carries the hash of some build of its
    kernel (it may lag the source until the next profiling run)."""
    for path in ("compare", "record"):
        text = open(bench.counters_file("corpus", path)).read()
        rec = json.loads(text.split("```json\n", 1)[1].split("\n```", 1)[0])
        assert rec["workload"] == "corpus" and len(rec["kernel_hash"]) == 16
        assert rec["traffic_bytes_per_launch"] > 0


def test_oracle_leg_reports_cores_cpu_and_single_core():
    """The CPU leg on a few tiny rows: thread count, CPU model, single-core figure."""
    import numpy as np
    import synth
    w = synth.WORKLOADS["tiny"]
    a, b = synth.tiny(w["seed"], 0, 16, w["v"])
    res = bench.cpu_leg(a, b, 20, synth.DEFAULT_EDGES, 0.05, single_core=True)
    assert res["kind"] == "oracle" and res["cores"] >= 1 and res["value"] > 0
    assert isinstance(res["cpu"], str) and res["cpu"]
    assert res["single_core"]["cores"] == 1 and res["single_core"]["value"] > 0
