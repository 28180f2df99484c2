"""Host logic of bench.py that decides what its JSON line reports (CPU only)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _summary(tmp_path, workload, config, sha, traffic=1.5e10):
    p = tmp_path / f"fa_prefill_sparse_{workload}.md"
    p.write_text("\n".join([
        "# summary", "", "## Values read by bench.py", "",
        f"workload: {workload}",
        f"config: {json.dumps(config, sort_keys=True)}",
        f"source_sha256: {sha}",
        f"traffic_bytes_per_launch: {traffic}",
        "avg_duration_ms: 70.0", ""]))
    return p


CFG = {"workload": "w: a layer", "gamma": 0.95, "seq_len": 131072, "score_stride": 1,
       "skip_threshold": 0.0, "budget": {"mode": "dynamic", "last_blocks": 1},
       "input_sha256_16": "0123456789abcdef"}


def test_traffic_is_read_only_for_the_same_workload_config_and_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    sha = bench.kernel_source_hash()
    _summary(tmp_path, "w", CFG, sha, 4.9e10)
    assert bench.profiled_traffic("w", dict(CFG)) == pytest.approx(4.9e10)
    # another gamma, stride, budget or input is another workload for the counters
    for key, val in (("gamma", 0.8), ("score_stride", 2), ("input_sha256_16", "f" * 16),
                     ("budget", {"mode": "fixed", "fixed_blocks": 64})):
        other = dict(CFG)
        other[key] = val
        assert bench.profiled_traffic("w", other) is None, key
    # a summary of other workloads or other kernel sources is never used
    assert bench.profiled_traffic("v", dict(CFG)) is None
    _summary(tmp_path, "w", CFG, "0" * 64)
    assert bench.profiled_traffic("w", dict(CFG)) is None


def test_missing_or_malformed_summary_gives_null(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench.profiled_traffic("w", dict(CFG)) is None
    p = _summary(tmp_path, "w", CFG, bench.kernel_source_hash())
    p.write_text(p.read_text().replace("traffic_bytes_per_launch: 15000000000.0",
                                       "traffic_bytes_per_launch: n/a"))
    assert bench.profiled_traffic("w", dict(CFG)) is None


def test_committed_profiles_name_their_workload_and_hash_the_kernel_sources():
    prof = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(prof) if n.startswith("fa_prefill_sparse_")]
    assert names, "no sparse-attention profile committed"
    for n in names:
        kv = {}
        for line in open(os.path.join(prof, n)).read().splitlines():
            if ":" in line:
                k, v = line.split(":", 1)
                kv.setdefault(k.strip(), v.strip())
        assert kv.get("workload") == n[len("fa_prefill_sparse_"):-3], n
        assert len(kv.get("source_sha256", "")) == 64, n
        json.loads(kv["config"])
        assert float(kv["traffic_bytes_per_launch"]) > 0


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


def test_sparse_attention_kernel_names_are_recognised():
    assert bench._is_sparse_attention("void pxa::fa_prefill_kernel<128, false, false>(__bf16 const*)")
    assert bench._is_sparse_attention("void pxa::fa_prefill_kernel<64, false, true>(x)")
    assert not bench._is_sparse_attention("void pxa::fa_prefill_kernel<128, true, false>(x)")
    assert not bench._is_sparse_attention("void pxa::proxy_score_kernel<128, 1, false>(x)")


def test_live_traffic_is_null_without_the_profiler(monkeypatch):
    import shutil
    monkeypatch.setattr(shutil, "which", lambda name: None)
    a = bench.argparse.Namespace(workload="w", budget="dynamic:1", score_stride=1, skip_threshold=0.0,
                                 gamma=None, seq_len=None)
    assert bench.live_traffic(a) is None
