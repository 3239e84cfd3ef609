"""The benchmark's host-side contract, on the CPU: it measures one GPU and refuses more,
its CPU baseline times the oracle on a bounded sample, and the HBM traffic it reports is
taken only from a profile of the current kernel sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _run_bench(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused_with_a_message(args, env):
    r = _run_bench(args, env)
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_times_the_oracle_on_a_bounded_sample():
    import bench
    from kronecker_factored_transforms_amd import synth as S
    for name, bits in (("hidden_n8192", 4), ("hidden_n8192", 8), ("kv_h8_d128", 4)):
        inp = S.make(name, T=96)
        cb = bench.cpu_baseline(inp, 0.3, bits)
        assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s"
        assert cb["value"] > 0 and cb["cores"] >= 1
        assert "tokens of the same workload" in cb["sample"]
        json.dumps(cb)


def test_traffic_is_reported_only_for_the_current_kernel_sources(tmp_path, monkeypatch):
    import bench
    assert bench.traffic_from_profile("no_such_workload", "no_such_kernel") is None
    # a summary whose source hash differs from the current sources is ignored
    prof = tmp_path / "profiles"
    prof.mkdir()
    body = "hbm_bytes_per_launch: 123456\nkernel_sources_sha256: {}\n"
    (prof / "traffic_k_w.md").write_text(body.format("0" * 64))
    current = bench.kernel_source_sha256()
    (prof / "traffic_k2_w.md").write_text(body.format(current))
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: current)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profile("w", "k") is None
    assert bench.traffic_from_profile("w", "k2") == 123456.0


def test_source_hash_ignores_comments_and_blank_lines():
    import bench
    code = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    same = "/* header\n   text */\nint f(int x) {\n\n  return x + 1;\n}  // end\n"
    other = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench._code_text(code) == bench._code_text(same)
    assert bench._code_text(code) != bench._code_text(other)
