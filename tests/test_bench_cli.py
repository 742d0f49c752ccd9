"""bench.py's command-line contract on the host: one JSON line, a refusal of
more than one GPU, and the host-only prefix-cache component (no GPU)."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=timeout, cwd=ROOT)


def test_more_than_one_gpu_is_refused_for_every_component():
    for extra in ([], ["--component", "swap"], ["--component", "prefix_cache"], ["--component", "allocator"]):
        r = _bench("--gpus", "2", *extra)
        assert r.returncode == 2, (extra, r.stdout, r.stderr)
        assert "measures one GPU" in r.stderr
        assert r.stdout.strip() == ""


def test_prefix_cache_component_prints_one_json_line():
    r = _bench("--component", "prefix_cache", "--no-cpu", "--steps", "300")
    assert r.returncode == 0, r.stderr
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config"):
        assert key in rec, key
    assert rec["value"] > 0 and rec["higher_is_better"] is True and "workload" in rec["config"]
    # every request but the first finds the shared prompt's full blocks cached
    assert 0.5 < rec["prefill_tokens_saved_frac"] < 1.0


def test_allocator_component_prints_one_json_line():
    r = _bench("--component", "allocator")
    assert r.returncode == 0, r.stderr
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    assert rec["unit"] == "ns/block" and rec["value"] > 0 and rec["higher_is_better"] is False
    assert rec["cpu_baseline"]["kind"] == "oracle" and rec["cpu_baseline"]["value"] > rec["value"]
    assert "cpu_model" in rec["cpu_baseline"]["host"] and len(rec["pages"]) == 2
