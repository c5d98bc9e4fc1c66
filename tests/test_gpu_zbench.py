"""bench.py on the GPU: the one JSON line it prints keeps its contract."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_roofline_and_cpu_baseline():
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    print("[bench contract] default workload (65536-token fp8 prefill), 2 steps", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2",
                        "--warmup", "1", "--settle-ms", "20", "--cpu-seconds", "0.5"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=400)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    # whole-step throughput: queries per step over the measured step time
    n = d["config"]["queries"]
    assert d["value"] == pytest.approx(n / (d["ms_per_step"] * 1e-3), rel=2e-3)
    assert d["config"]["workload"] == "prefill_t65536_cp8_fp8"
    roof = d["roofline"]
    assert roof["bound"] in ("hbm", "mfma", "alu")
    assert roof["unit"] in ("GB/s", "TFLOP/s")
    assert 0 < roof["frac"] <= 1 and roof["peak"] > 0
    assert roof["achieved"] == pytest.approx(roof["frac"] * roof["peak"], rel=1e-2)
    # the own-KV cache write is measured after the timed region, outside the step
    for k in ("kv_cache_write(latent)", "kv_cache_write(indexer_k)"):
        w = d["outside_step"][k]
        assert w["avg_us"] > 0 and w["bytes"] > 0 and 0 < w["frac"] <= 1
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
