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


@pytest.mark.gpu
def test_bench_all_ranks_reports_both_split_modes():
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    print("[bench balance] prefill_t8000_cp8, every rank, both split modes", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload",
                        "prefill_t8000_cp8", "--all-ranks", "--steps", "2", "--warmup", "1",
                        "--settle-ms", "0", "--cpu-seconds", "0"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=400)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads([l for l in r.stdout.splitlines() if l.strip()][-1])
    bal = d["rank_balance"]
    assert set(bal) == {"round-robin", "in-seq"}
    for mode, b in bal.items():
        assert b["split"] == mode
        assert len(b["ms_per_step"]) == 8 and all(t > 0 for t in b["ms_per_step"])
        assert b["queries"] == [1000] * 8
        mean = sum(b["ms_per_step"]) / 8
        assert b["spread"] == pytest.approx((max(b["ms_per_step"]) - min(b["ms_per_step"])) / mean,
                                            abs=2e-4)
    # causal pairs per rank, in closed form: round-robin rank r has
    # sum_j (r + 8j + 1); the in-sequence split's rank r sum_{p=1000r}^{1000r+999} (p + 1)
    rr_pairs = [sum(r + 8 * j + 1 for j in range(1000)) for r in range(8)]
    is_pairs = [(1000 * r + 1000) * (1000 * r + 1001) // 2 - (1000 * r) * (1000 * r + 1) // 2
                for r in range(8)]
    assert bal["round-robin"]["indexer_pairs"] == rr_pairs
    assert bal["in-seq"]["indexer_pairs"] == is_pairs
    # the contiguous split leaves rank 7 with 15x rank 0's indexer work
    assert bal["in-seq"]["spread"] > bal["round-robin"]["spread"]
