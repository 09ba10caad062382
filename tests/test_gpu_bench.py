"""bench.py's output contract on the GPU: one JSON line with the metric, the
dominant kernel's roofline (per-dispatch timing, every kernel of the stage,
the stage), the prefill and expert-cache blocks and the CPU baseline, at a
few steps of the default workload; and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=300):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=timeout, cwd=ROOT)
    return r


def test_bench_json_contract():
    print("bench: 30 decode steps, 2 prefill steps, 16-slot cache, 1 s of oracle", flush=True)
    r = _bench("--steps", "30", "--warmup", "3", "--prefill-steps", "2", "--cache-slots", "32",
               "--cache-steps", "4", "--cpu-seconds", "1")
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 30 and d["value"] > 0 and d["unit"] == "tokens/s"
    assert d["config"]["workload"] == "k3_decode_t1"
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0.0 < rf["frac"] < 1.0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["kernel"].startswith("gateup") and set(rf["kernels"]) == {"gateup", "down_combine"}
    assert rf["avg_ms"] == rf["kernels"]["gateup"]["avg_ms"] and rf["event_samples"] >= 1
    assert 0.0 < rf["stage"]["frac"] < 1.0
    # the stage holds both kernels: it takes longer than the dominant one alone
    assert rf["stage"]["avg_ms"] > rf["avg_ms"]
    p = d["prefill"]
    assert p["workload"] == "k3_prefill_t4096" and p["tokens_per_s"] > 0
    assert set(p["roofline"]["kernels"]) == {"active_list", "quantize", "gateup", "down", "combine"}
    assert 0.0 < p["roofline"]["mfma_frac"] < 1.0
    c = d["cache"]
    assert c["slots"] == 32 and c["oracle_lru_hit_rate"] == c["hit_rate"]
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1


def test_bench_refuses_more_than_one_gpu():
    r = _bench("--gpus", "2", timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout
