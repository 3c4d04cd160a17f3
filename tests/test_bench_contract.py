"""The benchmark's command-line contract: one GPU only, and one JSON line
with the fields the measurement record needs."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_small_run_prints_one_json_line():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    args = [sys.executable, BENCH, "--quiet", "--ring", "2", "--steps", "40", "--warmup", "5",
            "--tokens", "16", "--dense-steps", "5", "--cpu-seconds", "0.5", "--trace-samples", "8",
            "--repeat-steps", "20",
            "--stack-tokens", "0", "--layout-steps", "0", "--gated-steps", "0", "--batches",
            "--head-calls", "20", "--head-ring", "2",
            "--ffn-rhos", "0.1", "--ffn-sets", "8"]
    r = subprocess.run(args, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 40 and d["warmup"] == 5
    assert d["unit"] == "tokens/s" and d["value"] > 0 and d["higher_is_better"] is True
    assert "workload" in d["config"]
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9 and rf["achieved"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["sample"]
    assert cb["one_thread"]["tokens_per_s"] > 0 and cb["dense"]["tokens_per_s"] > 0
    assert cb["cpu_model"] and cb["host_cpus"] >= 1
    assert d["traced_steps"] == 8 and rf["samples"] == 8 and d["kernel_sum_within_traced_span"]
    assert len(d["repeats_ms_per_step"]) == 5 and d["cache_hot"]["median5_ms_per_step"] > 0
    assert d["ambiguous"]["tokens"] > 0 and d["ambiguous"]["in_margin_per_token"] >= 0
    assert d["sparse_ffn_only"]["by_rho"][0]["ms_per_call"] > 0
    assert [r["batch"] for r in d["head_predictor"]["by_batch"]] == [1, 32]
