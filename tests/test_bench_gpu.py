"""bench.py on the GPU, briefly: exactly one JSON line on stdout with the
fields of its contract (metric, value, unit, steps, roofline with bound,
achieved, peak, frac and traffic, cpu_baseline with value, unit, cores, kind
and sample, the workload config), and the beside-records it reports by
default."""
from __future__ import annotations

import json
import subprocess
import sys

import pytest

from tests.conftest import ROOT

pytestmark = pytest.mark.gpu


def test_bench_json_line():
    print("[bench] short run of bench.py", flush=True)
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--steps", "3", "--warmup", "1",
                        "--spinup", "0.05", "--cpu-seconds", "1"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    j = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "spinup_s"):
        assert key in j, key
    assert j["n_gpus"] == 1 and j["steps"] == 3 and j["warmup"] == 1
    assert j["value"] > 0 and j["unit"] == "TFLOP/s" and j["dtype"] == "bf16"
    assert j["config"]["workload"] == "n8k_causal_peaky"
    rf = j["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = j["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    for rec in ("secondary", "backward", "window", "split", "dropout", "varlen", "decode",
                "cold", "zero_operands", "board_power_w", "sclk_mhz"):
        assert rec in j, rec
    z = j["zero_operands"]
    assert z["kernel_us_mean"] > 0 and abs(z["frac"] - z["tflops"] / 2500.0) < 1e-3
    assert [e["workload"] for e in j["extra"]] == ["n4k_full", "n8k_full", "n16k_d64"]
    for e in j["extra"]:
        assert e["tflops"] > 0 and abs(e["frac"] - e["tflops"] / 2500.0) < 1e-3
    assert j["parity_sample"]["floor_aware_ok"]
    # the stored last good line is found and every default record compared
    reg = j["regression"]
    assert reg["status"] == "checked" and reg["last_good"] == "bench_last_good.json"
    assert reg["checked"] >= 17 and reg["worst"]["ratio"] > 0
