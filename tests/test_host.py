"""CPU tests of the host-side pieces: the seeded input generator (the one
module both the HIP path and the oracle read), the workload definitions the
bench reports, and bench.py's command-line contract."""
from __future__ import annotations

import json
import subprocess
import sys

import numpy as np
import pytest
import torch

from io_aware_transformer_amd.inputs import WORKLOADS, bits, make_qkv, make_workload
from tests.conftest import ROOT


def test_generator_is_deterministic_and_seed_dependent():
    a = make_qkv(1, 2, 33, 64, "bf16", seed=5)
    b = make_qkv(1, 2, 33, 64, "bf16", seed=5)
    c = make_qkv(1, 2, 33, 64, "bf16", seed=6)
    for x, y in zip(a, b):
        assert np.array_equal(bits(x), bits(y))
    assert not np.array_equal(bits(a[0]), bits(c[0]))
    # q, k and v are distinct draws of one stream
    assert not np.array_equal(bits(a[0]), bits(a[1]))


@pytest.mark.parametrize("dtype,tdt", [("f16", torch.float16), ("bf16", torch.bfloat16)])
def test_generator_follows_the_recipe(dtype, tdt):
    """q, k, v = one CPU generator's randn draws in that order, q and k times
    the gain in fp32, each cast once (round to nearest even)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(11)
    shape = (2, 1, 17, 8)
    q, k, v = (torch.randn(shape, generator=g, dtype=torch.float32) for _ in range(3))
    got = make_qkv(*shape, dtype, seed=11, qk_gain=3.0)
    want = ((q * 3.0).to(tdt), (k * 3.0).to(tdt), v.to(tdt))
    for x, y in zip(got, want):
        assert x.dtype == tdt and x.shape == shape
        assert np.array_equal(bits(x), bits(y))


def test_bits_rejects_other_types():
    with pytest.raises(TypeError):
        bits(torch.zeros(3))
    with pytest.raises(ValueError):
        make_qkv(1, 1, 2, 8, "f32")


def test_workload_flops_convention():
    for w in WORKLOADS.values():
        full = 4.0 * w.B * w.H * w.N ** 2 * w.d
        assert w.flops == (full / 2 if w.causal else full)
        assert w.scale == float(np.float32(1.0 / np.sqrt(w.d)))
    w = WORKLOADS["n8k_causal_peaky"]
    assert (w.B, w.H, w.N, w.d, w.dtype, w.causal, w.qk_gain) == (1, 32, 8192, 128, "bf16",
                                                                 True, 3.0)
    q, k, v = make_workload(WORKLOADS["tiny"])
    assert q.shape == (1, 2, 256, 64) and q.dtype == torch.float16


def _bench(*args):
    return subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], capture_output=True,
                          text=True, timeout=120)


@pytest.mark.parametrize("n", ["2", "8"])
def test_bench_refuses_more_than_one_gpu(n):
    r = _bench("--gpus", n)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_bench_help_names_every_option():
    r = _bench("--help")
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--workload", "--secondary", "--extra",
                "--backward", "--window", "--split", "--dropout", "--varlen", "--decode",
                "--spinup", "--last-good", "--regression-threshold", "--fail-on-regression",
                "--save-last-good", "--no-zeros", "--no-cold", "--no-cpu-baseline"):
        assert opt in r.stdout, opt


def test_bench_without_gpu_fails_loudly():
    """No GPU visible: a non-zero exit and no JSON line (never a CPU number)."""
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = _bench("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    for line in r.stdout.splitlines():
        with pytest.raises(json.JSONDecodeError):
            json.loads(line)


def test_binding_has_no_fallback(monkeypatch, tmp_path):
    """Without the HIP library (and with no way to build it) every entry
    point raises; nothing computes on the CPU instead."""
    import io_aware_transformer_amd as fa

    def no_hipcc():
        raise RuntimeError("hipcc not found: the HIP library cannot be built")

    monkeypatch.setattr(fa, "_lib", None)
    monkeypatch.setattr(fa, "_LIB_PATH", tmp_path / "missing" / "libfa_fwd.so")
    monkeypatch.setattr(fa, "_build", no_hipcc)
    q = torch.zeros((1, 1, 8, 64), dtype=torch.float16)
    calls = [
        lambda: fa.fa_fwd(0, 0, 0, 0, 0, 1, 1, 8, 64, 0, 0.125, fa.FA_DTYPE_F16),
        lambda: fa.fa_bwd(*([0] * 10), 1, 1, 8, 64, 0, 0.125, fa.FA_DTYPE_F16),
        lambda: fa.fa_fwd_varlen(*([0] * 6), 1, 1, 8, 8, 64, 0, 0.125, fa.FA_DTYPE_F16),
        lambda: fa.fa_bwd_varlen(*([0] * 11), 1, 1, 8, 8, 64, 0, 0.125, fa.FA_DTYPE_F16),
        lambda: fa.fa_bwd_workspace_size(1, 1, 8),
    ]
    for c in calls:
        with pytest.raises(RuntimeError, match="hipcc not found"):
            c()
    # the tensor-level wrappers refuse CPU tensors outright
    with pytest.raises(ValueError, match="no CPU path"):
        fa.attention(q, q, q)
    with pytest.raises(ValueError, match="no CPU path"):
        fa.attention_backward(q, q, q, q, torch.zeros((1, 1, 8)), q)


def test_bench_reads_the_marked_engine_clock(tmp_path):
    """bench.py reports the engine clock from the DPM line marked '*'."""
    import bench
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("S: 1843Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    assert bench.read_sclk_mhz(str(f)) == 1843
    f.write_text("0: 500Mhz\n1: 2400Mhz *\n")
    assert bench.read_sclk_mhz(str(f)) == 2400
    f.write_text("0: 500Mhz\n1: 2400Mhz\n")
    assert bench.read_sclk_mhz(str(f)) is None


def test_bench_reads_board_power(tmp_path):
    """hwmon power files hold microwatts."""
    import bench
    f = tmp_path / "power1_input"
    f.write_text("1391000000\n")
    assert bench.read_power_w(str(f)) == 1391.0


def test_bench_regression_check():
    """Each tracked figure is compared with the same record and workload of
    the stored line; a figure under the threshold is reported, one missing
    from either line is not compared."""
    import copy
    import bench
    good = json.loads((ROOT / "bench_last_good.json").read_text())
    figs = bench.tracked_figures(good)
    # the stored line is a complete default run: the headline and every record
    for key in ("value[n8k_causal_peaky]", "roofline.achieved[n8k_causal_peaky]",
                "secondary[n4k_causal].tflops", "extra[n16k_d64].tflops",
                "backward[n8k_causal_peaky].tflops", "decode[1:32:1:32768].gbs"):
        assert key in figs, key
    assert good["config"]["workload"] == "n8k_causal_peaky"
    assert good["parity_sample"]["floor_aware_ok"] is True

    same = bench.regression_check(good, good, 0.9, "g")
    assert same["ok"] and same["checked"] == len(figs) and same["regressed"] == {}
    assert same["worst"]["ratio"] == 1.0

    cur = copy.deepcopy(good)
    cur["value"] = good["value"] * 0.8
    cur["extra"][0]["tflops"] = good["extra"][0]["tflops"] * 0.95
    cur["backward"]["workload"] = "other"       # not comparable: skipped
    r = bench.regression_check(cur, good, 0.9, "g")
    assert not r["ok"]
    assert r["regressed"] == {"value[n8k_causal_peaky]": 0.8}
    assert r["worst"] == {"figure": "value[n8k_causal_peaky]", "ratio": 0.8}
    assert r["checked"] == len(figs) - 1

    missing = bench.regression_check(good, None, 0.9, "none.json")
    assert missing["status"] == "missing" and missing["ok"]


def test_bench_extra_workloads_exist():
    """The default extra records name workloads of the input recipe: the
    non-causal N4096 / N8192 d128 bf16 points and the few-head d64 one."""
    from io_aware_transformer_amd.inputs import WORKLOADS
    src = (ROOT / "bench.py").read_text()
    assert '"--extra", default="n4k_full,n8k_full,n16k_d64"' in src
    for name in ("n4k_full", "n8k_full", "n16k_d64"):
        w = WORKLOADS[name]
        assert w.d in (64, 128) and w.causal is False
    assert (WORKLOADS["n4k_full"].N, WORKLOADS["n8k_full"].N) == (4096, 8192)


def test_attention_backward_validates_lse():
    """attention_backward checks the forward's row statistics before any
    launch: the kernel reads B*H*N contiguous fp32 values from lse."""
    import io_aware_transformer_amd as fa
    q = torch.zeros((2, 3, 8, 64), dtype=torch.bfloat16)
    good = torch.zeros((2, 3, 8), dtype=torch.float32)
    with pytest.raises(TypeError, match="lse must be float32"):
        fa.attention_backward(q, q, q, q, good.half(), q)
    with pytest.raises(TypeError, match="lse must be float32"):
        fa.attention_backward(q, q, q, q, good.double(), q)
    with pytest.raises(ValueError, match=r"lse must be a contiguous \[B,H,N\]"):
        fa.attention_backward(q, q, q, q, torch.zeros((2, 3, 7)), q)
    with pytest.raises(ValueError, match=r"lse must be a contiguous \[B,H,N\]"):
        fa.attention_backward(q, q, q, q, torch.zeros((6, 8)), q)
    with pytest.raises(ValueError, match=r"lse must be a contiguous \[B,H,N\]"):
        fa.attention_backward(q, q, q, q, torch.zeros((2, 8, 3)).transpose(1, 2), q)
    with pytest.raises(ValueError, match=r"\[B,H,N,d\]"):
        fa.attention_backward(q[0], q[0], q[0], q[0], good[0], q[0])
    # a well-formed call gets as far as the device check
    with pytest.raises(ValueError, match="no CPU path"):
        fa.attention_backward(q, q, q, q, good, q)
