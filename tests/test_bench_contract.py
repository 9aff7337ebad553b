"""bench.py's output contract: one JSON line with the driver's fields plus `roofline` and
`cpu_baseline`, and a clear refusal of more than one GPU (checked without a GPU)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
        "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"}


def run_bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=timeout, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2", timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
@pytest.mark.parametrize("workload", ["C2-c", "C3-bwd", "SM4", "D2"])
def test_json_line(workload):
    r = run_bench("--workload", workload, "--steps", "3", "--warmup", "1", "--cpu-rows", "64")
    print(r.stderr[-2000:], flush=True)
    assert r.returncode == 0
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert KEYS <= set(d), KEYS - set(d)
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["value"] > 0
    assert isinstance(d["config"], dict) and "workload" in d["config"]
    rf = d["roofline"]
    assert rf["bound"] in ("hbm", "mfma") and rf["peak"] > 0 and 0 < rf["frac"] < 1.5
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    if workload == "C2-c":
        # forward legs also carry provenance, the sampled clock and the timed launch's parity
        pv = d["provenance"]
        assert pv["seed"] == 102 and pv["gpu_arch"].startswith("gfx950") and len(pv["sources_sha256"]) == 16
        assert d["parity"]["rows"] == 64 and d["parity"]["pass"] is True
        assert d["metric"].startswith("attention fwd TFLOP/s (bf16, causal)")
        ck = d["clock"]
        assert ck["error"] is None, ck
        assert ck["probes"] >= 1 and 100 < ck["min_mhz"] <= ck["median_mhz"] <= ck["max_mhz"] < 3000
        assert ck["clock_adjusted_peak_tflops"] == pytest.approx(2500.0 * ck["median_mhz"] / 2400.0)


@pytest.mark.gpu
def test_gemm_reference_leg():
    """The context leg: the vendor bf16 GEMM's line has the driver's fields, an MFMA roofline
    whose fraction matches its figures, no CPU baseline, and a measured clock."""
    r = run_bench("--workload", "GEMM-ref", "--steps", "3", "--warmup", "1")
    print(r.stderr[-2000:], flush=True)
    assert r.returncode == 0
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert KEYS <= set(d), KEYS - set(d)
    assert d["cpu_baseline"] is None and d["value"] > 0 and "not mifa" in d["metric"]
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    assert d["clock"]["error"] is None, d["clock"]


@pytest.mark.gpu
def test_hbm_reference_leg():
    """The HBM context leg: a copy rate and a read rate, both below the 8 TB/s peak."""
    r = run_bench("--workload", "HBM-ref", "--steps", "3", "--warmup", "1")
    print(r.stderr[-2000:], flush=True)
    assert r.returncode == 0
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert KEYS <= set(d), KEYS - set(d)
    assert d["cpu_baseline"] is None and "not mifa" in d["metric"]
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and 0 < rf["frac"] < 1.0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    assert 0 < d["config"]["sum_gbs"] < 8000.0


@pytest.mark.gpu
def test_cold_cache_leg():
    """--cold rotates through copies whose total exceeds twice the 256 MiB last-level cache, and a
    workload below the ridge (C2 causal, 204 FLOP/B) reports the HBM roofline in GB/s."""
    r = run_bench("--workload", "C2-c", "--cold", "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    print(r.stderr[-2000:], flush=True)
    assert r.returncode == 0
    d = json.loads([l for l in r.stdout.splitlines() if l.strip()][0])
    c = d["config"]
    assert c["cold_cache"] is True and c["rotating_copies"] * c["compulsory_hbm_bytes"] > 2 * (256 << 20)
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["achieved"] - c["compulsory_gbs"]) < 1e-6 * rf["achieved"]


def test_forward_roofline_choice_and_formulas():
    """Host logic of the forward legs: FLOPs 4 B H N^2 d (halved when causal), compulsory bytes
    (bf16 Q, K, V read once, fp32 O and LSE written once), and the roofline the arithmetic
    intensity implies (ridge 2.5e15 / 8e12 = 312.5 FLOP/B)."""
    sys.path.insert(0, ROOT)
    import bench
    from io_aware_softmax_mifa_amd import workloads as W

    assert bench.RIDGE_FLOP_PER_BYTE == 312.5
    w = W.by_name("C4")
    assert bench.flops(w) == 4.0 * 32 * 16384 ** 2 * 128 / 2
    assert bench.compulsory_bytes(w) == 673185792
    expect = {"C1-nc": "hbm", "C1-c": "hbm", "C2-nc": "mfma", "C2-c": "hbm", "C3": "mfma", "C4": "mfma", "C5": "mfma"}
    for name, bound in expect.items():
        w = W.by_name(name)
        f, cb = bench.flops(w), bench.compulsory_bytes(w)
        r = bench.forward_roofline(f, cb, 1.0)
        assert r["bound"] == bound, name
        assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-12
        if bound == "mfma":
            assert r["unit"] == "TFLOP/s" and abs(r["achieved"] - f / 1e-3 / 1e12) < 1e-6 * r["achieved"]
        else:
            assert r["unit"] == "GB/s" and abs(r["achieved"] - cb / 1e-3 / 1e9) < 1e-6 * r["achieved"]


