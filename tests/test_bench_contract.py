"""bench.py's command line and output: one JSON line with the fields its
readers depend on, one GPU only."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=240):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=timeout)


def test_more_than_one_gpu_exits_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in r.stderr


@pytest.mark.gpu
def test_decode_line_has_every_field():
    print("case bench.py --steps 4 --warmup 1 --no-cpu-baseline --no-extra", flush=True)
    r = _bench("--steps", "4", "--warmup", "1", "--no-cpu-baseline", "--no-extra")
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    for k, t in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int), ("warmup", int),
                 ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str), ("dtype", str), ("data", str),
                 ("config", dict), ("roofline", dict), ("step_ms", dict), ("ceilings", dict)]:
        assert isinstance(d[k], t), k
    assert d["n_gpus"] == 1 and d["steps"] == 4 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["vs_baseline"] is None and d["cpu_baseline"] is None
    # the default workload is the largest that fits one GPU
    assert d["config"]["workload"] == "decode_h128" and d["config"]["batch"] == 64 and d["config"]["heads"] == 128
    assert 1 <= d["config"]["graph_steps"] <= 4 and 4 % d["config"]["graph_steps"] == 0
    st = d["step_ms"]
    assert st["n"] == 4 and 0 < st["p10"] <= st["median"] <= st["p90"]
    rf = d["roofline"]
    # 128 heads: 242 FLOP per byte, below the 312 FLOP/B ridge, so HBM bounds it
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["frac"] <= 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    # the achieved rate is the algorithmic bytes over the kernel's event-timed duration
    assert abs(rf["achieved"] - rf["alg_bytes_per_launch"] / (rf["kernel_avg_us"] * 1e-6) / 1e9) < 1e-6 * rf["achieved"]
    assert abs(rf["tflops"] - rf["alg_flops_per_launch"] / (rf["kernel_avg_us"] * 1e-6) / 1e12) < 1e-6 * rf["tflops"]
    assert 0 < rf["mfma_frac"] <= 1
    assert rf["traffic"] is None or rf["traffic"] > 0.9 * rf["alg_bytes_per_launch"]
    c = d["ceilings"]
    assert 1000 < c["hbm_read_GBps"] < 8000 * 1.05
    assert 100 < c["mfma_bf16_16x16x32_TFLOPs"] < 2500 * 1.05 and 100 < c["mfma_bf16_32x32x16_TFLOPs"] < 2500 * 1.05
    assert 0 < c["lds_read_b128_B_per_clk_cu"] and 0 < c["lds_read_tr_b64_B_per_clk_cu"]
    assert abs(rf["hbm_frac_of_measured"] - rf["hbm_GBps"] / c["hbm_read_GBps"]) < 1e-9
