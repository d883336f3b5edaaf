"""Host logic of bench.py, no GPU: the refusal of more than one GPU, the
gate/up roofline's bound and fractions, the source-hash gate on the counted
traffic, the per-step percentiles and the per-config routing report."""
import hashlib
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}),
                                      (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, **env))
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_roofline_mixtral_prefill_is_mfma_bound():
    # 4 T k H F = 4 * 4096 * 2 * 4096 * 14336 = 1.9241e12 flop; bytes = 8
    # experts' gate+up (1.8790e9) + tokens (33.55e6) + activation (234.9e6)
    # = 2.1475e9: 896 flop/B, above the 312.5 flop/B ridge
    r = bench.gate_up_roofline(gen.MIXTRAL, 4096, 8, 1779.9e-6)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["achieved"] == pytest.approx(1081.0, abs=0.1)
    assert r["frac"] == pytest.approx(0.4324, abs=1e-4)
    assert r["hbm_frac"] == pytest.approx(2.1475e9 / 1779.9e-6 / 8e12, abs=1e-4)


def test_roofline_64_experts_is_hbm_bound():
    # S = 1024 pairs: 4 * 1024 * 2048 * 1408 = 11.81e9 flop; bytes = 64
    # experts' gate+up (738.2e6) + tokens (2.097e6) + activation (2.884e6) =
    # 743.2e6: 15.9 flop/B, below the ridge
    r = bench.gate_up_roofline(gen.QWEN, 512, 64, 0.1336e-3)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(5563.0, abs=1.0)
    assert r["frac"] == pytest.approx(0.6953, abs=1e-4)
    assert r["mfma_frac"] == pytest.approx(11.81e9 / 0.1336e-3 / 2.5e15, abs=1e-4)


def _profile(tmp_path, digest, extra):
    p = tmp_path / "prof.md"
    p.write_text("# summary\n\nsource_sha256 expert_grouped.hip: " + digest + "\n" + extra)
    return str(p)


def test_traffic_only_while_the_source_matches(tmp_path):
    src = os.path.join(ROOT, "mixture_experts_amd", "csrc", "expert_grouped.hip")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    line = "traffic_bytes_per_launch: 7.2435e+09\ntraffic_bytes_per_launch_x: 1.5e9\n"
    good = _profile(tmp_path, digest, line)
    assert bench.measured_traffic(good) == 7.2435e9
    assert bench.measured_traffic(good, "traffic_bytes_per_launch_x") == 1.5e9
    assert bench.measured_traffic(good, "traffic_bytes_per_launch_y") is None
    stale = _profile(tmp_path, "0" * 64, line)
    assert bench.measured_traffic(stale) is None
    assert bench.measured_traffic(str(tmp_path / "missing.md")) is None


def test_percentiles():
    assert bench.percentiles([float(v) for v in range(1, 11)]) == [1.9, 5.5, 9.1]
    assert bench.percentiles([2.5]) == [2.5, 2.5, 2.5]


def test_routing_report_counts_loads_and_near_ties():
    shape = gen.LayerShape("t", H=2, F=8, E=3, k=1, dtype="bf16")
    one, two = 0x3F80, 0x4000  # bf16 bit patterns of 1.0 and 2.0
    x = np.array([[one, 0], [0, one], [one, one]], dtype=np.uint16)
    wr = np.array([[one, one, 0], [0, 0, two]], dtype=np.uint16)  # [H][E]
    # logits: [1, 1, 0] (tie), [0, 0, 2], [1, 1, 2] (margin 1)
    r = bench.routing_stats(shape, x, wr, None, [2, 0, 1])
    assert r == {"experts_touched": 2, "load_min": 0, "load_median": 1.0, "load_max": 2,
                 "near_ties": 1}
    # a bias that separates experts 0 and 1 by less than 1e-3 keeps the tie near
    b = np.array([0.0, 5e-4, 0.0], dtype=np.float32)
    assert bench.routing_stats(shape, x, wr, b, [2, 0, 1])["near_ties"] == 1
    b = np.array([0.0, 0.5, 0.0], dtype=np.float32)
    assert bench.routing_stats(shape, x, wr, b, [2, 0, 1])["near_ties"] == 0
