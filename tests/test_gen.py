"""The seeded input generator (host side): pinned to published definitions."""
import math
import os

import numpy as np
import pytest
from scipy import stats

import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_known_answer():
    want = [int(l, 16) for l in open(os.path.join(GOLDEN, "splitmix64_seed0.txt"))
            if l.startswith("0x")]
    got = [gen.lib().gen_splitmix64_output(0, i) for i in range(len(want))]
    assert got == want


def test_log_and_cos_against_libm():
    rng = np.random.default_rng(1)
    L = gen.lib()
    for u in list(rng.uniform(1e-300, 1.0, 2000)) + [1.0, 0.5, 2.0 ** -53, math.sqrt(0.5)]:
        assert abs(L.gen_log01_host(u) - math.log(u)) <= 4e-16 * max(1.0, abs(math.log(u)))
    for v in list(rng.uniform(0.0, 1.0, 2000)) + [0.0, 0.25, 0.5, 0.75, 0.125]:
        assert abs(L.gen_cos2pi01_host(v) - math.cos(2 * math.pi * v)) <= 2e-15


def test_normal_distribution():
    a = gen.normal(0, 0, gen.T_X, 200_000, 1.0, "f64")
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1.0) < 0.01
    assert stats.kstest(a, "norm").pvalue > 1e-3


def test_rounding_chain_and_determinism():
    d = gen.normal(3, 2, gen.T_WG, 5000, 0.02, "f64", idx0=777)
    f = gen.normal(3, 2, gen.T_WG, 5000, 0.02, "f32", idx0=777)
    b = gen.normal(3, 2, gen.T_WG, 5000, 0.02, "bf16", idx0=777)
    assert np.array_equal(d.astype(np.float32), f)  # fp64 -> fp32 RNE
    # fp32 -> bf16 RNE: the kept value is the nearest bf16, ties to even bits
    wide = gen.bf16_bits_to_f32(b).astype(np.float64)
    up = gen.bf16_bits_to_f32(b + 1).astype(np.float64)
    dn = gen.bf16_bits_to_f32(b - 1).astype(np.float64)
    err = np.abs(wide - f)
    assert np.all(err <= np.abs(up - f)) and np.all(err <= np.abs(dn - f))
    # counter property: any sub-range equals the same slice of a longer run
    f2 = gen.normal(3, 2, gen.T_WG, 100, 0.02, "f32", idx0=777 + 1234)
    assert np.array_equal(f2, f[1234:1334])


def test_streams_differ():
    a = gen.normal(0, 0, gen.T_WG, 64, 1.0, "f64")
    b = gen.normal(0, 0, gen.T_WU, 64, 1.0, "f64")
    c = gen.normal(0, 1, gen.T_WG, 64, 1.0, "f64")
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_zipf_bias():
    b = gen.zipf_bias(128)
    assert b[0] == np.float32(2.0)
    assert np.all(np.diff(b) < 0)
    assert abs(b[9] - 2.0 * 10 ** -1.1) < 1e-6


def test_expert_blob_layout():
    s = gen.TINY
    blob = gen.gen_experts(s)
    assert blob.size == s.E * s.stride
    Wg, Wu, Wd = gen.expert_views(s, blob, 3)
    want = gen.normal(0, 0, gen.T_WD, s.H * s.F, gen.SIGMA_W, "f32", idx0=3 * s.H * s.F)
    assert np.array_equal(Wd.ravel(), want)
    part = gen.gen_experts(s, experts=[3])
    assert np.array_equal(part[3 * s.stride:4 * s.stride], blob[3 * s.stride:4 * s.stride])
    assert not part[:3 * s.stride].any()
