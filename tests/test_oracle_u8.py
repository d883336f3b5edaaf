"""Pins of the oracle's uint8 expert weights: the quantiser (one affine map
per matrix from its range, read as (q - zero) * scale) and the layer on
dequantised weights.

The quantiser is pinned by a grid it must reproduce exactly, exact zero,
the half-step error bound of rounding to the nearest level, the range end
points and monotonicity; the layer by equality with the bf16 layer on
weights that lie on the grid, and by a dense masked brute force in numpy.
"""
import numpy as np
import pytest

import gen
import oracle


def bf16_bits(v):
    """float64 values exactly representable in bf16 -> bit patterns."""
    f = np.asarray(v, np.float32)
    bits = f.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def dequant(q, scale, zero):
    return (q.astype(np.float64) - zero) * np.float64(scale)


def test_grid_is_reproduced_exactly():
    # values (i - 128) / 128, i = 0..255, shuffled: range [-1, 127/128], so
    # scale = (255/128) / 255 = 1/128 and zero = 128 exactly, and q = i
    rng = np.random.default_rng(1)
    i = rng.permutation(256)
    w = bf16_bits((i - 128) / 128.0)
    q, scale, zero, mn, mx = oracle.quantize_u8(w)
    assert scale == np.float32(1 / 128) and zero == 128
    assert mn == -1.0 and mx == np.float32(127 / 128)
    assert np.array_equal(q, i.astype(np.uint8))
    assert np.array_equal(dequant(q, scale, zero), (i - 128) / 128.0)


def test_all_zero_matrix():
    q, scale, zero, mn, mx = oracle.quantize_u8(np.zeros(100, np.uint16))
    assert (scale, zero, mn, mx) == (1.0, 0, 0.0, 0.0) and not q.any()


@pytest.mark.parametrize("seed,sigma,shift", [(0, 0.02, 0.0), (1, 1.0, 0.0), (2, 0.02, 0.05),
                                              (3, 3.0, -7.0)])
def test_error_bound_zero_ends_and_monotone(seed, sigma, shift):
    rng = np.random.default_rng(seed)
    v = (rng.normal(shift, sigma, 5000)).astype(np.float32)
    v[::97] = 0.0
    w = (v.view(np.uint32) >> 16).astype(np.uint16)           # truncate to bf16
    x = gen.bf16_bits_to_f32(w).astype(np.float64)
    q, scale, zero, mn, mx = oracle.quantize_u8(w)
    assert mn == min(0.0, x.min()) and mx == max(0.0, x.max())
    assert scale == np.float32(np.float32(mx - mn) / np.float32(255))
    assert 0 <= zero <= 255
    d = dequant(q, scale, zero)
    # rounding to the nearest of 256 levels: within half a step (plus the
    # fp32 rounding of w / scale)
    assert np.abs(d - x).max() <= scale * (0.5 + 1e-5)
    # zero is a level: stored zeros come back exactly
    assert np.all(q[x == 0.0] == zero) and np.all(d[x == 0.0] == 0.0)
    # the range end points map to the end codes
    assert q[np.argmin(x)] == 0 if x.min() < 0 else True
    assert q[np.argmax(x)] >= 254 if x.max() > 0 else True
    # order preserving
    o = np.argsort(x, kind="stable")
    assert np.all(np.diff(q[o].astype(int)) >= 0)


def test_expert_blocks_hold_three_matrices_and_parameters():
    shape = gen.LayerShape("u", H=32, F=48, E=3, k=2, dtype="bf16", seed=4)
    ex = gen.gen_experts(shape)
    H, F = shape.H, shape.F
    st = oracle.u8_stride(H, F)
    assert st % 256 == 0 and st >= 3 * H * F + 64
    u8 = oracle.quantize_experts_u8(ex, shape.stride, shape.E, H, F)
    for e in range(shape.E):
        p = oracle.u8_params(u8, st, e, H, F)
        for m, W in enumerate(gen.expert_views(shape, ex, e)):
            q, scale, zero, mn, mx = oracle.quantize_u8(W)
            got = u8[e * st + m * H * F:e * st + (m + 1) * H * F]
            assert np.array_equal(got, q.ravel())
            assert (p.scale[m], p.zero[m], p.min[m], p.max[m]) == (scale, zero, mn, mx)


def _grid_experts(shape, rng):
    """bf16 experts whose every matrix lies on the grid (q - 128) * 2^-10 with
    both end codes present, so that quantising gives back q exactly."""
    blob = np.zeros(shape.E * shape.stride, np.uint8)
    H, F = shape.H, shape.F
    codes = []
    for e in range(shape.E):
        q = rng.integers(0, 256, (3, H * F))
        q[:, 0], q[:, 1] = 0, 255
        w = bf16_bits((q - 128) * 2.0 ** -10)
        blob[e * shape.stride:e * shape.stride + 3 * H * F * 2] = w.view(np.uint8).ravel()
        codes.append(q)
    return blob, codes


def test_u8_layer_on_the_grid_equals_the_bf16_layer():
    shape = gen.LayerShape("g", H=32, F=40, E=4, k=2, dtype="bf16", seed=5)
    rng = np.random.default_rng(5)
    ex, codes = _grid_experts(shape, rng)
    H, F = shape.H, shape.F
    st = oracle.u8_stride(H, F)
    u8 = oracle.quantize_experts_u8(ex, shape.stride, shape.E, H, F)
    for e in range(shape.E):
        p = oracle.u8_params(u8, st, e, H, F)
        assert list(p.scale) == [2.0 ** -10] * 3 and list(p.zero) == [128] * 3
        assert np.array_equal(u8[e * st:e * st + 3 * H * F], codes[e].ravel().astype(np.uint8))
    wr = gen.gen_router(shape)
    x = gen.gen_x(shape, 17)
    ref = oracle.layer_from_gen(shape, wr, None, ex).forward(x)
    got = oracle.layer_from_gen(shape, wr, None, None, u8_experts=u8, u8_stride=st).forward(x)
    for key in ("y", "idx", "w", "perm"):
        assert np.array_equal(got[key], ref[key]), key


@pytest.mark.parametrize("E,k", [(8, 2), (6, 3)])
def test_u8_layer_equals_dense_masked_brute_force(E, k):
    shape = gen.LayerShape("m", H=24, F=32, E=E, k=k, dtype="bf16", seed=6)
    H, F, T = shape.H, shape.F, 11
    ex = gen.gen_experts(shape)
    st = oracle.u8_stride(H, F)
    u8 = oracle.quantize_experts_u8(ex, shape.stride, E, H, F)
    wr = gen.gen_router(shape)
    x = gen.gen_x(shape, T)
    r = oracle.layer_from_gen(shape, wr, None, None, u8_experts=u8, u8_stride=st).forward(x)
    X = gen.bf16_bits_to_f32(x).astype(np.float64)
    logits = X @ gen.bf16_bits_to_f32(wr).astype(np.float64)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    assert (order == r["idx"]).all()
    sel = np.take_along_axis(logits, order, 1)
    g = np.exp(sel - sel[:, :1])
    mask = np.zeros((T, E))
    np.put_along_axis(mask, order, g / g.sum(1, keepdims=True), 1)
    y = np.zeros((T, H))
    for e in range(E):
        p = oracle.u8_params(u8, st, e, H, F)
        base = e * st
        W = [dequant(u8[base + m * H * F:base + (m + 1) * H * F], p.scale[m], p.zero[m])
             for m in range(3)]
        Wg, Wu, Wd = W[0].reshape(F, H), W[1].reshape(F, H), W[2].reshape(H, F)
        a = np.vectorize(oracle.bf16_round)(X @ Wg.T / (1 + np.exp(-(X @ Wg.T))) * (X @ Wu.T))
        y += mask[:, e:e + 1] * (a @ Wd.T)
    rms = np.sqrt((y ** 2).mean())
    assert np.abs(r["y"] - y).max() <= 1e-12 * rms


def test_u8_layer_rejects_bad_layouts():
    shape = gen.LayerShape("b", H=16, F=16, E=2, k=1, dtype="bf16", seed=7)
    wr = gen.gen_router(shape)
    small = oracle.u8_stride(16, 16) - 256  # less than 3HF + 64
    u8 = np.zeros(2 * oracle.u8_stride(16, 16), np.uint8)
    x = gen.gen_x(shape, 2)
    with pytest.raises(RuntimeError):
        oracle.layer_from_gen(shape, wr, None, None, u8_experts=u8, u8_stride=small).forward(x)
