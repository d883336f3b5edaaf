"""Pins of the fp64 CPU oracle to things other than itself.

Each test checks one part of the oracle against a closed form, a textbook
routine (stable sort, dense matrix products), an invariant, or brute force on
tiny inputs, chosen so that a dropped term, a wrong sign, a transposed operand
or a wrong index fails at least one of them.
"""
import math

import numpy as np
import pytest

import gen
import oracle


def make_layer(H, F, E, k, dtype="f32", seed=0, bias=None, layer=0):
    shape = gen.LayerShape("t", H=H, F=F, E=E, k=k, dtype=dtype, seed=seed)
    wr = gen.gen_router(shape, layer=layer)
    ex = gen.gen_experts(shape, layer=layer)
    return shape, oracle.layer_from_gen(shape, wr, bias, ex), wr, ex


def widen(a, dtype):
    return (gen.bf16_bits_to_f32(a) if dtype == "bf16" else a).astype(np.float64)


def silu(z):
    return z / (1.0 + np.exp(-z))


# --- hand-worked example (closed forms) ------------------------------------


def _worked(dtype):
    """H=2, F=2, E=3, k=2, x = (1, 2); every weight exact in fp32 and bf16.

    logits = x.Wr = (1, 2, 1): expert 1 first; experts 0 and 2 tie at 1 and
    the lower index (0) takes slot 1.  Gates: softmax(2, 1) = (e/(e+1), 1/(e+1)).
    Expert 1: g = (1, 0), u = (1, 2)      -> act = (silu(1), 0) -> y = (act0, 0)
    Expert 0: g = (2, 0), u = (1, 0)      -> act = (silu(2), 0) -> y = (0, act0)
    """
    npd = np.float32 if dtype == "f32" else np.uint16

    def st(a):
        a = np.asarray(a, np.float32)
        return a if dtype == "f32" else (a.view(np.uint32) >> 16).astype(np.uint16)

    H, F, E, k = 2, 2, 3, 2
    wr = st([[1.0, 0.0, 0.5], [0.0, 1.0, 0.25]])
    # per expert: Wg [F][H], Wu [F][H], Wd [H][F]
    Wg = {0: [[0, 1], [0, 0]], 1: [[1, 0], [0, 0]], 2: [[1, 1], [1, 1]]}
    Wu = {0: [[1, 0], [0, 0]], 1: [[1, 0], [0, 1]], 2: [[1, 1], [1, 1]]}
    Wd = {0: [[0, 0], [1, 0]], 1: [[1, 0], [0, 2]], 2: [[5, 5], [5, 5]]}
    es = 4 if dtype == "f32" else 2
    stride = 256
    blob = np.zeros(E * stride, np.uint8)
    for e in range(E):
        m = np.concatenate([st(Wg[e]).ravel(), st(Wu[e]).ravel(), st(Wd[e]).ravel()])
        blob[e * stride: e * stride + m.size * es] = m.view(np.uint8)
    L = oracle.Layer(H, F, E, k, dtype, wr, None, blob, stride)
    x = st([[1.0, 2.0]]).astype(npd)
    return L, x


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_worked_example(dtype):
    L, x = _worked(dtype)
    r = L.forward(x)
    assert r["idx"].tolist() == [[1, 0]]
    e = math.e
    assert abs(r["w"][0, 0] - e / (e + 1)) < 1e-15 and abs(r["w"][0, 1] - 1 / (e + 1)) < 1e-15
    s1 = 1.0 / (1.0 + math.exp(-1.0))            # silu(1) = sigma(1)
    s2 = 2.0 / (1.0 + math.exp(-2.0))            # silu(2)
    if dtype == "bf16":                          # act stored in bf16: 8 significant bits
        s1 = round(s1 * 256) / 256               # 187/256
        s2 = round(s2 * 128) / 128               # 225/128
        assert (s1, s2) == (187 / 256, 225 / 128)
    want = [e / (e + 1) * s1, 1 / (e + 1) * s2]
    assert np.allclose(r["y"][0], want, rtol=1e-15, atol=0)
    assert r["counts"].tolist() == [1, 1, 0]
    assert r["perm"].tolist() == [1, 0] and r["inv"].tolist() == [1, 0]


# --- P1: tie rule and softmax with all-equal logits --------------------------


@pytest.mark.parametrize("E,k", [(8, 2), (16, 4), (8, 8), (5, 1)])
def test_equal_logits_pick_lowest_indices(E, k):
    idx, w = oracle.topk_softmax(np.zeros((3, E)), k)
    assert (idx == np.arange(k)).all()
    assert (w == 1.0 / k).all() if k in (1, 2, 4, 8) else np.allclose(w, 1.0 / k)
    shape, L, wr, ex = make_layer(16, 8, E, k)
    zero = oracle.Layer(16, 8, E, k, "f32", np.zeros_like(wr), None, ex, shape.stride)
    r = zero.forward(gen.gen_x(shape, 5))
    assert (r["idx"] == np.arange(k)).all()


# --- P2: gates, closed form for k = 2 and invariants ---------------------


def test_gate_closed_form_and_invariants():
    rng = np.random.default_rng(7)
    Lg = rng.normal(0, 2, (500, 16))
    idx, w = oracle.topk_softmax(Lg, 2)
    l0 = Lg[np.arange(500), idx[:, 0]]
    l1 = Lg[np.arange(500), idx[:, 1]]
    logistic = 1.0 / (1.0 + np.exp(l1 - l0))
    assert np.all(np.abs(w[:, 0] - logistic) <= 4 * np.spacing(logistic))
    for k in (1, 3, 4, 7):
        idx, w = oracle.topk_softmax(Lg, k)
        assert np.all(np.abs(w.sum(1) - 1.0) <= 8 * np.finfo(float).eps)
        assert np.all(np.diff(w, axis=1) <= 0)
        assert np.all(w[:, 0] >= 1.0 / k - 1e-15)


# --- P3: top-k with k = E is a stable sort by (-logit, index) -------------


def test_topk_full_sort_equals_stable_sort():
    rng = np.random.default_rng(3)
    Lg = rng.integers(-3, 4, (400, 9)).astype(np.float64)  # many exact ties
    Lg[:5] = -0.0  # signed zeros compare equal
    Lg[5:10, ::2] = 0.0
    idx, _ = oracle.topk_softmax(Lg, 9)
    for t in range(400):
        want = sorted(range(9), key=lambda e: (-Lg[t, e], e))
        assert idx[t].tolist() == want
    idx3, _ = oracle.topk_softmax(Lg, 3)
    assert (idx3 == idx[:, :3]).all()


# --- P4: forced routing by bias ----------------------------------------


def test_bias_forces_routing_and_known_permutation():
    H, F, E, k, T = 16, 8, 8, 3, 11
    bias = (-10.0 * np.arange(E)).astype(np.float32)
    shape, L, wr, ex = make_layer(H, F, E, k, bias=bias)
    r = L.forward(gen.gen_x(shape, T))
    assert (r["idx"] == np.arange(k)).all()
    assert r["counts"].tolist() == [T] * k + [0] * (E - k)
    want_perm = [t * k + j for j in range(k) for t in range(T)]
    assert r["perm"].tolist() == want_perm
    assert r["offsets"].tolist() == [min(e, k) * T for e in range(E + 1)]


# --- P5: dispatch is a stable counting sort ------------------------------


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (37, 8, 2), (200, 64, 2), (129, 128, 4), (0, 4, 2)])
def test_dispatch_invariants(T, E, k):
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).reshape(T, k) \
        if T else np.zeros((0, k), np.int32)
    counts, offsets, perm, inv = oracle.dispatch(idx, E)
    assert counts.sum() == T * k
    assert (np.diff(offsets) == counts).all() and offsets[0] == 0
    assert sorted(perm.tolist()) == list(range(T * k))
    assert (inv[perm] == np.arange(T * k)).all()
    pairs = sorted((int(idx[s // k, s % k]), s // k, s) for s in range(T * k))
    assert perm.tolist() == [s for _, _, s in pairs]
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert (idx.ravel()[seg] == e).all()
        assert np.all(np.diff(seg // k) > 0)


# --- P6: E = 1, k = 1 is a dense SwiGLU FFN ------------------------------


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_expert_is_dense_swiglu(dtype):
    H, F, T = 24, 40, 9
    shape, L, wr, ex = make_layer(H, F, 1, 1, dtype=dtype)
    x = gen.gen_x(shape, T)
    r = L.forward(x)
    assert (r["w"] == 1.0).all()
    Wg, Wu, Wd = (widen(m, dtype) for m in gen.expert_views(shape, ex, 0))
    X = widen(x, dtype)
    a = silu(X @ Wg.T) * (X @ Wu.T)
    if dtype == "bf16":
        a = np.vectorize(oracle.bf16_round)(a)
    y = a @ Wd.T
    assert np.abs(r["y"] - y).max() <= 1e-13 * np.abs(y).max()


# --- P7: sparse dispatch equals the dense masked sum (brute force) -------


@pytest.mark.parametrize("E,k,dtype", [(8, 2, "f32"), (6, 3, "f32"), (5, 5, "f32"), (8, 2, "bf16")])
def test_sparse_equals_dense_masked(E, k, dtype):
    H, F, T = 16, 24, 13
    shape, L, wr, ex = make_layer(H, F, E, k, dtype=dtype)
    x = gen.gen_x(shape, T)
    r = L.forward(x)
    X = widen(x, dtype)
    logits = X @ widen(wr, dtype)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    assert (order == r["idx"]).all()
    sel = np.take_along_axis(logits, order, 1)
    g = np.exp(sel - sel[:, :1])
    gates = g / g.sum(1, keepdims=True)
    mask = np.zeros((T, E))
    np.put_along_axis(mask, order, gates, 1)
    y = np.zeros((T, H))
    for e in range(E):                      # every expert on every token
        Wg, Wu, Wd = (widen(m, dtype) for m in gen.expert_views(shape, ex, e))
        a = silu(X @ Wg.T) * (X @ Wu.T)
        if dtype == "bf16":
            a = np.vectorize(oracle.bf16_round)(a)
        y += mask[:, e:e + 1] * (a @ Wd.T)
    rms = np.sqrt((y ** 2).mean())
    assert np.abs(r["y"] - y).max() <= 1e-12 * rms


# --- gate variants: raw-logit gates, soft routing (k = E) -------------------


def test_raw_gate_weights_are_the_selected_logits():
    """Raw gate [m.nxbn.cn/news/47896 sec. 3.2; www.pnsm.cn/news/1892388.html
    sec. 3.3]: same selection as the softmax gate, weights = those logits."""
    rng = np.random.default_rng(3)
    lg = rng.normal(size=(40, 12))
    lg[5, 3] = lg[5, 7] = lg[5].max() + 1.0      # planted tie for the top slot
    lg[9, :] = 0.25                               # all equal
    i_s, _ = oracle.topk(lg, 4, "softmax")
    i_r, w_r = oracle.topk(lg, 4, "raw")
    assert (i_r == i_s).all()
    assert np.array_equal(w_r, np.take_along_axis(lg, i_r.astype(np.int64), 1))
    assert list(i_r[5, :2]) == [3, 7] and list(i_r[9]) == [0, 1, 2, 3]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_raw_gate_equals_dense_brute_force(dtype):
    H, F, E, k, T = 16, 24, 6, 2, 11
    shape, _, wr, ex = make_layer(H, F, E, k, dtype=dtype)
    L = oracle.layer_from_gen(shape, wr, None, ex, gate="raw")
    x = gen.gen_x(shape, T)
    r = L.forward(x)
    X = widen(x, dtype)
    logits = X @ widen(wr, dtype)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    assert (order == r["idx"]).all()
    mask = np.zeros((T, E))
    np.put_along_axis(mask, order, np.take_along_axis(logits, order, 1), 1)
    y = np.zeros((T, H))
    for e in range(E):
        Wg, Wu, Wd = (widen(m, dtype) for m in gen.expert_views(shape, ex, e))
        a = silu(X @ Wg.T) * (X @ Wu.T)
        if dtype == "bf16":
            a = np.vectorize(oracle.bf16_round)(a)
        y += mask[:, e:e + 1] * (a @ Wd.T)
    assert np.abs(r["y"] - y).max() <= 1e-12 * np.sqrt((y ** 2).mean())
    t = L.tokens(x, np.array([0, 4, 10], np.int32))
    assert np.array_equal(t["y"], r["y"][[0, 4, 10]]) and np.array_equal(t["w"], r["w"][[0, 4, 10]])


def test_raw_gate_router_scaling_is_exact():
    """Doubling the router doubles every logit exactly, keeps the selection,
    and doubles the raw weights, so the output doubles bit for bit."""
    shape, _, wr, ex = make_layer(16, 24, 8, 2)
    x = gen.gen_x(shape, 9)
    r1 = oracle.layer_from_gen(shape, wr, None, ex, gate="raw").forward(x)
    r2 = oracle.layer_from_gen(shape, 2 * wr, None, ex, gate="raw").forward(x)
    assert (r1["idx"] == r2["idx"]).all()
    assert np.array_equal(r2["w"], 2 * r1["w"]) and np.array_equal(r2["y"], 2 * r1["y"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_soft_routing_k_equals_E_is_dense_softmax_mixture(dtype):
    """Soft routing, read as weighting every expert instead of a hard top-k
    selection [m.nxbn.cn/news/47896 sec. 2.2, soft_route()]: with k = E the
    layer is sum_e softmax(L)_e FFN_e(x) over all experts."""
    H, F, E, T = 16, 24, 8, 7
    shape, L, wr, ex = make_layer(H, F, E, E, dtype=dtype)
    x = gen.gen_x(shape, T)
    r = L.forward(x)
    X = widen(x, dtype)
    logits = X @ widen(wr, dtype)
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    assert np.allclose(np.sort(r["w"], 1), np.sort(p, 1), rtol=0, atol=1e-15)
    assert all(sorted(row) == list(range(E)) for row in r["idx"].tolist())
    y = np.zeros((T, H))
    for e in range(E):
        Wg, Wu, Wd = (widen(m, dtype) for m in gen.expert_views(shape, ex, e))
        a = silu(X @ Wg.T) * (X @ Wu.T)
        if dtype == "bf16":
            a = np.vectorize(oracle.bf16_round)(a)
        y += p[:, e:e + 1] * (a @ Wd.T)
    assert np.abs(r["y"] - y).max() <= 1e-12 * np.sqrt((y ** 2).mean())


# --- expert capacity with token dropping -------------------------------------


def _capacity_reference(idx, E, cap):
    """Independent statement of the rule: per expert, its (token, slot) pairs
    in ascending slot id s = t*k + j, the first `cap` kept."""
    flat = idx.ravel()
    keep = np.zeros(flat.size, bool)
    for e in range(E):
        s_e = np.flatnonzero(flat == e)          # ascending
        keep[s_e[:cap] if cap > 0 else s_e] = True
    return keep


@pytest.mark.parametrize("E,k,T,cap", [(8, 2, 300, 50), (5, 3, 64, 7), (16, 1, 40, 1), (4, 4, 30, 30)])
def test_capacity_dispatch_brute_force(E, k, T, cap):
    rng = np.random.default_rng(E * 100 + cap)
    # heavily skewed routing: experts 0 and 1 get most pairs
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[: T // 2, 0] = 0
    idx[: T // 2, 1 % k] = 1 if k > 1 else 0
    for t in range(T):  # keep the k experts of a token distinct
        if len(set(idx[t])) < k:
            idx[t] = rng.permutation(E)[:k]
    counts, offsets, perm, inv = oracle.dispatch(idx, E, capacity=cap)
    keep = _capacity_reference(idx, E, cap)
    raw = np.bincount(idx.ravel(), minlength=E)
    assert (counts == np.minimum(raw, cap)).all()
    assert offsets[0] == 0 and (np.diff(offsets) == counts).all()
    nk = int(offsets[-1])
    assert (inv[~keep] == -1).all() and (perm[nk:] == -1).all()
    kept_s = np.flatnonzero(keep)
    assert sorted(perm[:nk].tolist()) == kept_s.tolist()          # a bijection onto the kept pairs
    assert (inv[perm[:nk]] == np.arange(nk)).all()
    for e in range(E):                                           # expert-major, slot order inside
        seg = perm[offsets[e]:offsets[e + 1]]
        assert (idx.ravel()[seg] == e).all() and (np.diff(seg) > 0).all()


def test_capacity_at_or_above_the_largest_count_changes_nothing():
    shape, L0, wr, ex = make_layer(16, 24, 8, 2)
    x = gen.gen_x(shape, 40)
    r0 = L0.forward(x)
    cap = int(r0["counts"].max())
    for c in (cap, cap + 5):
        r = oracle.layer_from_gen(shape, wr, None, ex, capacity=c).forward(x)
        for key in ("y", "idx", "w", "counts", "offsets", "perm", "inv"):
            assert np.array_equal(r[key], r0[key]), (c, key)


@pytest.mark.parametrize("dtype,cap", [("f32", 3), ("bf16", 5), ("f32", 1)])
def test_capacity_forward_equals_dense_masked(dtype, cap):
    H, F, E, k, T = 16, 24, 6, 2, 25
    shape, _, wr, ex = make_layer(H, F, E, k, dtype=dtype)
    L = oracle.layer_from_gen(shape, wr, None, ex, capacity=cap)
    x = gen.gen_x(shape, T)
    r = L.forward(x)
    X = widen(x, dtype)
    logits = X @ widen(wr, dtype)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    assert (order == r["idx"]).all()
    sel = np.take_along_axis(logits, order, 1)
    g = np.exp(sel - sel[:, :1])
    gates = g / g.sum(1, keepdims=True)
    keep = _capacity_reference(order, E, cap).reshape(T, k)
    assert keep.sum() < T * k                                      # the capacity bites
    y = np.zeros((T, H))
    for e in range(E):
        Wg, Wu, Wd = (widen(m, dtype) for m in gen.expert_views(shape, ex, e))
        a = silu(X @ Wg.T) * (X @ Wu.T)
        if dtype == "bf16":
            a = np.vectorize(oracle.bf16_round)(a)
        ye = a @ Wd.T
        wcol = np.where((order == e) & keep, gates, 0.0).sum(1)      # unrenormalised weights
        y += wcol[:, None] * ye
    assert np.abs(r["y"] - y).max() <= 1e-12 * np.sqrt((y ** 2).mean())
    toks = np.array([0, 7, 24], np.int32)
    t = L.tokens(x, toks, keep=keep[toks].astype(np.int32))
    assert np.array_equal(t["y"], r["y"][toks])


# --- P8: algebraic properties --------------------------------------------


def _blob_with(shape, ex, fn):
    out = ex.copy()
    for e in range(shape.E):
        views = gen.expert_views(shape, out, e)
        fn(*views)
    return out


def test_scaling_and_zero_up_projection():
    shape, L, wr, ex = make_layer(16, 24, 8, 2)
    x = gen.gen_x(shape, 10)
    y = L.forward(x)["y"]

    def dbl(Wg, Wu, Wd):
        Wd *= 2

    y2 = oracle.layer_from_gen(shape, wr, None, _blob_with(shape, ex, dbl)).forward(x)["y"]
    assert np.array_equal(y2, 2 * y)

    def zero_u(Wg, Wu, Wd):
        Wu[:] = 0

    y0 = oracle.layer_from_gen(shape, wr, None, _blob_with(shape, ex, zero_u)).forward(x)["y"]
    assert not y0.any()


def test_token_permutation_equivariance():
    shape, L, wr, ex = make_layer(16, 24, 8, 2)
    x = gen.gen_x(shape, 17)
    r = L.forward(x)
    p = np.random.default_rng(0).permutation(17)
    rp = L.forward(x[p])
    assert np.array_equal(rp["y"], r["y"][p])
    assert np.array_equal(rp["counts"], r["counts"])


def test_expert_relabelling_invariance():
    shape, L, wr, ex = make_layer(16, 24, 8, 2)
    x = gen.gen_x(shape, 12)
    y = L.forward(x)["y"]
    sigma = np.random.default_rng(1).permutation(8)   # new expert i = old expert sigma[i]
    wr2 = wr[:, sigma]
    ex2 = np.zeros_like(ex)
    for i, old in enumerate(sigma):
        ex2[i * shape.stride:(i + 1) * shape.stride] = ex[old * shape.stride:(old + 1) * shape.stride]
    y2 = oracle.layer_from_gen(shape, wr2, None, ex2).forward(x)["y"]
    assert np.array_equal(y, y2)


# --- per-token path, override path, bf16 rounding, prenorm -----------------


def test_token_subset_matches_full_forward():
    shape, L, wr, ex = make_layer(32, 48, 16, 4, dtype="bf16", bias=gen.zipf_bias(16))
    x = gen.gen_x(shape, 40)
    r = L.forward(x)
    toks = [0, 7, 39, 7]
    s = L.tokens(x, toks)
    assert np.array_equal(s["y"], r["y"][toks])
    assert np.array_equal(s["idx"], r["idx"][toks])
    # overriding with the oracle's own choice changes nothing
    s2 = L.tokens(x, toks, idx_override=s["idx"])
    assert np.array_equal(s2["y"], s["y"])
    # a different expert set gives the masked sum over that set
    ov = np.array([[5, 3, 1, 0]] * 4, np.int32)
    s3 = L.tokens(x, toks, idx_override=ov)
    X = widen(x[toks], "bf16")
    lg = s3["logits"][:, [5, 3, 1, 0]]
    g = np.exp(lg - lg[:, :1])
    gates = g / g.sum(1, keepdims=True)
    want = sum(gates[:, j:j + 1] * np.stack([L.expert_ffn(e, X[n]) for n in range(4)])
               for j, e in enumerate([5, 3, 1, 0]))
    assert np.allclose(s3["y"], want, rtol=0, atol=1e-13 * np.abs(want).max())


def test_bf16_round():
    r = oracle.bf16_round
    assert r(1.0) == 1.0 and r(0.0) == 0.0 and r(-2.5) == -2.5
    assert r(1.0 + 2 ** -8) == 1.0                      # tie, even mantissa kept
    assert r(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6        # tie, rounds up to even
    assert r(1.0 + 2 ** -8 + 2 ** -30) == 1.0 + 2 ** -7
    assert r(-(1.0 + 3 * 2 ** -8)) == -(1.0 + 2 ** -6)
    # against the fp32 bit trick (textbook RNE) on fp32-representable values
    f = np.random.default_rng(0).normal(0, 3, 5000).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    b = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    want = b.astype(np.uint32).view(np.float32).astype(np.float64)
    got = np.array([r(float(v)) for v in f])
    assert np.array_equal(got, want)


def test_prenorm_closed_forms():
    ones = np.ones((1, 64), np.float32)
    out = gen.bf16_bits_to_f32(oracle.prenorm_bf16(ones))
    assert (out == 1.0).all()                            # 1/sqrt(1 + 1e-6) rounds to 1
    h = np.array([[3.0, 4.0]], np.float32)               # rms = sqrt(12.5)
    out = gen.bf16_bits_to_f32(oracle.prenorm_bf16(h)).astype(np.float64)
    # 3/sqrt(12.5) = 0.84853 -> nearest bf16 217/256; 4/sqrt(12.5) = 1.13137 -> 145/128
    assert out[0].tolist() == [217 / 256, 145 / 128]
    hr = np.random.default_rng(2).normal(0, 50, (4, 256)).astype(np.float32)
    o = gen.bf16_bits_to_f32(oracle.prenorm_bf16(hr)).astype(np.float64)
    assert np.allclose(np.sqrt((o ** 2).mean(1)), 1.0, atol=5e-3)
    assert (np.sign(o) == np.sign(hr)).all()
    o2 = gen.bf16_bits_to_f32(oracle.prenorm_bf16(hr * 4)).astype(np.float64)
    assert np.array_equal(o, o2)                         # scale invariance (eps negligible)


def test_invalid_arguments_rejected():
    with pytest.raises(RuntimeError):
        oracle.topk_softmax(np.zeros((2, 4)), 5)
    with pytest.raises(RuntimeError):
        oracle.topk_softmax(np.array([[0.0, np.nan, 1.0]]), 1)
    with pytest.raises(RuntimeError):
        oracle.dispatch(np.array([[0, 9]]), 4)
