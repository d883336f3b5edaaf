"""Exact logit ties through the small-batch route kernels (T <= 64), which
route and dispatch from their own logits and are never given logits from
outside: the tie rule (equal logits: the lower expert index first) and the
softmax over the picks must come out of every one of them.

Ties are planted in the router itself:
  * a zero router: every logit is (signed) zero, so every token takes
    experts 0..k-1 with weight 1/k;
  * a router whose columns come in identical pairs (2m, 2m+1): the two
    logits of a pair are the same sum in the same order on either side, so
    they tie exactly, on the GPU and in the oracle.

Kernels reached (bf16 layers): the single-token route (T = 1, E = 8 or 16,
H a multiple of 1024), the one-workgroup-per-16-tokens route (E <= 16,
T <= 64), the split-hidden route (E = 64), and their residual-stream
variants through the forward.
"""
import numpy as np
import pytest
import torch

import gen
import mixture_experts_amd as moe
import oracle
from moe_cases import Case, check_rows, near_tie_gap

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


def tie_router(shape, kind: str) -> np.ndarray:
    """[H][E] bf16 bit patterns: all zero, or columns in identical pairs."""
    if kind == "zero":
        return np.zeros((shape.H, shape.E), np.uint16)
    wr = gen.gen_router(shape).reshape(shape.H, shape.E).copy()
    wr[:, 1::2] = wr[:, 0::2]
    return wr


ROUTE_CASES = [
    # H, E, k, T: kernel
    (1024, 8, 2, 1),    # single-token route, one 16-byte router row
    (1024, 16, 4, 1),   # single-token route, two 16-byte router rows
    (4096, 8, 2, 1),    # single-token route at the Mixtral width
    (1024, 8, 2, 4),    # one workgroup
    (1024, 16, 4, 4),
    (1024, 8, 2, 40),   # one workgroup per 16 tokens, the last one dispatches
    (1024, 16, 4, 40),
    (512, 16, 8, 64),
    (1024, 64, 2, 1),   # split-hidden route (many experts)
    (1024, 64, 2, 33),
    (2048, 64, 8, 64),
    (256, 8, 2, 7),     # H not a multiple of 512: split-hidden route with 8 experts
    # batches beyond 64 tokens: logits and top-k of 32-token tiles in one launch
    (1024, 8, 2, 100),
    (2048, 64, 4, 300),
    (1024, 256, 16, 70),  # k beyond 8: selection by ranks
]


@pytest.mark.parametrize("H,E,k,T", ROUTE_CASES)
def test_zero_router_routes_to_first_k_experts(H, E, k, T):
    """All logits zero: slots 0..k-1 take experts 0..k-1, each weight 1/k."""
    shape = gen.LayerShape(f"tz{H}_{E}_{k}", H=H, F=128, E=E, k=k, dtype="bf16")
    _log("zero router", H, E, k, T)
    c = Case(shape, T, router=tie_router(shape, "zero"), bias=None,
             experts=gen.gen_experts(shape))
    x = gen.gen_x(shape, T)
    r = c.route(x)
    idx = r["idx"].reshape(T, k)
    assert np.array_equal(idx, np.tile(np.arange(k, dtype=np.int32), (T, 1)))
    assert np.array_equal(r["w"], np.full(T * k, np.float32(1.0 / k), np.float32))
    counts, offsets, perm, inv = oracle.dispatch(idx, E)
    for key, ref in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        assert np.array_equal(r[key], ref), key
    c.close()


@pytest.mark.parametrize("H,E,k,T", ROUTE_CASES)
def test_paired_router_columns_tie_to_lower_index(H, E, k, T):
    """Columns 2m and 2m+1 identical, k even: the picks come in whole pairs,
    the lower index first, the two weights of a pair equal; apart from near
    ties between different pairs the indices equal the oracle's, and the
    weights match the oracle's gates at those picks (to the accuracy of the
    GPU's own fp32 logits: 1e-5 absolute)."""
    shape = gen.LayerShape(f"tp{H}_{E}_{k}", H=H, F=128, E=E, k=k, dtype="bf16")
    _log("paired router", H, E, k, T)
    wr = tie_router(shape, "pairs")
    c = Case(shape, T, router=wr, bias=None, experts=gen.gen_experts(shape))
    x = gen.gen_x(shape, T)
    r = c.route(x)
    idx = r["idx"].reshape(T, k)
    w = r["w"].reshape(T, k)
    assert np.all(idx[:, 0::2] % 2 == 0) and np.array_equal(idx[:, 1::2], idx[:, 0::2] + 1)
    assert np.array_equal(w[:, 0::2], w[:, 1::2])
    lg = c.orc.logits(x)
    assert np.array_equal(lg[:, 0::2], lg[:, 1::2])  # the oracle ties exactly too
    idx_o, w_o = oracle.topk(lg, k)
    gap = near_tie_gap(lg, k)  # k even: slots k-1 and k belong to different pairs
    far = gap >= 1e-3
    _log(f"  near ties between pairs {int((~far).sum())} / {T}")
    assert np.array_equal(idx[far], idx_o[far])
    # weights: the oracle's gates of the GPU's picks
    w_ref = np.empty((T, k))
    for t in range(T):
        z = np.exp(lg[t, idx[t]] - lg[t, idx[t, 0]])
        w_ref[t] = z / z.sum()
    assert np.abs(w.astype(np.float64) - w_ref).max() <= 1e-5
    counts, offsets, perm, inv = oracle.dispatch(idx, E)
    for key, ref in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        assert np.array_equal(r[key], ref), key
    c.close()


FWD_CASES = [
    # H, F, E, k, T, flags
    (1024, 256, 8, 2, 1, 0),
    (1024, 256, 16, 4, 4, 0),
    (1024, 256, 8, 2, 40, 0),
    (1024, 256, 64, 2, 33, 0),
    (1024, 256, 8, 2, 1, moe.MOE_FLAG_RESIDUAL_PRENORM),
    (1024, 256, 16, 4, 16, moe.MOE_FLAG_RESIDUAL_PRENORM),
    (1024, 256, 8, 2, 40, moe.MOE_FLAG_RESIDUAL_PRENORM),
    # single tokens on the matrix-vector kernels
    (1024, 2048, 8, 2, 1, 0),
    (1024, 2048, 16, 4, 1, 0),
    (1024, 2048, 8, 2, 1, moe.MOE_FLAG_RESIDUAL_PRENORM),
]


@pytest.mark.parametrize("kind", ["zero", "pairs"])
@pytest.mark.parametrize("H,F,E,k,T,flags", FWD_CASES)
def test_forward_with_tied_router(kind, H, F, E, k, T, flags):
    """The whole layer through the same kernels (including the routes that
    normalise the residual stream themselves): every row against the oracle."""
    shape = gen.LayerShape(f"tf{H}_{F}_{E}_{k}", H=H, F=F, E=E, k=k, dtype="bf16")
    _log("forward tied router", kind, H, F, E, k, T, flags)
    c = Case(shape, T, flags=flags, router=tie_router(shape, kind), bias=None,
             experts=gen.gen_experts(shape))
    if flags & moe.MOE_FLAG_RESIDUAL_PRENORM:
        h = gen.normal(0, 0, gen.T_X, T * H, 1.0, "f32").reshape(T, H)
        d = torch.from_numpy(h.copy()).cuda()
        r = c.layer.route(d, T)
        c.layer.forward(d, d)  # in place: y = h + MoE(norm(h))
        torch.cuda.synchronize()
        branch = d.cpu().numpy().astype(np.float64) - h.astype(np.float64)
        xt = oracle.prenorm_bf16(h)
        idx = r["idx"].cpu().numpy()
        st = check_rows(c, xt, np.arange(T), branch, idx)
    else:
        x = gen.gen_x(shape, T)
        y = c.forward(x)
        idx = c.route(x)["idx"]
        st = check_rows(c, x, np.arange(T), y, idx)
    if kind == "zero":
        assert np.array_equal(idx.reshape(T, k), np.tile(np.arange(k, dtype=np.int32), (T, 1)))
    _log("  ", st)
    c.close()
