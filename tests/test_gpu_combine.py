"""Step 5 folded into the streaming down projection, through the C ABI.

Where every 16-row hidden slice can have a workgroup of its own, the down
projection keeps the k expert rows of each token in LDS and writes y itself,
with the combine's operations in the combine's order.  A layer created with
MOE_FLAG_COMBINE_SEPARATE runs the separate combine kernel instead; the two
must agree bit for bit (plain and residual layers, dropped pairs, bf16 and
uint8 experts), and the folded one must match the oracle."""
import numpy as np
import pytest
import torch

import gen
import mixture_experts_amd as moe
from moe_cases import Case, check_rows, to_dev

pytestmark = pytest.mark.gpu

# 8192 / 16 = 512 hidden slices: more than the compute units of any one GPU
SHAPE = gen.LayerShape("fold", H=8192, F=256, E=8, k=2, dtype="bf16")


def _log(*a):
    print(*a, flush=True)


def _pair(shape, T, flags=0, capacity=0, u8=False):
    """Two layers on the same weights: folded combine and separate combine."""
    wr, b = gen.gen_router(shape), gen.gen_bias(shape)
    d_wr = to_dev(wr)
    d_b = None if b is None else to_dev(b)
    ex = torch.empty(shape.E * shape.stride, dtype=torch.uint8, device="cuda")
    gen.experts_device(shape, ex.data_ptr(), stream=torch.cuda.current_stream().cuda_stream)
    st, fmt = shape.stride, moe.MOE_EXPERT_DTYPE
    if u8:
        st = moe.u8_stride(shape.H, shape.F)
        q = torch.zeros(shape.E * st, dtype=torch.uint8, device="cuda")
        moe.moe_quantize_experts_u8(ex, shape.stride, shape.E, shape.H, shape.F, q, st)
        ex, fmt = q, moe.MOE_EXPERT_U8
    torch.cuda.synchronize()
    mk = lambda f: moe.MoELayer(shape.H, shape.F, shape.E, shape.k, T, moe.MOE_BF16, d_wr, ex, st,
                                d_b, f, expert_capacity=capacity, expert_format=fmt)
    return mk(flags), mk(flags | moe.MOE_FLAG_COMBINE_SEPARATE), (d_wr, d_b, ex)


def _run(layer, x, T, shape, inplace):
    if inplace:  # residual stream updated in place: y aliases x
        h = x.clone()
        layer.forward(h, h)
        torch.cuda.synchronize()
        return h.cpu().numpy()
    y = torch.empty((T, shape.H), dtype=torch.float32, device="cuda")
    layer.forward(x, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("T,flags,capacity,u8", [
    (1, 0, 0, False), (3, 0, 0, False), (16, 0, 0, False), (64, 0, 0, False),
    (128, 0, 0, False),                                   # T*k = 256 pairs, the largest folded
    (200, 0, 0, False),                                   # beyond it: both separate
    (16, 0, 3, False),                                    # pairs dropped by the capacity
    (1, moe.MOE_FLAG_RESIDUAL_PRENORM, 0, False), (16, moe.MOE_FLAG_RESIDUAL_PRENORM, 0, False),
    (1, moe.MOE_FLAG_GATE_RAW, 0, False),
    (1, 0, 0, True), (2, moe.MOE_FLAG_RESIDUAL_PRENORM, 0, True),
])
def test_folded_combine_is_bit_identical(T, flags, capacity, u8):
    _log("fold", T, flags, capacity, u8)
    shape = SHAPE
    a, b, keep = _pair(shape, T, flags, capacity, u8)
    prenorm = bool(flags & moe.MOE_FLAG_RESIDUAL_PRENORM)
    if prenorm:
        x = torch.from_numpy(gen.normal(0, 0, gen.T_X, T * shape.H, 1.0, "f32")
                             .reshape(T, shape.H)).cuda()
    else:
        x = to_dev(gen.gen_x(shape, T))
    ya = _run(a, x, T, shape, prenorm)
    yb = _run(b, x, T, shape, prenorm)
    assert np.isfinite(ya).all()
    assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32))
    a.close()
    b.close()
    del keep


@pytest.mark.parametrize("T", [1, 5, 64])
def test_folded_combine_against_the_oracle(T):
    _log("fold oracle", T)
    c = Case(SHAPE, T)
    x = gen.gen_x(SHAPE, T)
    y = c.forward(x)
    r = c.route(x)
    check_rows(c, x, np.arange(T), y, r["idx"])
    c.close()
