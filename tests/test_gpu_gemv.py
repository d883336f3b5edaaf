"""The single-token path (T = 1) through the C ABI: matrix-vector kernels for
the expert FFN, with the combine folded into the down projection.

Every case is a T = 1 forward of a bf16 or uint8 layer whose hidden and FFN
widths pick one instantiation of the kernels (gate/up rows of 2, 4, 6 or 8
pieces of 1 KB; down rows of one to four chunks of 4, 6, 7 or 8 pieces),
checked against the oracle row by row; the folded combine must equal
the separate combine kernel bit for bit (plain and residual layers, the
residual updated in place); the streaming kernels, forced by flag, must give
the oracle's output too.
"""
import numpy as np
import pytest
import torch

import gen
import mixture_experts_amd as moe
from moe_cases import Case, U8Case, check_rows, to_dev

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


# u8, H, F, E, k, flags
CASES = [
    (False, 1024, 2048, 8, 2, 0),      # gate/up 2 pieces per row, down 1 chunk of 4
    (False, 2048, 4096, 8, 2, 0),      # 4; 1 x 8
    (False, 3072, 6144, 4, 2, 0),      # 6; 2 x 6
    (False, 4096, 8192, 4, 2, 0),      # 8; 2 x 8
    (False, 2048, 7168, 4, 2, 0),      # 4; 2 x 7
    (False, 1024, 14336, 4, 2, 0),     # 2; 4 x 7
    (False, 1024, 2048, 16, 8, 0),     # eight routed experts
    (False, 1024, 2048, 1, 1, 0),      # one expert: a dense SwiGLU FFN
    (False, 1024, 2048, 8, 2, moe.MOE_FLAG_GATE_RAW),
    (False, 1024, 2048, 8, 2, moe.MOE_FLAG_COMBINE_SEPARATE),
    (True, 2048, 4096, 8, 2, 0),       # 2; 1 x 4
    (True, 4096, 8192, 4, 2, 0),       # 4; 1 x 8
    (True, 6144, 12288, 2, 2, 0),      # 6; 2 x 6
    (True, 8192, 4096, 2, 2, 0),       # 8; 1 x 4
    (True, 2048, 14336, 4, 2, 0),      # 2; 2 x 7 (the Mixtral down width)
    (True, 2048, 16384, 2, 2, 0),      # 2; 2 x 8
    (True, 2048, 4096, 16, 8, 0),
    (True, 2048, 4096, 8, 2, moe.MOE_FLAG_COMBINE_SEPARATE),
]


def _case(u8, H, F, E, k, flags, max_tokens=1):
    shape = gen.LayerShape(f"g{H}_{F}_{E}_{k}", H=H, F=F, E=E, k=k, dtype="bf16")
    return shape, (U8Case(shape, max_tokens, flags) if u8 else Case(shape, max_tokens, flags=flags))


@pytest.mark.parametrize("u8,H,F,E,k,flags", CASES)
def test_gemv_forward(u8, H, F, E, k, flags):
    _log("gemv forward", u8, H, F, E, k, flags)
    shape, c = _case(u8, H, F, E, k, flags)
    x = gen.gen_x(shape, 1)
    y = c.forward(x)
    st = check_rows(c, x, np.arange(1), y, c.route(x)["idx"])
    _log("  ", st)
    assert np.array_equal(y, c.forward(x))  # bitwise reproducible
    c.close()


@pytest.mark.parametrize("u8", [False, True])
def test_gemv_many_calls(u8):
    """One layer sized for 64 tokens called with single tokens in turn (and a
    batch in between): each call's row against the oracle."""
    _log("gemv many calls", u8)
    shape, c = _case(u8, 2048, 4096, 8, 2, 0, max_tokens=64)
    for seed, T in ((1, 1), (2, 1), (3, 40), (4, 1), (5, 1)):
        x = gen.gen_x(shape, T, seed=seed)
        y = c.forward(x)
        check_rows(c, x, np.arange(T), y, c.route(x)["idx"])
    c.close()


@pytest.mark.parametrize("u8", [False, True])
@pytest.mark.parametrize("E", [4, 8])
def test_gemv_and_stream_kernels_agree(u8, E):
    """The streaming kernels at T = 1 (forced by flag) against the oracle, and
    within the bf16 tolerance of the matrix-vector kernels."""
    _log("gemv vs stream", u8, E)
    ys = []
    for fl in (0, moe.MOE_FLAG_PATH_STREAM):
        shape, c = _case(u8, 4096, 14336 if u8 else 7168, E, 2, fl)
        x = gen.gen_x(shape, 1)
        y = c.forward(x)
        check_rows(c, x, np.arange(1), y, c.route(x)["idx"])
        ys.append(y)
        c.close()
    rms = np.sqrt(np.mean(ys[0].astype(np.float64) ** 2))
    assert np.abs(ys[0] - ys[1]).max() <= 2e-2 * rms


def _device_layers(shape, flags, u8):
    """Two layers on the same device weights: folded and separate combine."""
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
    mk = lambda f: moe.MoELayer(shape.H, shape.F, shape.E, shape.k, 1, moe.MOE_BF16, d_wr, ex, st,
                                d_b, f, expert_format=fmt)
    return mk(flags), mk(flags | moe.MOE_FLAG_COMBINE_SEPARATE), (d_wr, d_b, ex)


@pytest.mark.parametrize("u8,flags", [(False, 0), (True, 0),
                                      (False, moe.MOE_FLAG_RESIDUAL_PRENORM),
                                      (True, moe.MOE_FLAG_RESIDUAL_PRENORM),
                                      (False, moe.MOE_FLAG_GATE_RAW)])
def test_gemv_folded_combine_is_bit_identical(u8, flags):
    _log("gemv fold", u8, flags)
    shape = gen.LayerShape("gfold", H=4096, F=7168 if not u8 else 14336, E=8, k=2, dtype="bf16")
    a, b, keep = _device_layers(shape, flags, u8)
    prenorm = bool(flags & moe.MOE_FLAG_RESIDUAL_PRENORM)
    outs = []
    for layer in (a, b):
        if prenorm:  # the residual stream updated in place: y aliases x
            h = torch.from_numpy(gen.normal(0, 0, gen.T_X, shape.H, 1.0, "f32")
                                 .reshape(1, shape.H)).cuda()
            layer.forward(h, h)
        else:
            x = to_dev(gen.gen_x(shape, 1))
            h = torch.empty((1, shape.H), dtype=torch.float32, device="cuda")
            layer.forward(x, h)
        torch.cuda.synchronize()
        outs.append(h.cpu().numpy())
    assert np.isfinite(outs[0]).all()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    a.close()
    b.close()
    del keep
