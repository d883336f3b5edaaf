"""Forward calls captured in a HIP graph and replayed: every replay equals the
eager result bit for bit, with eager work of the same layer (on other inputs)
between the replays.  One case per launch sequence: the single-token route
with the folded combine (plain, residual, uint8 experts, rows of 4 and 8 KB),
the router and
dispatch kernels with the grouped GEMMs (one-workgroup dispatch, and the
histogram / scan / scatter dispatch of 16384 pairs), the LDS-staged router
with the streaming kernels, and the route of several workgroups (17 to 64
tokens) with the streaming kernels, bf16 and uint8."""
import numpy as np
import pytest
import torch

import gen
import mixture_experts_amd as moe
from moe_cases import to_dev

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


CASES = [
    # H, F, E, k, T, flags, uint8 experts
    (4096, 256, 8, 2, 1, 0, False),
    (4096, 256, 8, 2, 1, moe.MOE_FLAG_RESIDUAL_PRENORM, False),
    (4096, 256, 8, 2, 1, 0, True),
    (2048, 2048, 8, 2, 1, 0, False),
    (4096, 4096, 8, 2, 1, moe.MOE_FLAG_RESIDUAL_PRENORM, True),
    (1024, 512, 8, 2, 700, moe.MOE_FLAG_PATH_GROUPED, False),
    (2048, 256, 64, 2, 200, 0, False),
    (2048, 1408, 128, 4, 4096, 0, False),
    # T = 17..64: the route of several workgroups whose last one dispatches
    # and resets the completion counter (every replay must find it at zero)
    (2048, 512, 8, 2, 48, 0, False),
    (2048, 512, 8, 2, 64, 0, True),
]


@pytest.mark.parametrize("H,F,E,k,T,flags,u8", CASES)
def test_graph_replays_match_eager(H, F, E, k, T, flags, u8):
    _log("graph", H, F, E, k, T, flags, u8)
    shape = gen.LayerShape(f"g{H}_{F}_{E}", H=H, F=F, E=E, k=k, dtype="bf16")
    st0 = torch.cuda.current_stream()
    d_wr = to_dev(gen.gen_router(shape))
    ex = torch.empty(shape.E * shape.stride, dtype=torch.uint8, device="cuda")
    gen.experts_device(shape, ex.data_ptr(), stream=st0.cuda_stream)
    stride, fmt = shape.stride, moe.MOE_EXPERT_DTYPE
    if u8:
        stride = moe.u8_stride(H, F)
        q = torch.zeros(E * stride, dtype=torch.uint8, device="cuda")
        moe.moe_quantize_experts_u8(ex, shape.stride, E, H, F, q, stride)
        ex, fmt = q, moe.MOE_EXPERT_U8
    torch.cuda.synchronize()
    layer = moe.MoELayer(H, F, E, k, T, moe.MOE_BF16, d_wr, ex, stride, None, flags,
                         expert_format=fmt)
    prenorm = bool(flags & moe.MOE_FLAG_RESIDUAL_PRENORM)
    if prenorm:
        x0 = torch.from_numpy(gen.normal(0, 0, gen.T_X, T * H, 1.0, "f32").reshape(T, H)).cuda()
        other = torch.from_numpy(gen.normal(1, 0, gen.T_X, T * H, 1.0, "f32").reshape(T, H)).cuda()
    else:
        x0 = to_dev(gen.gen_x(shape, T))
        other = to_dev(gen.gen_x(shape, T, seed=1))
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    h = torch.empty((T, H), dtype=torch.float32, device="cuda")

    def step(stream):
        if prenorm:  # the residual stream, updated in place
            h.copy_(x0)
            moe.moe_forward(layer.handle, h, T, h, stream)
        else:
            moe.moe_forward(layer.handle, x0, T, y, stream)

    out = h if prenorm else y
    step(st0.cuda_stream)
    torch.cuda.synchronize()
    eager = out.cpu().numpy()
    side = torch.cuda.Stream()
    side.wait_stream(st0)
    with torch.cuda.stream(side):  # warm up on the capture stream
        step(side.cuda_stream)
    st0.wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream().cuda_stream)
    y2 = torch.empty((T, H), dtype=torch.float32, device="cuda")
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), eager.view(np.uint32)), rep
        # eager work of the same layer between the replays
        if prenorm:
            h2 = other.clone()
            moe.moe_forward(layer.handle, h2, T, h2, st0.cuda_stream)
        else:
            moe.moe_forward(layer.handle, other, T, y2, st0.cuda_stream)
        torch.cuda.synchronize()
    assert np.isfinite(eager).all()
    del g
    layer.close()
