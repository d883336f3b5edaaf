"""Stacked layers (residual inside the forward call, parameter-free RMS
normalisation of the branch input): device input generation, graph replay,
and per-layer parity at the 32-layer Mixtral-shaped size.
"""
import numpy as np
import pytest
import torch

import gen
import mixture_experts_amd as moe
import oracle
from moe_cases import check_rows, to_dev

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dtype,seed,layer,tensor,idx0,n", [
    ("bf16", 0, 0, gen.T_WG, 0, 100_000), ("bf16", 0, 31, gen.T_WD, 3 * 2 ** 31 + 5, 70_001),
    ("f32", 7, 2, gen.T_X, 12345, 50_000), ("bf16", 3, 5, gen.T_WU, 2 ** 33, 4097)])
def test_device_generator_matches_host(dtype, seed, layer, tensor, idx0, n):
    host = gen.normal(seed, layer, tensor, n, 0.02, dtype, idx0=idx0)
    d = torch.empty(n, dtype=torch.int16 if dtype == "bf16" else torch.float32, device="cuda")
    gen.normal_device(seed, layer, tensor, n, 0.02, dtype, d.data_ptr(), idx0=idx0,
                      stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    dev = d.cpu().numpy().view(host.dtype)
    assert np.array_equal(dev, host)


class Stack:
    """A stack of bf16 layers whose experts share one contiguous device buffer
    (layer l's expert e at blob + (l*E + e)*stride), generated on the device."""

    def __init__(self, shape, nlayers, max_tokens):
        self.shape, self.n = shape, nlayers
        st = torch.cuda.current_stream().cuda_stream
        self.blob = torch.empty(nlayers * shape.E * shape.stride, dtype=torch.uint8, device="cuda")
        self.routers = []
        self.layers = []
        for l in range(nlayers):
            base = self.blob.data_ptr() + l * shape.E * shape.stride
            gen.experts_device(shape, base, layer=l, stream=st)
            wr = to_dev(gen.gen_router(shape, layer=l))
            self.routers.append(wr)
            self.layers.append(moe.MoELayer(shape.H, shape.F, shape.E, shape.k, max_tokens,
                                            moe.MOE_BF16, wr, base, shape.stride,
                                            flags=moe.MOE_FLAG_RESIDUAL_PRENORM))
        torch.cuda.synchronize()

    def forward(self, h, T, stream=None):
        for L in self.layers:
            moe.moe_forward(L.handle, h, T, h, stream)

    def host_experts(self, l, experts):
        return gen.gen_experts(self.shape, layer=l, experts=experts)

    def close(self):
        for L in self.layers:
            L.close()


@pytest.mark.parametrize("T", [12, 64])  # 64: separate branch normalisation, several-workgroup route
def test_stack_graph_replay_matches_eager(T):
    shape = gen.LayerShape("gstack", H=512, F=256, E=8, k=2, dtype="bf16")
    s = Stack(shape, 4, T)
    x0 = torch.from_numpy(gen.normal(0, 0, gen.T_X, T * shape.H, 1.0, "f32")).cuda().view(T, shape.H)
    h = torch.empty_like(x0)
    h.copy_(x0)
    s.forward(h, T)
    torch.cuda.synchronize()
    eager = h.cpu().numpy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream
        h.copy_(x0)
        s.forward(h, T)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h.copy_(x0)
        s.forward(h, T)
    other = torch.from_numpy(gen.normal(1, 0, gen.T_X, T * shape.H, 1.0, "f32")).cuda().view(T, shape.H)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(h.cpu().numpy(), eager), f"replay {rep}"
        # eager work on the same layers between replays
        h2 = other.clone()
        s.forward(h2, T)
        torch.cuda.synchronize()
    s.close()


@pytest.mark.parametrize("T", [1, 4, 16, 64])
def test_mixtral_stack_32_layers_teacher_forced(T):
    """The 32-layer Mixtral-shaped stack (90 GB of experts in one buffer):
    each sampled layer's branch output against the oracle fed with the GPU's
    residual stream at that layer's input."""
    shape = gen.MIXTRAL
    s = Stack(shape, 32, 64)
    h = torch.from_numpy(gen.normal(0, 0, gen.T_X, T * shape.H, 1.0, "f32")).cuda().view(T, shape.H)
    ins = []
    for l, L in enumerate(s.layers):
        ins.append(h.cpu().numpy())
        moe.moe_forward(L.handle, h, T, h)
    torch.cuda.synchronize()
    outs = ins[1:] + [h.cpu().numpy()]
    assert np.isfinite(outs[-1]).all()
    rms_last = float(np.sqrt(np.mean(outs[-1].astype(np.float64) ** 2)))
    _log(f"  T={T}: residual stream rms after 32 layers {rms_last:.3f}")
    for l in (0, 17, 31):
        h_in = ins[l]
        r = s.layers[l].route(to_dev(h_in), T)
        torch.cuda.synchronize()
        idx = r["idx"].cpu().numpy().reshape(T, shape.k)
        xt = oracle.prenorm_bf16(h_in)
        ex = s.host_experts(l, sorted(set(idx.ravel().tolist())))
        orc = oracle.layer_from_gen(shape, gen.gen_router(shape, layer=l), None, ex)

        class C:  # what check_rows needs
            pass
        c = C()
        c.shape, c.orc = shape, orc
        branch = outs[l].astype(np.float64) - h_in.astype(np.float64)
        st = check_rows(c, xt, np.arange(T), branch, idx)
        _log(f"  layer {l}: {st}")
    s.close()
