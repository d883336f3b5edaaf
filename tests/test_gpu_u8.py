"""uint8 expert weights on the GPU through the C ABI: the quantiser bit for
bit against the oracle's, and layers on uint8 experts against the oracle's
layer on the same (dequantised) experts."""
import numpy as np
import pytest
import torch

import gen
import mixture_experts_amd as moe
import oracle
from moe_cases import U8Case, check_rows, quantize_on_gpu, to_dev

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("H,F,E,seed", [(256, 384, 3, 0), (512, 256, 2, 1), (16, 32, 5, 2)])
def test_quantizer_bit_exact(H, F, E, seed):
    _log("quantize", H, F, E)
    shape = gen.LayerShape("q", H=H, F=F, E=E, k=1, dtype="bf16", seed=seed)
    ex = gen.gen_experts(shape)
    # plant: exact zeros, negative zeros, an all-zero matrix, a one-signed matrix
    per = H * F
    v = ex.view(np.uint16)
    v[:per * 3:37] = 0
    v[5:per * 3:41] = 0x8000
    e1 = shape.stride // 2
    v[e1:e1 + per] = 0                                  # expert 1: Wg all zero
    v[e1 + per:e1 + 2 * per] &= 0x7FFF                  # expert 1: Wu non-negative
    d_u8, st = quantize_on_gpu(shape, to_dev(ex))
    ref = oracle.quantize_experts_u8(ex, shape.stride, E, H, F, st)
    got = d_u8.cpu().numpy()
    for e in range(E):
        blk = slice(e * st, e * st + 3 * per + 64)     # codes and parameter block
        assert np.array_equal(got[blk], ref[blk]), e


def test_quantizer_bit_exact_mixtral_expert():
    shape = gen.MIXTRAL
    e = 5
    ex = gen.gen_experts(shape, experts=[e])
    one = ex[e * shape.stride:(e + 1) * shape.stride]
    d_u8, st = quantize_on_gpu(shape, to_dev(one), E=1)
    ref = oracle.quantize_experts_u8(one, shape.stride, 1, shape.H, shape.F, st)
    got = d_u8.cpu().numpy()
    n = 3 * shape.H * shape.F + 64
    assert np.array_equal(got[:n], ref[:n])


U8_SMALL = [
    # H, F, E, k, T, flags
    (256, 256, 8, 2, 1, 0),
    (256, 256, 8, 2, 5, 0),
    (1024, 256, 8, 2, 64, 0),
    (512, 384, 4, 2, 300, 0),          # several token passes; F % 256 != 0 (128-wide chunks)
    (256, 640, 16, 4, 100, 0),
    (256, 128, 64, 8, 60, 0),
    (512, 256, 8, 2, 40, moe.MOE_FLAG_GATE_RAW),
    (768, 256, 3, 1, 1100, 0),         # a large batch on the streaming kernels
    # K % 512 == 0: the item sizes chosen per batch (1, 4, 16 rows per expert)
    (512, 512, 8, 2, 1, 0),
    (512, 512, 8, 2, 4, 0),
    (512, 512, 8, 2, 16, 0),
    (512, 512, 8, 2, 64, 0),
]


@pytest.mark.parametrize("H,F,E,k,T,flags", U8_SMALL)
def test_u8_forward_small(H, F, E, k, T, flags):
    _log("u8 forward", H, F, E, k, T, flags)
    shape = gen.LayerShape(f"u{H}_{F}_{E}_{k}", H=H, F=F, E=E, k=k, dtype="bf16")
    c = U8Case(shape, T, flags)
    # the codes are the oracle quantiser's
    src = gen.gen_experts(shape)
    assert np.array_equal(c.u8, oracle.quantize_experts_u8(src, shape.stride, E, H, F, c.st))
    x = gen.gen_x(shape, T)
    y = c.forward(x)
    r = c.route(x)
    st = check_rows(c, x, np.arange(T), y, r["idx"])
    _log("  ", st)
    assert np.array_equal(y, c.forward(x))
    c.close()


@pytest.mark.parametrize("T,nsample", [(1, None), (4, None), (16, 8), (64, 8)])
def test_u8_mixtral_decode(T, nsample):
    _log("u8 mixtral decode", T)
    shape = gen.MIXTRAL
    c = U8Case(shape, T)
    x = gen.gen_x(shape, T)
    y = c.forward(x)
    r = c.route(x)
    idx = r["idx"].reshape(T, shape.k)
    if nsample is None:
        toks = np.arange(T)
    else:
        rng = np.random.default_rng(T)
        toks = np.unique(np.concatenate([[0, T - 1], rng.choice(T, nsample, False)]))
    st = check_rows(c, x, toks, y[toks], idx[toks])
    _log("  ", st)
    c.close()


# T = 1: the single-token route forms the normalisation itself and the
# matrix-vector kernels run (H and F multiples of 1 KB of codes); T = 4: the
# normalisation folded into a one-workgroup route; T = 24, 64: a separate
# normalisation launch and the route of several workgroups
@pytest.mark.parametrize("H,F,T", [(512, 512, 24), (1024, 1024, 1), (1024, 1024, 4),
                                   (1024, 1024, 64)])
def test_u8_residual_stack_teacher_forced(H, F, T):
    """Three stacked uint8 layers in place (RESIDUAL_PRENORM: the normalised
    bf16 branch input is what the uint8 kernels read in fp16), each checked
    against the oracle fed with the GPU's residual stream at that layer."""
    _log("u8 residual stack", H, F, T)
    shape = gen.LayerShape("u8stack", H=H, F=F, E=8, k=2, dtype="bf16")
    cases = [U8Case(shape, T, moe.MOE_FLAG_RESIDUAL_PRENORM, layer=l) for l in range(3)]
    h = torch.from_numpy(gen.normal(0, 0, gen.T_X, T * shape.H, 1.0, "f32").reshape(T, shape.H)).cuda()
    for c in cases:
        h_in = h.cpu().numpy()
        c.layer.forward(h, h)
        torch.cuda.synchronize()
        h_out = h.cpu().numpy()
        xt = oracle.prenorm_bf16(h_in)
        r = c.layer.route(torch.from_numpy(h_in).cuda(), T)
        torch.cuda.synchronize()
        branch = h_out.astype(np.float64) - h_in.astype(np.float64)
        st = check_rows(c, xt, np.arange(T), branch, r["idx"].cpu().numpy())
        _log("  ", st)
    for c in cases:
        c.close()


def test_u8_close_to_the_bf16_layer():
    """Quantisation error of the scheme itself, for the record: the uint8 layer
    against the bf16 layer it was made from (not a parity bar)."""
    shape = gen.LayerShape("cmp", H=1024, F=512, E=8, k=2, dtype="bf16")
    T = 64
    c = U8Case(shape, T)
    x = gen.gen_x(shape, T)
    y8 = c.forward(x)
    ref = oracle.layer_from_gen(shape, c.router, c.bias, gen.gen_experts(shape)).forward(x)
    rms = np.sqrt((ref["y"] ** 2).mean())
    rel = np.abs(y8 - ref["y"]).max() / rms
    _log(f"  uint8 vs bf16 layer: max |diff| / rms = {rel:.3e}")
    assert rel < 0.1
    c.close()
