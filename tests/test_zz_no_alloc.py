"""moe_forward_noalloc (workspace in the library's static device array, no
allocation) against moe_forward through a created layer: two calls in a row,
the second with a smaller batch, each compared with moe_forward on the same
input.  Kernels that are the same on both give the same bits; where the
grouped down projection runs (no tail split without a workspace for it) the
outputs agree within the bf16 bar, and both match the oracle."""
import numpy as np
import pytest
import torch

import gen
import mixture_experts_amd as moe
from moe_cases import Case, check_rows, to_dev

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


G = moe.MOE_FLAG_PATH_GROUPED
CASES = [
    # name, shape, flags, (T1, T2), bit-exact
    ("mixtral_decode", gen.MIXTRAL, 0, (16, 4), True),
    ("stream_separate_combine", gen.LayerShape("na1", H=512, F=1024, E=8, k=2, dtype="bf16"),
     moe.MOE_FLAG_COMBINE_SEPARATE, (40, 3), True),
    ("qwen_shape", gen.QWEN, 0, (512, 100), True),
    ("grouped_tail", gen.LayerShape("na2", H=256, F=2048, E=8, k=2, dtype="bf16"), G,
     (600, 300), False),
    ("grouped_large_split_h", gen.LayerShape("na3", H=512, F=384, E=4, k=2, dtype="bf16"), 0,
     (700, 65), False),
    ("f32", gen.TINY, 0, (32, 5), True),
]


def _desc(c: Case, max_tokens: int, flags: int):
    s = c.shape
    return moe.make_desc(s.H, s.F, s.E, s.k, max_tokens,
                         moe.MOE_F32 if s.dtype == "f32" else moe.MOE_BF16, c.d_router,
                         c.d_experts, s.stride, c.d_bias, flags)


@pytest.mark.parametrize("name,shape,flags,Ts,exact", CASES)
def test_noalloc_matches_forward(name, shape, flags, Ts, exact):
    _log("noalloc", name, Ts)
    c = Case(shape, Ts[0], flags=flags)
    desc = _desc(c, Ts[0], flags)
    for i, T in enumerate(Ts):
        x_np = gen.gen_x(shape, T, seed=100 + i)
        x = to_dev(x_np)
        y_ref = torch.empty((T, shape.H), dtype=torch.float32, device="cuda")
        y_na = torch.full((T, shape.H), float("nan"), dtype=torch.float32, device="cuda")
        c.layer.forward(x, y_ref)
        moe.moe_forward_noalloc(desc, x, T, y_na)
        torch.cuda.synchronize()
        a, b = y_ref.cpu().numpy(), y_na.cpu().numpy()
        assert np.isfinite(b).all()
        rms = float(np.sqrt(np.mean(a.astype(np.float64) ** 2)))
        rel = float(np.abs(a.astype(np.float64) - b).max()) / rms
        _log(f"  T={T}: max |noalloc - forward| / rms = {rel:.3e}")
        if exact:
            assert np.array_equal(a, b)
        else:
            assert rel <= 1e-2
            st = check_rows(c, x_np, np.arange(T), b, c.route(x_np)["idx"])
            _log("   oracle", st)
    c.close()


def test_noalloc_residual_in_place():
    """Stacked-layer mode, y aliasing x: T = 40, then T = 1."""
    shape = gen.LayerShape("na4", H=1024, F=256, E=8, k=2, dtype="bf16")
    fl = moe.MOE_FLAG_RESIDUAL_PRENORM
    c = Case(shape, 40, flags=fl)
    desc = _desc(c, 40, fl)
    for T in (40, 1):
        h = gen.normal(T, 0, gen.T_X, T * shape.H, 1.0, "f32").reshape(T, shape.H)
        d1, d2 = torch.from_numpy(h.copy()).cuda(), torch.from_numpy(h.copy()).cuda()
        c.layer.forward(d1, d1)
        moe.moe_forward_noalloc(desc, d2, T, d2)
        torch.cuda.synchronize()
        assert np.array_equal(d1.cpu().numpy(), d2.cpu().numpy())
    c.close()


def test_noalloc_rejects_a_workspace_beyond_the_array():
    """Mixtral-shaped layer at T = 4096 needs far more than the array: a
    clear error, and nothing runs (y keeps its contents)."""
    shape = gen.MIXTRAL
    T = 4096
    dummy_w = torch.zeros(shape.H * shape.E, dtype=torch.int16, device="cuda")
    dummy_e = torch.zeros(256, dtype=torch.uint8, device="cuda")
    desc = moe.make_desc(shape.H, shape.F, shape.E, shape.k, T, moe.MOE_BF16, dummy_w,
                         dummy_e, shape.stride)
    x = torch.zeros((T, shape.H), dtype=torch.int16, device="cuda")
    y = torch.full((T, shape.H), 7.0, dtype=torch.float32, device="cuda")
    rc = moe.lib().moe_forward_noalloc(desc, x.data_ptr(), T, y.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
    assert rc == moe.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
    # T above max_tokens: invalid argument
    rc = moe.lib().moe_forward_noalloc(desc, x.data_ptr(), T + 1, y.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
    assert rc == moe.MOE_ERR_INVALID_ARG
