"""GPU parity of libmoe against the fp64 CPU oracle, through the C ABI.

Routing (indices, counts, offsets, permutation, inverse) is compared bit for
bit when both sides are given the same fp32 logits; end to end, indices match
except at near ties; outputs are compared with the bars of moe_cases.
"""
import numpy as np
import pytest
import torch

import gen
import mixture_experts_amd as moe
import oracle
from moe_cases import Case, check_rows, near_tie_gap, to_dev

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


def routing_reference(logits32: np.ndarray, E: int, k: int, gate: str = "softmax",
                      capacity: int = 0):
    idx, w = oracle.topk(logits32.astype(np.float64), k, gate)
    counts, offsets, perm, inv = oracle.dispatch(idx, E, capacity)
    return dict(idx=idx.ravel(), w=w.ravel(), counts=counts, offsets=offsets, perm=perm, inv=inv)


def assert_routing_equal(gpu: dict, ref: dict):
    for key in ("idx", "counts", "offsets", "perm", "inv"):
        assert np.array_equal(gpu[key], ref[key]), key
    w_ref32 = ref["w"].astype(np.float32)
    ulp = np.spacing(np.abs(w_ref32)).astype(np.float64)
    assert np.all(np.abs(gpu["w"].astype(np.float64) - ref["w"]) <= 2 * ulp)


def f32_shape(E, k, H=8, F=8):
    return gen.LayerShape(f"route_E{E}k{k}", H=H, F=F, E=E, k=k, dtype="f32")


# ---------------------------------------------------------------- routing ---


@pytest.mark.parametrize("E,k,T", [(8, 2, 1), (8, 2, 64), (8, 2, 65), (3, 3, 100), (17, 4, 333),
                                   (64, 2, 1000), (128, 4, 2500), (200, 8, 129), (256, 8, 700),
                                   (1, 1, 40), (256, 1, 3),
                                   # 8192 pairs: the one-workgroup dispatch at its largest;
                                   # 8194: the three dispatch kernels
                                   (256, 8, 1024), (16, 2, 4097),
                                   # k > 8: selection by ranks (soft routing at k = E)
                                   (64, 64, 50), (128, 128, 20), (64, 12, 300), (200, 33, 40),
                                   (256, 256, 3)])
def test_route_given_logits_bit_exact(E, k, T):
    _log("route given logits", E, k, T)
    rng = np.random.default_rng(E * 1000 + T)
    lg = rng.normal(0, 1.5, (T, E)).astype(np.float32)
    # plant ties: integer-valued rows, all-equal rows, signed zeros
    lg[::5] = np.round(lg[::5])
    lg[1::7] = 0.0
    lg[2::11, ::2] = -0.0
    c = Case(f32_shape(E, k), T)
    gpu = c.layer.route(None, T, logits_in=torch.from_numpy(lg).cuda())
    torch.cuda.synchronize()
    gpu = {kk: v.cpu().numpy() for kk, v in gpu.items()}
    assert_routing_equal(gpu, routing_reference(lg, E, k))
    c.close()


@pytest.mark.parametrize("E,k,T", [(8, 2, 1), (8, 2, 300), (64, 2, 97), (256, 8, 40),
                                   (64, 16, 97), (128, 128, 9)])
def test_route_raw_gate_given_logits_bit_exact(E, k, T):
    """Raw gate: the same selection; the weights are the given fp32 logits."""
    rng = np.random.default_rng(7 * E + T)
    lg = rng.normal(0, 1.5, (T, E)).astype(np.float32)
    lg[::5] = np.round(lg[::5])
    c = Case(f32_shape(E, k), T, flags=moe.MOE_FLAG_GATE_RAW)
    gpu = c.layer.route(None, T, logits_in=torch.from_numpy(lg).cuda())
    torch.cuda.synchronize()
    gpu = {kk: v.cpu().numpy() for kk, v in gpu.items()}
    ref = routing_reference(lg, E, k, "raw")
    assert_routing_equal(gpu, ref)
    assert np.array_equal(gpu["w"], np.take_along_axis(lg, gpu["idx"].reshape(T, k).astype(np.int64), 1).ravel())
    c.close()


CONFIGS = [("tiny", gen.TINY, 32), ("qwen", gen.QWEN, 512), ("mixtral_prefill", gen.MIXTRAL, 4096),
           ("deepseek", gen.DEEPSEEK, 8192), ("mixtral_decode", gen.MIXTRAL, 1)]


@pytest.mark.parametrize("name,shape,T", CONFIGS)
def test_route_config_logits_bit_exact_and_end_to_end(name, shape, T):
    """Oracle logits rounded to fp32 once drive both sides: bit-exact routing.
    Then the GPU's own logits: indices differ only at near ties."""
    _log("route config", name, T)
    c = Case(shape, T)
    x = gen.gen_x(shape, T)
    lg64 = c.orc.logits(x)
    lg32 = lg64.astype(np.float32)
    gpu = c.layer.route(None, T, logits_in=torch.from_numpy(lg32).cuda())
    torch.cuda.synchronize()
    gpu = {kk: v.cpu().numpy() for kk, v in gpu.items()}
    assert_routing_equal(gpu, routing_reference(lg32, shape.E, shape.k))
    own = c.route(x)
    idx_o, _ = oracle.topk_softmax(lg64, shape.k)
    gap = near_tie_gap(lg64, shape.k)
    diff = np.any(own["idx"].reshape(T, shape.k) != idx_o, axis=1)
    _log(f"  near ties {(gap < 1e-3).sum()} / {T}, routed differently {diff.sum()}")
    assert np.all(gap[diff] < 1e-3)
    c.close()


# ------------------------------------------------------------- forward -----

SMALL = [
    # dtype, H, F, E, k, T, flags
    ("f32", 64, 128, 8, 2, 32, 0),
    ("f32", 36, 20, 5, 3, 77, 0),
    ("bf16", 512, 384, 4, 2, 700, moe.MOE_FLAG_PATH_GROUPED),
    ("bf16", 512, 384, 4, 2, 700, moe.MOE_FLAG_PATH_STREAM),
    ("bf16", 256, 256, 8, 2, 1, 0),
    ("bf16", 256, 256, 8, 2, 5, 0),
    ("bf16", 1024, 256, 8, 2, 64, moe.MOE_FLAG_PATH_STREAM),
    ("bf16", 1024, 256, 8, 2, 64, moe.MOE_FLAG_PATH_GROUPED),
    ("bf16", 256, 640, 16, 4, 300, moe.MOE_FLAG_PATH_STREAM),
    ("bf16", 256, 640, 16, 4, 300, moe.MOE_FLAG_PATH_GROUPED),
    ("bf16", 768, 256, 3, 1, 1100, 0),
    ("bf16", 256, 128, 64, 8, 97, 0),
    # batches beyond 64 tokens with 33-64 experts: the router staged from its
    # [H][E] layout in the partial-logit kernel (E = 45: element by element)
    ("bf16", 768, 128, 45, 3, 200, 0),
    ("bf16", 512, 256, 40, 2, 1500, 0),
    # the single-token route (T = 1, E = 8 or 16, H % 1024 == 0)
    ("bf16", 1024, 256, 16, 4, 1, 0),
    ("bf16", 4096, 128, 8, 2, 1, 0),
    ("bf16", 2048, 128, 8, 2, 1, moe.MOE_FLAG_GATE_RAW),
    ("bf16", 2048, 128, 8, 2, 4, moe.MOE_FLAG_GATE_RAW),
    # raw-logit gates: fp32 router, each bf16 router kernel, both expert paths
    ("f32", 64, 128, 8, 2, 32, moe.MOE_FLAG_GATE_RAW),
    ("bf16", 512, 256, 8, 2, 5, moe.MOE_FLAG_GATE_RAW),
    ("bf16", 512, 384, 4, 2, 700, moe.MOE_FLAG_GATE_RAW | moe.MOE_FLAG_PATH_GROUPED),
    ("bf16", 512, 384, 4, 2, 300, moe.MOE_FLAG_GATE_RAW | moe.MOE_FLAG_PATH_STREAM),
    ("bf16", 256, 128, 64, 8, 60, moe.MOE_FLAG_GATE_RAW),
    # soft routing: every expert weighted (top_k == num_experts)
    ("bf16", 512, 256, 8, 8, 50, moe.MOE_FLAG_PATH_STREAM),
    ("bf16", 512, 256, 8, 8, 300, moe.MOE_FLAG_PATH_GROUPED),
    ("f32", 64, 128, 6, 6, 32, 0),
    # soft routing over the 64- and 128-expert workloads' expert counts (k > 8:
    # selection by ranks; small batches route in separate launches)
    ("bf16", 256, 128, 64, 64, 20, 0),
    ("bf16", 256, 128, 64, 64, 100, 0),
    ("bf16", 256, 128, 128, 128, 8, 0),
    ("bf16", 256, 128, 128, 128, 40, moe.MOE_FLAG_PATH_GROUPED),
    ("bf16", 512, 256, 32, 12, 70, 0),
    ("bf16", 256, 128, 64, 16, 33, moe.MOE_FLAG_GATE_RAW),
    ("f32", 64, 128, 16, 16, 32, 0),
    # streaming down projection with 1 KB row runs and 9-16 token rows per
    # pass (F % 512 == 0), with the combine folded in and kept apart
    ("bf16", 512, 1024, 8, 2, 16, 0),
    ("bf16", 512, 1024, 8, 2, 16, moe.MOE_FLAG_COMBINE_SEPARATE),
    ("bf16", 512, 1024, 8, 2, 12, 0),
    # one expert, top-1: the layer is a dense SwiGLU FFN (both expert paths)
    ("bf16", 512, 256, 1, 1, 20, 0),
    ("bf16", 512, 256, 1, 1, 300, 0),
    ("f32", 64, 128, 1, 1, 32, 0),
    # grouped down projection whose last tiles are split along K
    ("bf16", 256, 2048, 8, 2, 600, moe.MOE_FLAG_PATH_GROUPED),
    # the separate combine at k = 3, 5 and 7 (its loads unrolled per k)
    ("bf16", 256, 128, 8, 3, 200, moe.MOE_FLAG_PATH_GROUPED),
    ("bf16", 256, 128, 16, 5, 150, 0),
    ("bf16", 256, 128, 8, 7, 40, moe.MOE_FLAG_PATH_STREAM),
]


@pytest.mark.parametrize("dtype,H,F,E,k,T,flags", SMALL)
def test_forward_small_shapes(dtype, H, F, E, k, T, flags):
    _log("forward small", dtype, H, F, E, k, T, flags)
    shape = gen.LayerShape(f"s{H}_{F}_{E}_{k}", H=H, F=F, E=E, k=k, dtype=dtype)
    c = Case(shape, T, flags=flags)
    x = gen.gen_x(shape, T)
    y = c.forward(x)
    r = c.route(x)
    st = check_rows(c, x, np.arange(T), y, r["idx"])
    _log("  ", st)
    y2 = c.forward(x)
    assert np.array_equal(y, y2)  # bitwise reproducible
    c.close()


def test_forward_smaller_calls_reuse_layer():
    shape = gen.LayerShape("reuse", H=256, F=256, E=8, k=2, dtype="bf16")
    c = Case(shape, 500)
    for T in (500, 1, 37, 256, 499):
        x = gen.gen_x(shape, T, seed=T)
        y = c.forward(x)
        check_rows(c, x, np.arange(T), y, c.route(x)["idx"])
    c.close()


def test_grouped_and_stream_paths_agree():
    shape = gen.LayerShape("paths", H=512, F=256, E=8, k=2, dtype="bf16")
    x = gen.gen_x(shape, 200)
    ys = []
    for fl in (moe.MOE_FLAG_PATH_GROUPED, moe.MOE_FLAG_PATH_STREAM):
        c = Case(shape, 200, flags=fl)
        ys.append(c.forward(x))
        c.close()
    rms = np.sqrt(np.mean(ys[0].astype(np.float64) ** 2))
    assert np.abs(ys[0] - ys[1]).max() <= 2e-2 * rms


FULL = [("tiny", gen.TINY, 32, 0), ("mixtral_decode", gen.MIXTRAL, 1, 0),
        ("qwen", gen.QWEN, 512, 0), ("mixtral_prefill", gen.MIXTRAL, 4096, 512),
        ("deepseek", gen.DEEPSEEK, 8192, 2048)]


@pytest.mark.parametrize("name,shape,T,chunk", FULL)
def test_forward_config(name, shape, T, chunk):
    """The layer at the workloads' full sizes: every output row against the
    oracle (near-tie rule applied), with one RMS over the whole output."""
    _log("forward config", name, T)
    c = Case(shape, T)
    x = gen.gen_x(shape, T)
    y = c.forward(x)
    r = c.route(x)
    st = check_rows(c, x, np.arange(T), y, r["idx"], chunk=chunk, log=_log)
    _log("  ", st)
    assert np.array_equal(y, c.forward(x))  # bitwise reproducible
    c.close()


@pytest.mark.parametrize("H,F,E,k", [(512, 512, 8, 2), (256, 256, 128, 8)])
def test_forward_at_max_tokens(H, F, E, k):
    """T = 65536, the largest batch a layer takes: the grouped GEMMs over many
    rounds of tiles and the histogram / scan / scatter dispatch of T*k pairs
    (131072 and 524288); sampled rows (both ends and random ones) against the
    oracle, the whole output bitwise reproducible."""
    T = 65536
    _log("max tokens", H, F, E, k, T)
    shape = gen.LayerShape(f"max{H}_{F}_{E}_{k}", H=H, F=F, E=E, k=k, dtype="bf16")
    c = Case(shape, T)
    x = gen.gen_x(shape, T)
    y = c.forward(x)
    r = c.route(x)
    idx = r["idx"].reshape(T, k)
    rng = np.random.default_rng(7)
    toks = np.unique(np.concatenate([[0, 1, T - 2, T - 1], rng.choice(T, 60, False)]))
    st = check_rows(c, x, toks, y[toks], idx[toks])
    _log("  ", st)
    assert np.array_equal(y, c.forward(x))
    c.close()


@pytest.mark.parametrize("flags", [0, moe.MOE_FLAG_COMBINE_SEPARATE])
@pytest.mark.parametrize("T", [4, 16, 64])
def test_mixtral_decode_every_row(T, flags):
    """The Mixtral-shaped bf16 layer at decode batches: the weight-streaming
    kernels (1 KB row runs; 8, 16 and 32 token rows per pass; the down
    projection with the combine folded in and kept apart), every row against
    the oracle."""
    _log("mixtral decode", T, flags)
    c = Case(gen.MIXTRAL, 64, flags=flags)
    x = gen.gen_x(gen.MIXTRAL, T)
    y = c.forward(x)
    r = c.route(x)
    st = check_rows(c, x, np.arange(T), y, r["idx"])
    _log("  ", st)
    c.close()


def grouped_down_plan(counts, H, F, E, S, cus):
    """Host replica of the grouped down projection's persistent schedule for a
    layer that holds the tail-split workspace (then the K range stays whole: one
    plane): (K split, pieces per XCD share), pieces > 1 where the tail split
    runs."""
    nw = max(cus // 8, 1)
    ksplit = 1
    ntt = int(sum(-(-int(c) // 256) for c in counts))
    ntiles = ksplit * ntt * (H // 256)
    nk_slice = F // ksplit // 32
    pieces = []
    for xcd in range(8):
        q0, q1 = (xcd * ntiles) >> 3, ((xcd + 1) * ntiles) >> 3
        nleft = (q1 - q0) % nw
        pieces.append(max(1, min(nw // nleft, 4, nk_slice // 16)) if nleft else 1)
    return ksplit, pieces


def grouped_gate_up_pieces(counts, F, cus):
    """Host replica of the grouped gate/up schedule's last round: per XCD
    share, the number of token-row pieces each leftover tile is cut into."""
    nw = max(cus // 8, 1)
    ntiles = int(sum(-(-int(c) // 256) for c in counts)) * (F // 128)
    pieces = []
    for xcd in range(8):
        q0, q1 = (xcd * ntiles) >> 3, ((xcd + 1) * ntiles) >> 3
        nleft = (q1 - q0) % nw
        pieces.append(min(nw // nleft, 4) if nleft else 1)
    return pieces


def test_grouped_down_tail_split_every_row():
    """A grouped layer whose down projection runs the tail split (tiles of the
    last, partial round cut along K, finished by the fix-up launch) and whose
    gate/up cuts its last round's tiles into token-row pieces: both plans are
    replayed on the host to show the splits happen, then every row is
    compared with the oracle."""
    shape = gen.LayerShape("tail", H=256, F=2048, E=8, k=2, dtype="bf16")
    T = 600
    c = Case(shape, T, flags=moe.MOE_FLAG_PATH_GROUPED)
    x = gen.gen_x(shape, T)
    r = c.route(x)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ksplit, pieces = grouped_down_plan(r["counts"], shape.H, shape.F, shape.E, T * shape.k, cus)
    gu_pieces = grouped_gate_up_pieces(r["counts"], shape.F, cus)
    _log(f"  CUs {cus}, K split {ksplit}, pieces per XCD share {pieces}, "
         f"gate/up token pieces {gu_pieces}")
    assert max(pieces) >= 2
    assert max(gu_pieces) >= 2
    y = c.forward(x)
    st = check_rows(c, x, np.arange(T), y, r["idx"])
    _log("  ", st)
    assert np.array_equal(y, c.forward(x))
    c.close()


def test_residual_stack_teacher_forced():
    """Three stacked layers, y aliasing x: each layer checked against the
    oracle fed with the GPU's residual stream at that layer."""
    shape = gen.LayerShape("stack", H=512, F=256, E=8, k=2, dtype="bf16")
    T = 24
    cases = [Case(shape, T, flags=moe.MOE_FLAG_RESIDUAL_PRENORM, layer=l) for l in range(3)]
    h = torch.from_numpy(gen.normal(0, 0, gen.T_X, T * shape.H, 1.0, "f32").reshape(T, shape.H)).cuda()
    for c in cases:
        h_in = h.cpu().numpy()
        c.layer.forward(h, h)  # in place
        torch.cuda.synchronize()
        h_out = h.cpu().numpy()
        xt = oracle.prenorm_bf16(h_in)
        hin_d = torch.from_numpy(h_in).cuda()  # the GPU's routing of this layer's input
        r = c.layer.route(hin_d, T)
        torch.cuda.synchronize()
        branch = (h_out.astype(np.float64) - h_in.astype(np.float64))
        check_rows(c, xt, np.arange(T), branch, r["idx"].cpu().numpy())
    for c in cases:
        c.close()


def test_call_validation_on_device():
    shape = gen.LayerShape("val", H=256, F=256, E=8, k=2, dtype="bf16")
    c = Case(shape, 16)
    x = to_dev(gen.gen_x(shape, 16))
    y = torch.empty((16, 256), dtype=torch.float32, device="cuda")
    lib = moe.lib()
    h = c.layer.handle
    s = torch.cuda.current_stream().cuda_stream
    assert lib.moe_forward(h, x.data_ptr(), 0, y.data_ptr(), s) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_forward(h, x.data_ptr(), 17, y.data_ptr(), s) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_forward(h, x.data_ptr() + 2, 4, y.data_ptr(), s) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_forward(h, x.data_ptr(), 4, x.data_ptr(), s) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_forward(h, x.data_ptr(), 16, y.data_ptr(), s) == moe.MOE_OK
    torch.cuda.synchronize()
    c.close()


@pytest.mark.parametrize("name,shape,T", [("deepseek", gen.DEEPSEEK, 8192),
                                          ("mixtral_prefill", gen.MIXTRAL, 4096)])
def test_grouped_path_matches_stream_path_on_every_row(name, shape, T):
    """A property that holds at any size: the grouped-GEMM path and the
    weight-streaming path compute the same layer, so every output row must
    agree (and each path must repeat itself bit for bit).  The streaming path
    has no LDS staging, so this covers every tile of the grouped GEMMs,
    which the oracle can only sample."""
    _log("grouped vs stream", name, T)
    x = to_dev(gen.gen_x(shape, T))
    outs = {}
    for fl in (moe.MOE_FLAG_PATH_GROUPED, moe.MOE_FLAG_PATH_STREAM):
        c = Case(shape, T, flags=fl)
        ys = []
        for _ in range(3):
            y = torch.empty((T, shape.H), dtype=torch.float32, device="cuda")
            c.layer.forward(x, y)
            torch.cuda.synchronize()
            ys.append(y.cpu().numpy())
        assert all(np.array_equal(ys[0], yy) for yy in ys[1:]), "not reproducible"
        outs[fl] = ys[0].astype(np.float64)
        c.close()
    g, s = outs[moe.MOE_FLAG_PATH_GROUPED], outs[moe.MOE_FLAG_PATH_STREAM]
    rms = np.sqrt(np.mean(s ** 2))
    row_err = np.abs(g - s).max(axis=1)
    _log(f"  max |grouped - stream| / rms = {row_err.max() / rms:.3e}")
    assert np.all(row_err <= 1e-2 * rms), np.nonzero(row_err > 1e-2 * rms)[0][:20]


# ------------------------------------------------------- expert capacity ---


@pytest.mark.parametrize("E,k,T,cap", [(8, 2, 300, 40), (8, 2, 1000, 100), (64, 2, 777, 10),
                                       (3, 3, 100, 1), (128, 4, 2500, 60), (8, 2, 20, 100),
                                       (256, 8, 1024, 20), (16, 2, 4097, 300)])
def test_route_capacity_given_logits_bit_exact(E, k, T, cap):
    """Capacity on the dispatch kernels (one workgroup up to 8192 pairs, the
    multi-run kernels beyond): counts capped, the first
    pairs of each expert in slot order kept, dropped pairs inv = -1, perm -1
    beyond the kept pairs; bit-exact against the oracle."""
    _log("route capacity", E, k, T, cap)
    rng = np.random.default_rng(11 * E + T)
    lg = rng.normal(0, 1.5, (T, E)).astype(np.float32)
    lg[:, 0] += 1.0  # skew: expert 0 over-subscribed
    c = Case(f32_shape(E, k), T, capacity=cap)
    gpu = c.layer.route(None, T, logits_in=torch.from_numpy(lg).cuda())
    torch.cuda.synchronize()
    gpu = {kk: v.cpu().numpy() for kk, v in gpu.items()}
    ref = routing_reference(lg, E, k, capacity=cap)
    assert_routing_equal(gpu, ref)
    assert (gpu["counts"] <= cap).all()
    c.close()


CAP_CASES = [
    # dtype, H, F, E, k, T, capacity, flags  (router + dispatch kernel, expert path)
    ("bf16", 512, 256, 8, 2, 40, 6, 0),                              # one-workgroup routing, stream
    ("bf16", 256, 128, 64, 8, 60, 3, 0),                             # split-H small routing, stream
    ("bf16", 512, 384, 4, 2, 700, 200, moe.MOE_FLAG_PATH_GROUPED),   # dispatch kernels, grouped
    ("bf16", 512, 384, 4, 2, 700, 200, moe.MOE_FLAG_PATH_STREAM),    # dispatch kernels, stream
    ("bf16", 1024, 256, 8, 2, 4, 1, 0),                              # one-workgroup route, T = 4
    ("f32", 64, 128, 8, 2, 32, 4, 0),
    ("bf16", 256, 128, 16, 5, 150, 30, 0),                           # dropped pairs, k = 5
]


@pytest.mark.parametrize("dtype,H,F,E,k,T,cap,flags", CAP_CASES)
def test_forward_with_capacity(dtype, H, F, E, k, T, cap, flags):
    _log("forward capacity", dtype, H, F, E, k, T, cap, flags)
    shape = gen.LayerShape(f"c{H}_{F}_{E}_{k}", H=H, F=F, E=E, k=k, dtype=dtype)
    c = Case(shape, T, flags=flags, capacity=cap)
    x = gen.gen_x(shape, T)
    y = c.forward(x)
    r = c.route(x)
    counts, offsets, perm, inv = oracle.dispatch(r["idx"].reshape(T, k), E, cap)
    for key, ref in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        assert np.array_equal(r[key], ref), key  # the dispatch of the GPU's own routing
    keep = (inv >= 0).reshape(T, k)
    assert not keep.all()  # the capacity bites
    st = check_rows(c, x, np.arange(T), y, r["idx"], keep_rows=keep)
    _log("  ", st)
    assert np.array_equal(y, c.forward(x))
    c.close()


def test_deepseek_skewed_with_capacity():
    """The Zipf-skewed 128-expert workload with capacity 1.25 T k / E: the hot
    experts are cut to the capacity, every other expert keeps all its rows."""
    shape, T = gen.DEEPSEEK, 8192
    cap = int(1.25 * T * shape.k / shape.E)
    _log("deepseek capacity", cap)
    c = Case(shape, T, capacity=cap)
    x = gen.gen_x(shape, T)
    y = c.forward(x)
    r = c.route(x)
    idx = r["idx"].reshape(T, shape.k)
    counts, offsets, perm, inv = oracle.dispatch(idx, shape.E, cap)
    for key, ref in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        assert np.array_equal(r[key], ref), key
    raw = np.bincount(idx.ravel(), minlength=shape.E)
    assert (raw > cap).sum() >= 5 and (counts == np.minimum(raw, cap)).all()
    keep = (inv >= 0).reshape(T, shape.k)
    rng = np.random.default_rng(9)
    toks = np.unique(np.concatenate([[0, 1, T // 2, T - 1], rng.choice(T, 28, False)]))
    st = check_rows(c, x, toks, y[toks], idx[toks], keep_rows=keep[toks])
    _log("  ", st)
    c.close()
