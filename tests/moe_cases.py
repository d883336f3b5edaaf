"""Helpers shared by the GPU parity tests: build a device layer and its oracle
twin from the same seeded host inputs, and compare outputs under the rules
below.

Comparison rules
  * floating-point outputs: max |y_gpu - y_ref| <= tol * RMS(y_ref), with
    tol = 1e-5 for fp32 layers and 1e-2 for bf16 layers;
  * routing: a token whose k-th and (k+1)-th largest oracle logits differ by
    less than 1e-3 is a near tie.  If the GPU picked a different expert set
    (or order) for it, the GPU's set must still be a top-k set under a
    perturbation of at most 1e-3, and that token's reference output is the
    oracle's output recomputed with the GPU's experts.  Any other routing
    difference fails.
"""
from __future__ import annotations

import functools

import numpy as np
import torch

import gen
import mixture_experts_amd as moe
import oracle

NEAR_TIE = 1e-3
TOL = {"f32": 1e-5, "bf16": 1e-2}


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@functools.lru_cache(maxsize=4)
def host_inputs(shape: gen.LayerShape, layer: int = 0):
    """(router_w, bias, experts) of a layer, generated once per process."""
    return gen.gen_router(shape, layer), gen.gen_bias(shape), gen.gen_experts(shape, layer)


class Case:
    """A device layer and the oracle over the very same host arrays."""

    def __init__(self, shape: gen.LayerShape, max_tokens: int, flags: int = 0, layer: int = 0,
                 router=None, bias="default", experts=None, capacity: int = 0):
        wr, b, ex = host_inputs(shape, layer) if router is None or experts is None else (
            None, None, None)
        self.router = wr if router is None else router
        self.bias = b if isinstance(bias, str) else bias
        self.experts = ex if experts is None else experts
        self.shape = shape
        dt = moe.MOE_F32 if shape.dtype == "f32" else moe.MOE_BF16
        self.d_router = to_dev(self.router)
        self.d_bias = None if self.bias is None else to_dev(self.bias)
        self.d_experts = to_dev(self.experts)
        self.capacity = capacity
        self.layer = moe.MoELayer(shape.H, shape.F, shape.E, shape.k, max_tokens, dt,
                                  self.d_router, self.d_experts, shape.stride, self.d_bias, flags,
                                  expert_capacity=capacity)
        gate = "raw" if flags & moe.MOE_FLAG_GATE_RAW else "softmax"
        self.orc = oracle.layer_from_gen(shape, self.router, self.bias, self.experts, gate=gate,
                                         capacity=capacity)

    def forward(self, x_np: np.ndarray) -> np.ndarray:
        x = to_dev(x_np)
        y = torch.empty((x_np.shape[0], self.shape.H), dtype=torch.float32, device="cuda")
        self.layer.forward(x, y)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    def route(self, x_np: np.ndarray) -> dict:
        r = self.layer.route(to_dev(x_np), x_np.shape[0])
        torch.cuda.synchronize()
        return {k: v.cpu().numpy() for k, v in r.items()}

    def close(self):
        self.layer.close()


def near_tie_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """k-th minus (k+1)-th largest logit per row (inf when k == E)."""
    if k >= logits.shape[1]:
        return np.full(logits.shape[0], np.inf)
    s = -np.sort(-logits, axis=1)
    return s[:, k - 1] - s[:, k]


def reference_rows(case: Case, x_np: np.ndarray, tokens, gpu_idx_rows: np.ndarray,
                   keep_rows: np.ndarray | None = None, chunk: int = 0, log=None):
    """The oracle's output rows of `tokens` under the near-tie rule, and
    routing statistics.  Returns (y_ref [n, H] float64, stats).

    keep_rows [len(tokens), k]: with an expert capacity, the slots that are
    kept under the GPU's routing of all tokens (which tokens an expert drops
    depends on the others); the reference then uses the GPU's experts for
    every row, after the near-tie check has validated them.
    chunk > 0: the oracle is called on that many tokens at a time (log, if
    given, is called after each chunk), so large workloads report progress."""
    k = case.shape.k
    tokens = np.asarray(tokens, np.int32)
    gpu_idx_rows = np.asarray(gpu_idx_rows).reshape(len(tokens), k)
    n = len(tokens)
    step = n if chunk <= 0 else chunk
    y_ref = np.empty((n, case.shape.H), np.float64)
    stats = dict(tokens=n, near_ties=0, routed_differently=0)
    for c0 in range(0, n, max(step, 1)):
        sl = slice(c0, min(n, c0 + step))
        tk, gi = tokens[sl], gpu_idx_rows[sl]
        kp = None if keep_rows is None else np.asarray(keep_rows, np.int32).reshape(n, k)[sl]
        ref = case.orc.tokens(x_np, tk)
        gap = near_tie_gap(ref["logits"], k)
        differs = np.any(gi != ref["idx"], axis=1)
        stats["near_ties"] += int((gap < NEAR_TIE).sum())
        stats["routed_differently"] += int(differs.sum())
        yr = ref["y"]
        if differs.any():
            kth = -np.sort(-ref["logits"], axis=1)[:, k - 1]
            for i in np.nonzero(differs)[0]:
                chosen = ref["logits"][i, gi[i]]
                # allowed only for near ties, and only as a valid top-k under a
                # perturbation of at most NEAR_TIE (slot order: adjacent slots
                # may swap only when their logits are that close)
                assert len(set(gi[i].tolist())) == k, (tk[i], gi[i])
                assert np.all(chosen >= kth[i] - NEAR_TIE), (tk[i], gi[i], ref["idx"][i])
                assert np.all(np.diff(chosen) <= NEAR_TIE), (tk[i], chosen)
            fix = np.nonzero(differs)[0]
            yr[fix] = case.orc.tokens(x_np, tk[fix], idx_override=gi[fix])["y"]
        if kp is not None:
            yr = case.orc.tokens(x_np, tk, idx_override=gi, keep=kp)["y"]
            stats["dropped_slots"] = stats.get("dropped_slots", 0) + int((kp == 0).sum())
        y_ref[sl] = yr
        if log is not None:
            log(f"    oracle rows {sl.stop} / {n}")
    return y_ref, stats


def compare_rows(case: Case, y_gpu_rows: np.ndarray, y_ref: np.ndarray, stats: dict,
                 tol: float | None = None) -> dict:
    """max |y_gpu - y_ref| <= tol * RMS(y_ref), the RMS over all compared rows."""
    tol = TOL[case.shape.dtype] if tol is None else tol
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    err = float(np.abs(y_gpu_rows.astype(np.float64) - y_ref).max()) if y_ref.size else 0.0
    stats = dict(stats, rms=rms, max_err=err, rel=err / rms if rms > 0 else err)
    assert np.isfinite(y_gpu_rows).all()
    assert err <= tol * rms, stats
    return stats


def check_rows(case: Case, x_np: np.ndarray, tokens, y_gpu_rows: np.ndarray,
               gpu_idx_rows: np.ndarray, tol: float | None = None,
               keep_rows: np.ndarray | None = None, chunk: int = 0, log=None) -> dict:
    """Compare GPU output rows of `tokens` with the oracle, near-tie rule applied
    (see reference_rows and compare_rows)."""
    y_ref, stats = reference_rows(case, x_np, tokens, gpu_idx_rows, keep_rows, chunk, log)
    return compare_rows(case, y_gpu_rows, y_ref, stats, tol)


def quantize_on_gpu(shape, d_src, E=None):
    E = shape.E if E is None else E
    st = moe.u8_stride(shape.H, shape.F)
    dst = torch.zeros(E * st, dtype=torch.uint8, device="cuda")  # padding bytes defined
    moe.moe_quantize_experts_u8(d_src, shape.stride, E, shape.H, shape.F, dst, st)
    torch.cuda.synchronize()
    return dst, st


class U8Case:
    """A uint8-expert layer on the GPU and the oracle's layer on the same codes."""

    def __init__(self, shape, max_tokens, flags=0, layer=0):
        self.shape = shape
        self.router, self.bias = gen.gen_router(shape, layer), gen.gen_bias(shape)
        d_src = torch.empty(shape.E * shape.stride, dtype=torch.uint8, device="cuda")
        gen.experts_device(shape, d_src.data_ptr(), layer=layer,
                           stream=torch.cuda.current_stream().cuda_stream)
        self.d_u8, self.st = quantize_on_gpu(shape, d_src)
        del d_src
        self.u8 = self.d_u8.cpu().numpy()
        self.d_router = to_dev(self.router)
        self.d_bias = None if self.bias is None else to_dev(self.bias)
        self.layer = moe.MoELayer(shape.H, shape.F, shape.E, shape.k, max_tokens, moe.MOE_BF16,
                                  self.d_router, self.d_u8, self.st, self.d_bias, flags,
                                  expert_format=moe.MOE_EXPERT_U8)
        gate = "raw" if flags & moe.MOE_FLAG_GATE_RAW else "softmax"
        self.orc = oracle.layer_from_gen(shape, self.router, self.bias, None, gate=gate,
                                         u8_experts=self.u8, u8_stride=self.st)

    def forward(self, x):
        y = torch.empty((x.shape[0], self.shape.H), dtype=torch.float32, device="cuda")
        self.layer.forward(to_dev(x), y)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    def route(self, x):
        r = self.layer.route(to_dev(x), x.shape[0])
        torch.cuda.synchronize()
        return {k: v.cpu().numpy() for k, v in r.items()}

    def close(self):
        self.layer.close()
