"""ctypes binding of the fp64 CPU oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg.  The GPU library never imports, links or calls
anything here, and nothing here calls the GPU library.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

F32, BF16 = 0, 1
GATE_SOFTMAX, GATE_RAW = 0, 1
EXPERT_DTYPE, EXPERT_U8 = 0, 1
U8_PARAMS_BYTES = 64


class U8Params(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float * 3), ("zero", ctypes.c_int32 * 3),
                ("min", ctypes.c_float * 3), ("max", ctypes.c_float * 3),
                ("pad", ctypes.c_uint32 * 4)]


class _Layer(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("F", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("experts", ctypes.c_void_p), ("stride", ctypes.c_uint64),
                ("gate", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("expert_format", ctypes.c_int32)]


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.orc_logits.argtypes = [vp, vp, i32, vp]
        L.orc_topk_softmax.argtypes = [i32, i32, i32, vp, vp, vp]
        L.orc_topk.argtypes = [i32, i32, i32, i32, vp, vp, vp]
        L.orc_dispatch.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
        L.orc_dispatch_cap.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.orc_expert_ffn.argtypes = [vp, i32, vp, vp]
        L.orc_expert_rows.argtypes = [vp, vp, i32, vp, vp, vp]
        L.orc_combine.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.orc_layer_forward.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, vp, vp]
        L.orc_layer_tokens.argtypes = [vp, vp, i32, vp, i32, vp, vp, vp, vp, vp, vp]
        L.orc_prenorm_bf16.argtypes = [i32, i32, vp, vp]
        L.orc_quantize_u8.argtypes = [vp, ctypes.c_size_t, vp, vp, i32]
        L.orc_quantize_experts_u8.argtypes = [vp, ctypes.c_uint64, i32, i32, i32, vp,
                                              ctypes.c_uint64]
        L.orc_bf16_round.argtypes = [ctypes.c_double]
        L.orc_bf16_round.restype = ctypes.c_double
        L.orc_num_threads.argtypes = []
        L.orc_set_num_threads.argtypes = [i32]
        L.orc_set_num_threads.restype = None
        _LIB = L
    return _LIB


def _p(a):
    return None if a is None else a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


class Layer:
    """One MoE layer's weights as the oracle reads them (numpy arrays kept alive)."""

    def __init__(self, H, F, E, k, dtype, router_w, router_b, experts, stride, gate="softmax",
                 capacity=0, expert_format="dtype"):
        self.H, self.F, self.E, self.k = H, F, E, k
        self.gate = gate
        self.capacity = capacity
        self.dtype = dtype
        self.np_dtype = np.float32 if dtype == "f32" else np.uint16
        self.router_w = np.ascontiguousarray(router_w, dtype=self.np_dtype)
        self.router_b = None if router_b is None else np.ascontiguousarray(router_b, np.float32)
        self.experts = np.ascontiguousarray(experts)
        self.stride = stride
        self._s = _Layer(H, F, E, k, F32 if dtype == "f32" else BF16, _p(self.router_w),
                         _p(self.router_b), _p(self.experts), stride,
                         {"softmax": GATE_SOFTMAX, "raw": GATE_RAW}[gate], capacity,
                         {"dtype": EXPERT_DTYPE, "u8": EXPERT_U8}[expert_format])

    @property
    def ref(self):
        return ctypes.byref(self._s)

    def _x(self, x):
        x = np.ascontiguousarray(x, dtype=self.np_dtype)
        assert x.ndim == 2 and x.shape[1] == self.H
        return x

    def logits(self, x):
        x = self._x(x)
        out = np.empty((x.shape[0], self.E), np.float64)
        _check(lib().orc_logits(self.ref, _p(x), x.shape[0], _p(out)), "logits")
        return out

    def expert_ffn(self, e, xrow):
        xrow = np.ascontiguousarray(xrow, np.float64)
        out = np.empty(self.H, np.float64)
        _check(lib().orc_expert_ffn(self.ref, e, _p(xrow), _p(out)), "expert_ffn")
        return out

    def forward(self, x):
        """Full O1..O6: returns dict y, idx, w, counts, offsets, perm, inv."""
        x = self._x(x)
        T, k, E = x.shape[0], self.k, self.E
        r = dict(y=np.empty((T, self.H), np.float64), idx=np.empty((T, k), np.int32),
                 w=np.empty((T, k), np.float64), counts=np.empty(E, np.int32),
                 offsets=np.empty(E + 1, np.int32), perm=np.empty(T * k, np.int32),
                 inv=np.empty(T * k, np.int32))
        _check(lib().orc_layer_forward(self.ref, _p(x), T, _p(r["y"]), _p(r["idx"]),
                                       _p(r["w"]), _p(r["counts"]), _p(r["offsets"]),
                                       _p(r["perm"]), _p(r["inv"])), "layer_forward")
        return r

    def tokens(self, x, tokens, idx_override=None, keep=None):
        """Output rows of the listed tokens only: dict y, idx, w, logits.
        keep [n, k] (optional): slots that count (a capacity's drops)."""
        x = self._x(x)
        tokens = np.ascontiguousarray(tokens, np.int32)
        n, k = tokens.size, self.k
        ov = None if idx_override is None else np.ascontiguousarray(idx_override, np.int32)
        if ov is not None:
            assert ov.shape == (n, k)
        kp = None if keep is None else np.ascontiguousarray(keep, np.int32)
        if kp is not None:
            assert kp.shape == (n, k)
        r = dict(y=np.empty((n, self.H), np.float64), idx=np.empty((n, k), np.int32),
                 w=np.empty((n, k), np.float64), logits=np.empty((n, self.E), np.float64))
        _check(lib().orc_layer_tokens(self.ref, _p(x), x.shape[0], _p(tokens), n, _p(ov), _p(kp),
                                      _p(r["y"]), _p(r["idx"]), _p(r["w"]), _p(r["logits"])),
               "layer_tokens")
        return r


def topk_softmax(logits, k):
    logits = np.ascontiguousarray(logits, np.float64)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _check(lib().orc_topk_softmax(T, E, k, _p(logits), _p(idx), _p(w)), "topk_softmax")
    return idx, w


def topk(logits, k, gate="softmax"):
    """Selection (value desc, index asc) with the softmax or the raw gate."""
    logits = np.ascontiguousarray(logits, np.float64)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    g = {"softmax": GATE_SOFTMAX, "raw": GATE_RAW}[gate]
    _check(lib().orc_topk(T, E, k, g, _p(logits), _p(idx), _p(w)), "topk")
    return idx, w


def dispatch(idx, E, capacity=0):
    idx = np.ascontiguousarray(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    _check(lib().orc_dispatch_cap(T, E, k, capacity, _p(idx), _p(counts), _p(offsets), _p(perm),
                                  _p(inv)), "dispatch")
    return counts, offsets, perm, inv


def combine(w, inv, yp):
    w = np.ascontiguousarray(w, np.float64)
    inv = np.ascontiguousarray(inv, np.int32)
    yp = np.ascontiguousarray(yp, np.float64)
    T, k = w.shape
    H = yp.shape[1]
    y = np.empty((T, H), np.float64)
    _check(lib().orc_combine(T, H, k, _p(w), _p(inv), _p(yp), _p(y)), "combine")
    return y


def prenorm_bf16(h):
    h = np.ascontiguousarray(h, np.float32)
    T, H = h.shape
    out = np.empty((T, H), np.uint16)
    _check(lib().orc_prenorm_bf16(T, H, _p(h), _p(out)), "prenorm_bf16")
    return out


def bf16_round(v: float) -> float:
    return lib().orc_bf16_round(v)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the oracle's later parallel loops (timing only)."""
    lib().orc_set_num_threads(n)


def layer_from_gen(shape, router_w, router_b, experts, gate="softmax", capacity=0,
                   u8_experts=None, u8_stride=0) -> Layer:
    """The layer of a generated workload; with u8_experts (uint8 experts and
    their parameter blocks, stride u8_stride) the expert weights are those."""
    if u8_experts is not None:
        return Layer(shape.H, shape.F, shape.E, shape.k, shape.dtype, router_w, router_b,
                     u8_experts, u8_stride, gate=gate, capacity=capacity, expert_format="u8")
    return Layer(shape.H, shape.F, shape.E, shape.k, shape.dtype, router_w, router_b, experts,
                 shape.stride, gate=gate, capacity=capacity)


def quantize_u8(w_bf16):
    """One matrix of bf16 bit patterns -> (uint8 codes, scale, zero, min, max)."""
    w = np.ascontiguousarray(w_bf16, np.uint16)
    q = np.empty(w.shape, np.uint8)
    p = U8Params()
    _check(lib().orc_quantize_u8(_p(w), w.size, _p(q), ctypes.byref(p), 0), "quantize_u8")
    return q, p.scale[0], p.zero[0], p.min[0], p.max[0]


def u8_stride(H, F):
    """Bytes per uint8 expert: three matrices and the parameter block, to 256."""
    return (3 * H * F + U8_PARAMS_BYTES + 255) // 256 * 256


def quantize_experts_u8(experts, src_stride, E, H, F, dst_stride=None):
    """bf16 experts (bytes or uint16 array, E * src_stride bytes) -> uint8
    experts with parameter blocks (uint8 array of E * dst_stride bytes)."""
    src = np.ascontiguousarray(experts).view(np.uint8)
    dst_stride = u8_stride(H, F) if dst_stride is None else dst_stride
    dst = np.zeros(E * dst_stride, np.uint8)
    _check(lib().orc_quantize_experts_u8(_p(src), src_stride, E, H, F, _p(dst), dst_stride),
           "quantize_experts_u8")
    return dst


def u8_params(u8_experts, stride, e, H, F) -> U8Params:
    off = e * stride + 3 * H * F
    return U8Params.from_buffer_copy(np.ascontiguousarray(u8_experts[off:off + U8_PARAMS_BYTES]))
