"""Python binding of libmoe (include/moe.h): argument marshalling only.

Every step of the layer runs in the HIP kernels of ``libmoe.so``; this module
converts torch tensors (or raw integers) to device pointers and checks return
codes.  It raises if the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_NO_MEMORY = -2
MOE_ERR_DEVICE = -3
MOE_ERR_UNSUPPORTED = -4
MOE_F32 = 0
MOE_BF16 = 1
MOE_FLAG_RESIDUAL_PRENORM = 1 << 0
MOE_FLAG_PATH_GROUPED = 1 << 1
MOE_FLAG_PATH_STREAM = 1 << 2
MOE_FLAG_GATE_RAW = 1 << 3
MOE_FLAG_COMBINE_SEPARATE = 1 << 4
MOE_EXPERT_DTYPE = 0
MOE_EXPERT_U8 = 1
U8_PARAMS_BYTES = 64

MOE_STAGE_ROUTE, MOE_STAGE_DISPATCH, MOE_STAGE_GATE_UP, MOE_STAGE_DOWN, MOE_STAGE_COMBINE = range(5)
MOE_NUM_STAGES = 5
STAGE_NAMES = ("route", "dispatch", "gate_up", "down", "combine")

EXPORTED = ("moe_layer_create", "moe_route", "moe_forward", "moe_forward_ev", "moe_layer_free",
            "moe_quantize_experts_u8", "moe_forward_noalloc")
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

_ERRS = {MOE_ERR_INVALID_ARG: "invalid argument", MOE_ERR_NO_MEMORY: "out of device memory",
         MOE_ERR_DEVICE: "device error", MOE_ERR_UNSUPPORTED: "unsupported shape or mode"}


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {_ERRS.get(code, 'error')} ({code})")
        self.code = code


class moe_layer_desc(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("hidden", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("expert_base", ctypes.c_void_p), ("expert_stride", ctypes.c_uint64),
                ("expert_capacity", ctypes.c_int32), ("expert_format", ctypes.c_int32)]


_LIB = None


def lib():
    """The loaded libmoe.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.moe_layer_create.argtypes = [ctypes.POINTER(moe_layer_desc), ctypes.POINTER(ctypes.c_int)]
        L.moe_layer_create.restype = vp
        L.moe_route.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_route.restype = ctypes.c_int
        L.moe_forward.argtypes = [vp, vp, i32, vp, vp]
        L.moe_forward.restype = ctypes.c_int
        L.moe_forward_ev.argtypes = [vp, vp, i32, vp, vp, vp]
        L.moe_forward_ev.restype = ctypes.c_int
        L.moe_forward_noalloc.argtypes = [ctypes.POINTER(moe_layer_desc), vp, i32, vp, vp]
        L.moe_forward_noalloc.restype = ctypes.c_int
        L.moe_layer_free.argtypes = [vp]
        L.moe_layer_free.restype = None
        L.moe_quantize_experts_u8.argtypes = [vp, ctypes.c_uint64, i32, i32, i32, vp,
                                              ctypes.c_uint64, vp]
        L.moe_quantize_experts_u8.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _ptr(t):
    """Device pointer of a tensor, an int, or None (NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def make_desc(hidden, ffn, num_experts, top_k, max_tokens, dtype, router_w, expert_base,
              expert_stride, router_b=None, flags=0, expert_capacity=0,
              expert_format=MOE_EXPERT_DTYPE) -> moe_layer_desc:
    return moe_layer_desc(ctypes.sizeof(moe_layer_desc), hidden, ffn, num_experts, top_k,
                          max_tokens, dtype, flags, _ptr(router_w), _ptr(router_b),
                          _ptr(expert_base), expert_stride, expert_capacity, expert_format)


def u8_stride(H, F):
    """Bytes per uint8 expert: three matrices and the parameter block, to 256."""
    return (3 * H * F + U8_PARAMS_BYTES + 255) // 256 * 256


def moe_quantize_experts_u8(src, src_stride, E, H, F, dst, dst_stride, stream=None):
    rc = lib().moe_quantize_experts_u8(_ptr(src), src_stride, E, H, F, _ptr(dst), dst_stride,
                                       _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_quantize_experts_u8")


def moe_layer_create(desc: moe_layer_desc) -> int:
    st = ctypes.c_int(0)
    h = lib().moe_layer_create(ctypes.byref(desc), ctypes.byref(st))
    if not h:
        raise MoeError(st.value, "moe_layer_create")
    return h


def moe_route(layer, x, T, logits_in, topk_idx, topk_w, counts=None, offsets=None, perm=None,
              inv=None, stream=None):
    rc = lib().moe_route(layer, _ptr(x), T, _ptr(logits_in), _ptr(topk_idx), _ptr(topk_w),
                         _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv), _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_route")


def moe_forward(layer, x, T, y, stream=None):
    rc = lib().moe_forward(layer, _ptr(x), T, _ptr(y), _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_forward")


def moe_forward_ev(layer, x, T, y, stream, stage_events):
    """stage_events: MOE_NUM_STAGES + 1 raw hipEvent_t handles (ints) or None."""
    arr = None
    if stage_events is not None:
        assert len(stage_events) == MOE_NUM_STAGES + 1
        arr = (ctypes.c_void_p * len(stage_events))(*stage_events)
    rc = lib().moe_forward_ev(layer, _ptr(x), T, _ptr(y), _stream(stream), arr)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_forward_ev")


def moe_forward_noalloc(desc: moe_layer_desc, x, T, y, stream=None):
    """The forward that allocates nothing (workspace in the library's static
    device array); desc as for moe_layer_create."""
    rc = lib().moe_forward_noalloc(ctypes.byref(desc), _ptr(x), T, _ptr(y), _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_forward_noalloc")


def moe_layer_free(layer):
    lib().moe_layer_free(layer)


class MoELayer:
    """Owns a libmoe layer handle and keeps the weight tensors it borrows alive."""

    def __init__(self, hidden, ffn, num_experts, top_k, max_tokens, dtype, router_w, experts,
                 expert_stride, router_b=None, flags=0, expert_capacity=0,
                 expert_format=MOE_EXPERT_DTYPE):
        self._keep = (router_w, experts, router_b)
        self.H, self.F, self.E, self.k = hidden, ffn, num_experts, top_k
        self.max_tokens = max_tokens
        self.dtype = dtype
        self.flags = flags
        self.expert_capacity = expert_capacity
        self.expert_format = expert_format
        desc = make_desc(hidden, ffn, num_experts, top_k, max_tokens, dtype, router_w, experts,
                         expert_stride, router_b, flags, expert_capacity, expert_format)
        self.handle = moe_layer_create(desc)

    def forward(self, x, y, T=None, stream=None):
        moe_forward(self.handle, x, x.shape[0] if T is None else T, y, stream)
        return y

    def route(self, x, T, logits_in=None, stream=None):
        import torch
        dev = (x if x is not None else logits_in).device
        S = T * self.k
        out = dict(idx=torch.empty(S, dtype=torch.int32, device=dev),
                   w=torch.empty(S, dtype=torch.float32, device=dev),
                   counts=torch.empty(self.E, dtype=torch.int32, device=dev),
                   offsets=torch.empty(self.E + 1, dtype=torch.int32, device=dev),
                   perm=torch.empty(S, dtype=torch.int32, device=dev),
                   inv=torch.empty(S, dtype=torch.int32, device=dev))
        moe_route(self.handle, x, T, logits_in, out["idx"], out["w"], out["counts"],
                  out["offsets"], out["perm"], out["inv"], stream)
        return out

    def close(self):
        if self.handle:
            moe_layer_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
