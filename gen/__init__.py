"""Seeded synthetic inputs for the MoE layer (host side).

This module is the only thing the oracle side and the GPU side share: it
produces the input tensors (tokens, router, expert weights, router bias) and
holds none of the layer's arithmetic.  Every value is defined in
``gen/gen_core.h``: splitmix64 counters feeding Box-Muller, rounded to fp32
and, for bf16 storage, to bf16 (both round-to-nearest-even).

Storage conventions (the same on both sides):
  x          [T][H]           dtype
  router_w   [H][E]           dtype   (element (h, e) at h*E + e)
  router_b   [E]              fp32 or None
  experts    E blocks of ``stride`` bytes; block e holds
               Wg [F][H], Wu [F][H], Wd [H][F]   dtype
             (each projection stored output-major: element (h, f) of the
              logical [H, F] gate matrix sits at f*H + h)
Counter index of an element is its storage offset within its tensor, with
expert e's matrices offset by e*F*H.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

T_X, T_WR, T_WG, T_WU, T_WD = 0, 1, 2, 3, 4

SIGMA_X = 1.0
SIGMA_W = 0.02


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "libgen.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        u64, u32, i64, i32, dbl = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                   ctypes.c_int32, ctypes.c_double)
        vp = ctypes.c_void_p
        L.gen_splitmix64_output.argtypes = [u64, u64]
        L.gen_splitmix64_output.restype = u64
        L.gen_state.argtypes = [u64, u32, u32]
        L.gen_state.restype = u64
        L.gen_log01_host.argtypes = [dbl]
        L.gen_log01_host.restype = dbl
        L.gen_cos2pi01_host.argtypes = [dbl]
        L.gen_cos2pi01_host.restype = dbl
        for name in ("gen_normal_f64", "gen_normal_f32", "gen_normal_bf16"):
            fn = getattr(L, name)
            fn.argtypes = [u64, u32, u32, u64, i64, dbl, vp]
            fn.restype = None
        L.gen_zipf_bias.argtypes = [i32, dbl, dbl, vp]
        L.gen_zipf_bias.restype = None
        _LIB = L
    return _LIB


_DEV = None


def devlib():
    """The device generator (gen/libgendev.so, HIP); same values as `normal`."""
    global _DEV
    if _DEV is None:
        path = os.path.join(_HERE, "libgendev.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        for name in ("gen_device_normal_bf16", "gen_device_normal_f32"):
            fn = getattr(L, name)
            fn.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint64,
                           ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p]
            fn.restype = ctypes.c_int
        _DEV = L
    return _DEV


def normal_device(seed: int, layer: int, tensor: int, n: int, sigma: float, dtype: str,
                  out_ptr: int, idx0: int = 0, stream: int = 0) -> None:
    """Values idx0 .. idx0+n-1 of stream (seed, layer, tensor) into device
    memory at out_ptr (bf16 bits or fp32), bit-identical to `normal`."""
    fn = {"bf16": devlib().gen_device_normal_bf16, "f32": devlib().gen_device_normal_f32}[dtype]
    rc = fn(seed, layer, tensor, idx0, n, sigma, out_ptr, stream)
    if rc != 0:
        raise RuntimeError(f"device generator failed ({rc})")


def experts_device(shape: "LayerShape", base_ptr: int, layer: int = 0, seed: int | None = None,
                   stream: int = 0) -> None:
    """gen_experts(shape, layer) written straight into device memory at base_ptr
    (E blocks of shape.stride bytes; padding bytes are left untouched)."""
    s = shape.seed if seed is None else seed
    per = shape.H * shape.F
    for e in range(shape.E):
        base = base_ptr + e * shape.stride
        for j, tid in enumerate((T_WG, T_WU, T_WD)):
            normal_device(s, layer, tid, per, SIGMA_W, shape.dtype,
                          base + j * per * shape.elem, idx0=e * per, stream=stream)


def normal(seed: int, layer: int, tensor: int, n: int, sigma: float, dtype: str,
           idx0: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """Values idx0 .. idx0+n-1 of stream (seed, layer, tensor).

    dtype: "f64" (no rounding), "f32", or "bf16" (returned as uint16 bits).
    """
    npdt = {"f64": np.float64, "f32": np.float32, "bf16": np.uint16}[dtype]
    if out is None:
        out = np.empty(n, dtype=npdt)
    assert out.dtype == npdt and out.size == n and out.flags.c_contiguous
    fn = {"f64": lib().gen_normal_f64, "f32": lib().gen_normal_f32,
          "bf16": lib().gen_normal_bf16}[dtype]
    fn(seed, layer, tensor, idx0, n, sigma, out.ctypes.data)
    return out


def zipf_bias(E: int, s: float = 1.1, scale: float = 2.0) -> np.ndarray:
    out = np.empty(E, dtype=np.float32)
    lib().gen_zipf_bias(E, s, scale, out.ctypes.data)
    return out


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class LayerShape:
    name: str
    H: int
    F: int
    E: int
    k: int
    dtype: str  # "f32" or "bf16"
    bias: str = "none"  # "none" or "zipf"
    seed: int = 0

    @property
    def elem(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def expert_bytes(self) -> int:
        return 3 * self.H * self.F * self.elem

    @property
    def stride(self) -> int:
        return (self.expert_bytes + 255) // 256 * 256

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == "f32" else np.uint16


# The five workloads: shapes, dtypes and routing-bias recipe.
TINY = LayerShape("tiny_f32", H=64, F=128, E=8, k=2, dtype="f32")
MIXTRAL = LayerShape("mixtral_8x7b_layer", H=4096, F=14336, E=8, k=2, dtype="bf16")
QWEN = LayerShape("qwen2_moe_layer", H=2048, F=1408, E=64, k=2, dtype="bf16")
DEEPSEEK = LayerShape("deepseek_moe_layer", H=2048, F=1408, E=128, k=4, dtype="bf16",
                      bias="zipf")
CONFIGS = {"tiny": (TINY, [32]), "mixtral": (MIXTRAL, [1, 4096]), "qwen": (QWEN, [512]),
           "deepseek": (DEEPSEEK, [8192]), "stack": (MIXTRAL, [1, 4, 16, 64])}
STACK_LAYERS = 32


def gen_x(shape: LayerShape, T: int, layer: int = 0, seed: int | None = None) -> np.ndarray:
    s = shape.seed if seed is None else seed
    return normal(s, layer, T_X, T * shape.H, SIGMA_X, shape.dtype).reshape(T, shape.H)


def gen_router(shape: LayerShape, layer: int = 0, seed: int | None = None) -> np.ndarray:
    s = shape.seed if seed is None else seed
    return normal(s, layer, T_WR, shape.H * shape.E, SIGMA_W, shape.dtype).reshape(
        shape.H, shape.E)


def gen_bias(shape: LayerShape) -> np.ndarray | None:
    if shape.bias == "zipf":
        return zipf_bias(shape.E)
    return None


def gen_experts(shape: LayerShape, layer: int = 0, seed: int | None = None,
                experts: range | list | None = None) -> np.ndarray:
    """Expert blob as a flat byte array: E blocks of shape.stride bytes.

    ``experts`` limits generation to those expert ids (the others stay zero),
    which is how a checker regenerates only the experts it needs.
    """
    s = shape.seed if seed is None else seed
    H, F, E = shape.H, shape.F, shape.E
    blob = np.zeros(E * shape.stride, dtype=np.uint8)
    per = H * F
    for e in (range(E) if experts is None else experts):
        base = e * shape.stride
        view = blob[base: base + 3 * per * shape.elem].view(shape.np_dtype)
        for j, tid in enumerate((T_WG, T_WU, T_WD)):
            normal(s, layer, tid, per, SIGMA_W, shape.dtype, idx0=e * per,
                   out=view[j * per:(j + 1) * per])
    return blob


def expert_views(shape: LayerShape, blob: np.ndarray, e: int):
    """(Wg [F,H], Wu [F,H], Wd [H,F]) storage views of expert e (dtype bits)."""
    H, F = shape.H, shape.F
    per = H * F
    base = e * shape.stride
    v = blob[base: base + 3 * per * shape.elem].view(shape.np_dtype)
    return v[:per].reshape(F, H), v[per:2 * per].reshape(F, H), v[2 * per:].reshape(H, F)
