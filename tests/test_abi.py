"""The C-ABI library: loads, exports what include/*.h declares, and rejects
bad arguments before touching the GPU (host logic only: no compute calls)."""
import ctypes
import glob
import os
import re

import pytest

import mixture_experts_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b(moe_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_header_declares_the_four_calls():
    assert set(moe.EXPORTED) <= declared_functions()


def test_library_exports_every_declared_symbol():
    lib = moe.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_desc_layout():
    assert ctypes.sizeof(moe.moe_layer_desc) == 72
    assert moe.moe_layer_desc.router_w.offset == 32
    assert moe.moe_layer_desc.expert_stride.offset == 56
    assert moe.moe_layer_desc.expert_capacity.offset == 64
    assert moe.moe_layer_desc.expert_format.offset == 68


def _desc(**kw):
    base = dict(hidden=256, ffn=256, num_experts=8, top_k=2, max_tokens=16, dtype=moe.MOE_BF16,
                router_w=0x10000, expert_base=0x20000, expert_stride=3 * 256 * 256 * 2,
                router_b=None, flags=0)
    base.update(kw)
    return moe.make_desc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(top_k=9, num_experts=8), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(num_experts=0), moe.MOE_ERR_INVALID_ARG),
    (dict(max_tokens=0), moe.MOE_ERR_INVALID_ARG),
    (dict(max_tokens=65537), moe.MOE_ERR_INVALID_ARG),
    (dict(dtype=7), moe.MOE_ERR_INVALID_ARG),
    (dict(router_w=None), moe.MOE_ERR_INVALID_ARG),
    (dict(expert_base=None), moe.MOE_ERR_INVALID_ARG),
    (dict(router_w=0x10008), moe.MOE_ERR_INVALID_ARG),
    (dict(expert_base=0x20004), moe.MOE_ERR_INVALID_ARG),
    (dict(router_b=0x30002), moe.MOE_ERR_INVALID_ARG),
    (dict(expert_stride=3 * 256 * 256 * 2 - 256), moe.MOE_ERR_INVALID_ARG),
    (dict(expert_stride=3 * 256 * 256 * 2 + 128), moe.MOE_ERR_INVALID_ARG),
    (dict(flags=1 << 7), moe.MOE_ERR_INVALID_ARG),
    (dict(expert_capacity=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(flags=moe.MOE_FLAG_PATH_GROUPED | moe.MOE_FLAG_PATH_STREAM), moe.MOE_ERR_INVALID_ARG),
    (dict(num_experts=300, top_k=2), moe.MOE_ERR_UNSUPPORTED),
    # soft routing (k = E) is supported, but its T*k rows must fit the workspace limits
    (dict(top_k=256, num_experts=256, max_tokens=65536), moe.MOE_ERR_UNSUPPORTED),
    (dict(hidden=320, expert_stride=3 * 320 * 256 * 2), moe.MOE_ERR_UNSUPPORTED),
    (dict(ffn=192, expert_stride=3 * 256 * 192 * 2), moe.MOE_ERR_UNSUPPORTED),
    (dict(dtype=moe.MOE_F32, hidden=6, ffn=8, expert_stride=768), moe.MOE_ERR_UNSUPPORTED),
    (dict(dtype=moe.MOE_F32, flags=moe.MOE_FLAG_RESIDUAL_PRENORM,
          expert_stride=3 * 256 * 256 * 4), moe.MOE_ERR_UNSUPPORTED),
    (dict(hidden=65536, ffn=65536, expert_stride=3 * 65536 * 65536 * 2), moe.MOE_ERR_UNSUPPORTED),
    # the residual stream's row is held in registers: H <= 16384
    (dict(hidden=16640, ffn=256, flags=moe.MOE_FLAG_RESIDUAL_PRENORM,
          expert_stride=3 * 16640 * 256 * 2), moe.MOE_ERR_UNSUPPORTED),
    (dict(expert_format=2), moe.MOE_ERR_INVALID_ARG),
    (dict(expert_format=-1), moe.MOE_ERR_INVALID_ARG),
    # uint8 experts: room for the 64-byte parameter block, bf16 layers, streaming path only
    (dict(expert_format=moe.MOE_EXPERT_U8, expert_stride=3 * 256 * 256), moe.MOE_ERR_INVALID_ARG),
    (dict(expert_format=moe.MOE_EXPERT_U8, expert_stride=3 * 256 * 256 + 256 + 128), moe.MOE_ERR_INVALID_ARG),
    (dict(expert_format=moe.MOE_EXPERT_U8, expert_stride=3 * 256 * 256 + 256, dtype=moe.MOE_F32),
     moe.MOE_ERR_UNSUPPORTED),
    (dict(expert_format=moe.MOE_EXPERT_U8, expert_stride=3 * 256 * 256 + 256, flags=moe.MOE_FLAG_PATH_GROUPED),
     moe.MOE_ERR_UNSUPPORTED),
])
def test_create_rejects_bad_descriptors(kw, code):
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_create(_desc(**kw))
    assert ei.value.code == code


def test_struct_size_is_checked():
    d = _desc()
    d.struct_size = 64
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_create(d)
    assert ei.value.code == moe.MOE_ERR_INVALID_ARG


def test_u8_stride_helper():
    assert moe.u8_stride(4096, 14336) == 3 * 4096 * 14336 + 256
    assert moe.u8_stride(256, 256) % 256 == 0 and moe.u8_stride(256, 256) >= 3 * 65536 + 64


@pytest.mark.parametrize("kw", [
    dict(src=None), dict(dst=None), dict(src=0x10008), dict(dst=0x20004), dict(E=0),
    dict(H=24), dict(F=40), dict(src_stride=6 * 256 * 256 - 256), dict(src_stride=6 * 65536 + 16),
    dict(dst_stride=3 * 256 * 256), dict(dst_stride=3 * 65536 + 320),
    dict(dst=0x10000 + 6 * 65536 - 256),                 # overlaps the source
    dict(H=32768, F=32768, src_stride=6 * 2 ** 30, dst_stride=3 * 2 ** 30 + 256),
])
def test_quantize_rejects_bad_arguments(kw):
    args = dict(src=0x10000, src_stride=6 * 256 * 256, E=2, H=256, F=256, dst=0x10000000,
                dst_stride=3 * 256 * 256 + 256)
    args.update(kw)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_quantize_experts_u8(args["src"], args["src_stride"], args["E"], args["H"],
                                    args["F"], args["dst"], args["dst_stride"], stream=0)
    assert ei.value.code == moe.MOE_ERR_INVALID_ARG


def test_null_handle_calls():
    lib = moe.lib()
    assert lib.moe_forward(None, None, 1, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route(None, None, 1, None, None, None, None, None, None, None,
                         None) == moe.MOE_ERR_INVALID_ARG
    lib.moe_layer_free(None)
    st = ctypes.c_int(0)
    assert not lib.moe_layer_create(None, ctypes.byref(st))
    assert st.value == moe.MOE_ERR_INVALID_ARG


def test_binding_constants_match_header():
    """Every MOE_* enumerator of include/moe.h has the same value in the binding."""
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    found = 0
    for name, val in re.findall(r"\b(MOE_[A-Z0-9_]+)\s*=\s*([^,\n}]+)", text):
        v = val.strip()
        m = re.fullmatch(r"1u?\s*<<\s*(\d+)", v)
        num = (1 << int(m.group(1))) if m else int(v, 0)
        assert getattr(moe, name) == num, name
        found += 1
    assert found >= 10
