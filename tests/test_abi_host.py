"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/moe_int4.h declares, sizes its workspaces, and rejects bad
arguments before enqueueing anything."""
import ctypes
import os
import re

import pytest

import grouped_int4_dequant_amd as moe
from grouped_int4_dequant_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe_int4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(moe_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("moe_route", "moe_grouped_gemm_int4", "moe_layer_forward", "moe_prefill_chunked",
              "moe_workspace_bytes", "moe_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = moe.load()
    for n in declared_functions():
        assert hasattr(lib, n), n


def qwen_layer_struct(d=2048, f=512, E=256, k=8, f_sh=512, ptr=0x1000):
    return B.MoeLayerT(d, f, E, k, f_sh, *([ptr] * 12))


def test_workspace_sizes():
    L = qwen_layer_struct()
    lib = moe.load()
    ws = lib.moe_workspace_bytes(2048, ctypes.byref(L))
    # x16 + h + h_sh + o + o_sh + the router's logits dominate
    big = 2048 * 2048 * 2 + 16384 * 512 * 2 + 2048 * 512 * 2 + 16384 * 2048 * 2 + 2048 * 2048 * 2 + 2048 * 256 * 4
    assert big < ws < big + 2 * 2 ** 20
    assert ws % 256 == 0
    assert lib.moe_workspace_bytes(2048, ctypes.byref(L)) == lib.moe_workspace_bytes(2048, ctypes.byref(L))
    assert lib.moe_workspace_bytes(0, ctypes.byref(L)) > 0
    assert lib.moe_workspace_bytes(-1, ctypes.byref(L)) == 0
    bad = qwen_layer_struct(d=2000)
    assert lib.moe_workspace_bytes(2048, ctypes.byref(bad)) == 0
    assert lib.moe_max_blocks(2048, 256, 8) == 2048 * 8 // 32 + 256
    assert lib.moe_max_blocks(161, 6, 1) == 12
    assert lib.moe_route_workspace_bytes(2048, 256) > 0
    assert lib.moe_route_workspace_bytes(2048, 4096) == 0


def test_prepared_bytes():
    lib = moe.load()
    L = qwen_layer_struct()
    MiB = 2 ** 20
    # the same bytes as the weights: codes (1 + 0.5 MiB per expert), one
    # 4-byte pair per group (128 + 64 KiB per expert), and the shared expert's
    # (after a 256-byte header of flags)
    expect = 256 + 256 * (MiB + MiB // 2) + 256 * (128 + 64) * 1024 + (MiB + MiB // 2 + 192 * 1024)
    assert lib.moe_prepared_bytes(ctypes.byref(L)) == expect
    assert lib.moe_prepared_bytes(ctypes.byref(qwen_layer_struct(f_sh=0))) == expect - (MiB + MiB // 2 + 192 * 1024)
    # d, f or f_sh not a multiple of 128: no prepared form
    for kw in (dict(d=320), dict(f=192), dict(f_sh=64)):
        assert lib.moe_prepared_bytes(ctypes.byref(qwen_layer_struct(**kw))) == 0
    assert lib.moe_prepared_bytes(None) == 0


def test_prepare_weights_rejects():
    lib = moe.load()
    L = qwen_layer_struct()
    n = lib.moe_prepared_bytes(ctypes.byref(L))
    assert lib.moe_prepare_weights(ctypes.byref(L), 0x1010, n, None) == B.MOE_EINVAL       # misaligned
    assert lib.moe_prepare_weights(ctypes.byref(L), None, n, None) == B.MOE_EINVAL
    assert lib.moe_prepare_weights(ctypes.byref(L), 0x1000, n - 1, None) == B.MOE_EWORKSPACE
    bad = qwen_layer_struct(d=320)
    assert lib.moe_prepare_weights(ctypes.byref(bad), 0x1000, n, None) == B.MOE_EUNSUPPORTED
    # a layer whose prepared copy is misaligned is rejected by the forward call
    L.prep = 0x1010
    assert lib.moe_layer_forward(ctypes.byref(L), 0x1000, 0x1000, 16, 0x1000, None, 0x1000, 1 << 30, None) == B.MOE_EINVAL


def test_status_strings():
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(moe.status_string(code), str) and moe.status_string(code)


@pytest.mark.parametrize("field,value,expect", [
    ("d", 2000, B.MOE_EUNSUPPORTED),
    ("f", 500, B.MOE_EUNSUPPORTED),
    ("f_sh", 100, B.MOE_EUNSUPPORTED),
    ("E", 2048, B.MOE_EUNSUPPORTED),
    ("f", 1 << 21, B.MOE_EUNSUPPORTED),   # one expert's gate/up codes: 2^30 words (4 GiB), past 32-bit byte offsets
    ("k", 300, B.MOE_EINVAL),
    ("k", 0, B.MOE_EINVAL),
    ("gu_q", None, B.MOE_EINVAL),
    ("dn_s", 0x1008, B.MOE_EINVAL),   # misaligned
])
def test_layer_forward_rejects_bad_layers(field, value, expect):
    L = qwen_layer_struct()
    setattr(L, field, value)
    lib = moe.load()
    st = lib.moe_layer_forward(ctypes.byref(L), 0x1000, 0x1000, 16, 0x1000, None, 0x1000, 1 << 30, None)
    assert st == expect


def test_layer_forward_rejects_bad_buffers():
    L = qwen_layer_struct()
    lib = moe.load()
    fwd = lambda *a: lib.moe_layer_forward(ctypes.byref(L), *a)
    assert fwd(None, 0x1000, 16, 0x1000, None, 0x1000, 1 << 30, None) == B.MOE_EINVAL
    assert fwd(0x1000, 0x1000, 16, 0x1004, None, 0x1000, 1 << 30, None) == B.MOE_EINVAL  # y misaligned
    assert fwd(0x1000, 0x1000, -1, 0x1000, None, 0x1000, 1 << 30, None) == B.MOE_EINVAL
    assert fwd(0x1000, 0x1000, 16, 0x1000, None, 0x1000, 100, None) == B.MOE_EWORKSPACE
    assert fwd(0x1000, 0x1000, 0, 0x1000, None, 0x1000, 0, None) == B.MOE_OK  # T == 0: no-op
    assert fwd(0x1000, 0x1000, 1 << 22, 0x1000, None, 0x1000, 1 << 40, None) == B.MOE_EUNSUPPORTED


def test_ablation_entry_point_validates_like_the_forward():
    L = qwen_layer_struct()
    lib = moe.load()
    abl = lambda *a: lib.moe_layer_forward_ablation(ctypes.byref(L), *a)
    for v in moe.ABLATIONS.values():
        assert abl(0x1000, 0x1000, 0, 0x1000, None, 0x1000, 0, None, v) == B.MOE_OK
        assert abl(None, 0x1000, 16, 0x1000, None, 0x1000, 1 << 30, None, v) == B.MOE_EINVAL
        assert abl(0x1000, 0x1000, 16, 0x1000, None, 0x1000, 100, None, v) == B.MOE_EWORKSPACE
    assert abl(0x1000, 0x1000, 16, 0x1000, None, 0x1000, 1 << 40, None, 4) == B.MOE_EINVAL
    assert abl(0x1000, 0x1000, 16, 0x1000, None, 0x1000, 1 << 40, None, -1) == B.MOE_EINVAL
    # the unfused form needs room for one projection's expanded weights
    base = lib.moe_workspace_bytes(16, ctypes.byref(L))
    assert lib.moe_ablation_workspace_bytes(16, ctypes.byref(L), 0) == base
    big = lib.moe_ablation_workspace_bytes(16, ctypes.byref(L), 3)
    assert big - base >= 2 * (256 * 1024 * 2048 + 1024 * 2048)
    assert lib.moe_ablation_workspace_bytes(16, ctypes.byref(L), 4) == 0
    assert abl(0x1000, 0x1000, 16, 0x1000, None, 0x1000, big - 1, None, 3) == B.MOE_EWORKSPACE


def test_router_logits_rejects_bad_arguments():
    lib = moe.load()
    rl = lib.moe_router_logits
    assert rl(0x1000, 0, 64, 0x1000, 16, 0x1000, None) == B.MOE_OK          # T == 0: no-op
    assert rl(None, 4, 64, 0x1000, 16, 0x1000, None) == B.MOE_EINVAL
    assert rl(0x1000, 4, 64, 0x1008, 16, 0x1000, None) == B.MOE_EINVAL      # unaligned
    assert rl(0x1000, -1, 64, 0x1000, 16, 0x1000, None) == B.MOE_EINVAL
    assert rl(0x1000, 4, 48, 0x1000, 16, 0x1000, None) == B.MOE_EUNSUPPORTED  # d % 32
    assert rl(0x1000, 4, 64, 0x1000, 2048, 0x1000, None) == B.MOE_EUNSUPPORTED
    assert rl(0x1000, 1 << 20, 64, 0x1000, 16, 0x1000, None) == B.MOE_EUNSUPPORTED


def test_route_and_gemm_reject_bad_arguments():
    lib = moe.load()
    r = B.MoeRoutingT(*([0x1000] * 9))
    assert lib.moe_route(0x1000, 64, 16, 17, ctypes.byref(r), 0x1000, 1 << 20, None) == B.MOE_EINVAL
    assert lib.moe_route(0x1000, 64, 2048, 8, ctypes.byref(r), 0x1000, 1 << 20, None) == B.MOE_EUNSUPPORTED
    assert lib.moe_route(0x1000, 0, 16, 2, ctypes.byref(r), None, 0, None) == B.MOE_OK  # T == 0
    assert lib.moe_route(None, 64, 16, 2, ctypes.byref(r), None, 0, None) == B.MOE_EINVAL
    assert lib.moe_route(0x1000, 64, 256, 65, ctypes.byref(r), 0x1000, 1 << 20, None) == B.MOE_EUNSUPPORTED
    need = lib.moe_route_workspace_bytes(64, 16)
    assert lib.moe_route(0x1000, 64, 16, 2, ctypes.byref(r), 0x1000, need - 1, None) == B.MOE_EWORKSPACE
    assert lib.moe_route(0x1000, 64, 16, 2, ctypes.byref(r), None, need, None) == B.MOE_EINVAL
    assert lib.moe_route(0x1000, 64, 16, 2, ctypes.byref(r), 0x1010, need, None) == B.MOE_EINVAL  # unaligned
    r0 = B.MoeRoutingT(*([0x1000] * 8 + [None]))
    assert lib.moe_route(0x1000, 64, 16, 2, ctypes.byref(r0), 0x1000, 1 << 20, None) == B.MOE_EINVAL
    g = lib.moe_grouped_gemm_int4
    args = [0x1000, 256, None, 128, 256, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 20, 0x1000, 128, None]
    bad = list(args); bad[3] = 100
    assert g(*bad) == B.MOE_EUNSUPPORTED
    bad = list(args); bad[0] = None
    assert g(*bad) == B.MOE_EINVAL
    bad = list(args); bad[1] = 100
    assert g(*bad) == B.MOE_EINVAL
    bad = list(args); bad[10] = 0
    assert g(*bad) == B.MOE_OK  # no blocks: nothing to do


def test_workspace_size_is_non_decreasing_in_tokens():
    """A workspace sized for T serves every smaller call: the few-token form's
    extra buffer must not make T = 8 need more than T = 9."""
    lib = moe.load()
    for shape in (dict(), dict(E=16, k=2), dict(f_sh=0)):
        L = qwen_layer_struct(**shape)
        sizes = [lib.moe_workspace_bytes(t, ctypes.byref(L)) for t in range(0, 40)]
        assert all(a <= b for a, b in zip(sizes, sizes[1:])), (shape, sizes)


def test_chunked_driver_checks_every_chunk_before_enqueueing():
    """17 tokens in chunks of 9: the 8-token tail takes the few-token form;
    a workspace one byte short of the larger need is rejected up front."""
    L = qwen_layer_struct()
    lib = moe.load()
    need = max(lib.moe_workspace_bytes(9, ctypes.byref(L)), lib.moe_workspace_bytes(8, ctypes.byref(L)))
    assert lib.moe_workspace_bytes(9, ctypes.byref(L)) == need
    st = lib.moe_prefill_chunked(ctypes.byref(L), 0x1000, 0x1000, 17, 9, 0x1000, 0x1000, need - 1, None)
    assert st == B.MOE_EWORKSPACE


def test_workspace_layout_offsets():
    lib = moe.load()
    T, d, f, k, f_sh = 2048, 2048, 512, 8, 512
    L = qwen_layer_struct()
    out = B.MoeWorkspaceLayoutT()
    assert lib.moe_workspace_layout(T, ctypes.byref(L), ctypes.byref(out)) == B.MOE_OK
    ws = lib.moe_workspace_bytes(T, ctypes.byref(L))
    assert out.decode_form == 0 and out.dec_h == -1
    for off in (out.x16, out.h, out.o):
        assert off >= 0 and off % 256 == 0
    assert out.x16 + 2 * T * d <= out.h
    assert out.h_sh == out.h + 2 * T * k * f          # shared rows follow the routed rows
    assert out.o_sh == out.o + 2 * T * k * d
    assert out.o_sh + 2 * T * d <= ws
    assert lib.moe_workspace_layout(1, ctypes.byref(L), ctypes.byref(out)) == B.MOE_OK
    assert out.decode_form == 1 and 0 <= out.dec_h and out.dec_h + 2 * (k + 1) * f <= lib.moe_workspace_bytes(1, ctypes.byref(L))
    assert lib.moe_workspace_layout(0, ctypes.byref(L), ctypes.byref(out)) == B.MOE_EINVAL
    assert lib.moe_workspace_layout(4, ctypes.byref(L), None) == B.MOE_EINVAL
    bad = qwen_layer_struct(d=2000)
    assert lib.moe_workspace_layout(4, ctypes.byref(bad), ctypes.byref(out)) == B.MOE_EINVAL
    L2 = qwen_layer_struct(f_sh=1024)                 # shared width differs: separate buffer
    assert lib.moe_workspace_layout(100, ctypes.byref(L2), ctypes.byref(out)) == B.MOE_OK
    assert out.h_sh >= out.h + 2 * 100 * k * f
    L3 = qwen_layer_struct(f_sh=0)
    assert lib.moe_workspace_layout(100, ctypes.byref(L3), ctypes.byref(out)) == B.MOE_OK
    assert out.h_sh == -1 and out.o_sh == -1
