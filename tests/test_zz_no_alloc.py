"""moe_layer_forward_noalloc (the entry point for callers that cannot
allocate) against moe_layer_forward on the same inputs, through the C ABI:
bit-equal outputs and routing over two calls in a row, the second smaller
than the first (the shared scratch array keeps the first call's contents),
plus a few-token call and the size limit."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from synth import moe_inputs as S

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_int4_dequant_amd as m
    m.load()
    return m


def upload(p, moe):
    sh = p.shape
    layer = moe.Layer.from_numpy(sh.d, sh.f, sh.E, sh.k, sh.f_sh, p.layer)
    x = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).cuda()
    lg = torch.from_numpy(p.logits).cuda()
    return layer, x, lg


def same(a, b):
    return bool(torch.equal(a, b))


@pytest.mark.timeout(300)
def test_noalloc_matches_layer_forward_two_calls_shrinking(moe):
    p = S.make_problem(1)  # T=512, d=2048, f=512, E=256, k=8, shared expert
    sh = p.shape
    layer, x, lg = upload(p, moe)
    for T in (512, 200, 1):  # second and third calls smaller than the first
        say(f"noalloc vs layer_forward T={T}")
        xs, ls = x[:T].contiguous(), lg[:T].contiguous()
        r_ref = moe.alloc_routing(T, sh.E, sh.k)
        r_na = moe.alloc_routing(T, sh.E, sh.k)
        y_ref = moe.layer_forward(layer, xs, ls, routing=r_ref)
        y_na = torch.full_like(y_ref, float("nan"))
        moe.layer_forward_noalloc(layer, xs, ls, y=y_na, routing=r_na)
        torch.cuda.synchronize()
        assert same(y_na, y_ref), f"T={T}: outputs differ"
        for key in r_ref:
            assert same(r_na[key], r_ref[key]), f"T={T}: routing tensor {key} differs"
        # without routing outputs (the few-token form then runs its own top-k)
        y_na2 = moe.layer_forward_noalloc(layer, xs, ls)
        y_ref2 = moe.layer_forward(layer, xs, ls)
        torch.cuda.synchronize()
        assert same(y_na2, y_ref2), f"T={T}: outputs without routing differ"


def test_noalloc_rejects_calls_beyond_the_scratch(moe):
    p = S.make_custom(16, S.LayerShape(d=2048, f=512, E=256, k=8, f_sh=512), seed=3)
    layer, _, _ = upload(p, moe)
    lib = moe.load()
    limit = 64 << 20
    T = 16
    while lib.moe_workspace_bytes(T, ctypes.byref(layer.c)) <= limit:
        T *= 2
    say(f"noalloc refuses T={T} (workspace {lib.moe_workspace_bytes(T, ctypes.byref(layer.c))} B)")
    x = torch.zeros((T, 2048), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((T, 256), dtype=torch.float32, device="cuda")
    y = torch.empty((T, 2048), dtype=torch.float32, device="cuda")
    st = lib.moe_layer_forward_noalloc(ctypes.byref(layer.c), x.data_ptr(), lg.data_ptr(), T, y.data_ptr(),
                                       None, torch.cuda.current_stream().cuda_stream)
    assert st == -3  # MOE_EWORKSPACE, nothing enqueued
