"""The fp16 range of the GPU path, through the C ABI (moe_layer_forward_checked):
x, the SwiGLU output h and the expert outputs o are kept in fp16, so values
of magnitude 65520 or more become infinite. The call reports that in the
caller's overflow word; values far below fp16's normal range only lose low
bits and leave the result within tolerance."""
import sys

import numpy as np
import pytest
import torch

import parity
from oracle import moe_oracle as O
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


SHAPE = S.LayerShape(d=2048, f=512, E=16, k=2, f_sh=512)


def run(moe, p, x_bits, start=0):
    layer = moe.Layer.from_numpy(SHAPE.d, SHAPE.f, SHAPE.E, SHAPE.k, SHAPE.f_sh, p.layer)
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()
    lg = torch.from_numpy(p.logits).cuda()
    flag = torch.full((1,), start, dtype=torch.int32, device="cuda")
    y = moe.layer_forward_checked(layer, x, lg, flag)
    torch.cuda.synchronize()
    return y.cpu().numpy(), int(flag.item())


def with_values(p, value, count, seed):
    """x with `count` entries per token set to +-value (bf16)."""
    rng = np.random.default_rng(seed)
    x = p.x.copy()
    for t in range(p.T):
        cols = rng.choice(SHAPE.d, size=count, replace=False)
        sign = rng.choice([-1.0, 1.0], size=count)
        x[t, cols] = S.f32_to_bf16_bits((sign * value).astype(np.float32))
    return x


@pytest.mark.parametrize("T", [64, 1, 4])  # prefill form; one-token and few-token forms
def test_in_range_sets_nothing(moe, T):
    p = S.make_custom(T, SHAPE, seed=300 + T)
    say(f"fp16 range T={T}: ordinary inputs")
    y, flag = run(moe, p, p.x)
    assert flag == 0
    m = O.error_metrics(y, O.moe_forward(p.layer, p.x, p.logits, SHAPE.k))
    assert m["rel_fro"] <= parity.REL_FRO and m["max_over_rms"] <= parity.MAX_OVER_RMS


@pytest.mark.parametrize("T", [64, 1, 4])
def test_large_activations_overflow_h(moe, T):
    """x entries of +-60000 convert to finite fp16 (no X bit), but the SwiGLU
    output of the affected tokens leaves fp16's range: the H bit is set and
    the bits the caller set beforehand are kept."""
    p = S.make_custom(T, SHAPE, seed=310 + T)
    say(f"fp16 range T={T}: x entries of +-60000")
    y, flag = run(moe, p, with_values(p, 60000.0, 4, seed=T), start=8)
    assert flag & 8
    assert not flag & moe.OVERFLOW_X
    assert flag & moe.OVERFLOW_H
    assert not np.all(np.isfinite(y))


@pytest.mark.parametrize("T", [64, 1, 4])
def test_activations_beyond_fp16_set_x(moe, T):
    p = S.make_custom(T, SHAPE, seed=320 + T)
    say(f"fp16 range T={T}: x entries of +-70000")
    _, flag = run(moe, p, with_values(p, 70000.0, 2, seed=T + 1))
    assert flag & moe.OVERFLOW_X


@pytest.mark.parametrize("T", [64, 1, 4])
def test_tiny_activations_stay_in_tolerance(moe, T):
    """A quarter of x below 2^-17 (where fp16 keeps fewer bits than bf16, down
    to its 2^-24 subnormal spacing) and some below 2^-25 (flushed to zero):
    no bit is set and y stays within the tolerance of the exact oracle."""
    p = S.make_custom(T, SHAPE, seed=330 + T)
    rng = np.random.default_rng(T)
    x = p.x.copy()
    mask = rng.random(x.shape) < 0.25
    tiny = rng.choice([3.1e-6, -5.3e-7, 2.2e-8, -1.7e-8], size=x.shape).astype(np.float32)
    x[mask] = S.f32_to_bf16_bits(tiny)[mask]
    say(f"fp16 range T={T}: {int(mask.sum())} entries of x below 2^-17")
    y, flag = run(moe, p, x)
    assert flag == 0
    m = O.error_metrics(y, O.moe_forward(p.layer, x, p.logits, SHAPE.k))
    say(f"  rel_fro={m['rel_fro']:.3e} max/rms={m['max_over_rms']:.3e}")
    assert m["rel_fro"] <= parity.REL_FRO and m["max_over_rms"] <= parity.MAX_OVER_RMS
