"""The captured layer (moe_layer_graph_*), through the C ABI: one-stream and
concurrent captures (the shared expert on a branch beside the routing) give
y equal bit for bit to moe_layer_forward on the same inputs, on every replay,
with the program's own eager work and synchronisations between replays, and
follow new contents of the bound input buffers."""
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


CASES = [
    # config / shape, T, concurrent, shared_unit_rows
    ("config2", 2048, True, 96),
    ("config2", 2048, True, 48),
    ("config2", 2048, False, 0),
    ("config1", 512, True, 96),
    ("edge", 300, True, 32),
    ("config0", 64, True, 0),
    ("decode", 4, True, 0),
    ("noshared", 200, True, 96),
]


def problem(name, T):
    if name.startswith("config"):
        return S.make_problem(int(name[-1]))
    if name == "decode":
        return S.make_custom(T, S.LayerShape(d=2048, f=512, E=256, k=8, f_sh=512), seed=9)
    if name == "noshared":
        return S.make_custom(T, S.LayerShape(d=512, f=256, E=16, k=2, f_sh=0), seed=10)
    return S.make_custom(T, S.LayerShape(d=1024, f=256, E=32, k=4, f_sh=512), seed=11)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,T,concurrent,rows", CASES)
def test_graph_equals_forward(moe, name, T, concurrent, rows):
    p = problem(name, T)
    sh = p.shape
    say(f"graph {name} T={T} concurrent={concurrent} shared rows={rows}")
    layer = moe.Layer.from_numpy(sh.d, sh.f, sh.E, sh.k, sh.f_sh, p.layer)
    x = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).cuda()
    lg = torch.from_numpy(p.logits).cuda()
    y_ref = moe.layer_forward(layer, x, lg)
    y = torch.full_like(y_ref, float("nan"))
    g = moe.LayerGraph(layer, x, lg, y, concurrent=concurrent, shared_unit_rows=rows)
    for rep in range(4):
        y.fill_(float("nan"))
        g.launch()
        # the program's own eager work between replays
        other = moe.layer_forward(layer, x, lg)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep} differs"
        assert torch.equal(other, y_ref)
    # new contents of the bound inputs: the graph recomputes from them
    rng = np.random.default_rng(T)
    lg2 = torch.from_numpy(rng.standard_normal(p.logits.shape).astype(np.float32)).cuda()
    lg.copy_(lg2)
    y2_ref = moe.layer_forward(layer, x, lg2)
    g.launch()
    torch.cuda.synchronize()
    assert torch.equal(y, y2_ref), "graph did not follow the new logits"
    g.close()
