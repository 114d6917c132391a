"""GPU parity at full size and at fp16-rounding tightness, through the C ABI.

For configs 0-3 every output row is compared with the exact fp64 oracle
(relative Frobenius <= 5e-3, max <= 2e-2 * rms) and, element by element, with
the oracle's fp16 storage emulation (tests/parity.py). Stage checks then read
the layer's own fp16 intermediates out of the workspace (moe_workspace_layout)
and hold each stage to its exact value computed from the stage's own GPU
inputs:
  x16  bit-equal to round_fp16(x);
  h    within half an fp16 spacing, plus the fp32 accumulation bound, of the
       exact SwiGLU of the GPU's x16 rows with the expert's fp16 weights;
  o    the same for the exact down projection of the GPU's h rows;
  y    within the fp32 rounding bound of sum_j g_j o_j + o_sh over the GPU's
       own gates and expert outputs.
At least 97 % of the h and o elements must equal the rounded exact value; the
rest are fp32 accumulation errors that sent a rounding the other way.

Pages cited (titles as published):
  Lily-ES  "Perplexity open sources Lily: un motor de inferencia ... para
           Qwen3.6-35B-A3B en Apple Silicon" (7minutos.es), "Precarga: ...":
           64-weight groups with one bf16 scale and bias, FP32 accumulation.
"""
import sys

import numpy as np
import pytest
import torch

import parity
from oracle import moe_oracle as O
from synth import moe_inputs as S

pytestmark = pytest.mark.gpu

ROUTE_KEYS = ("topk_ids", "counts", "offsets", "sorted_pair", "sorted_token", "pair_pos",
              "block_map", "num_blocks")
PERM8 = [0, 4, 1, 5, 2, 6, 3, 7]  # stored position p of an 8-run holds column PERM8[p]
MIN_EXACT_FRACTION = 0.97


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


def check_routing(got, ref):
    for key in ROUTE_KEYS:
        assert np.array_equal(got[key].cpu().numpy().reshape(-1), np.asarray(ref[key]).reshape(-1)), key
    assert np.max(np.abs(got["topk_w"].cpu().numpy().astype(np.float64) - ref["topk_w"])) <= 1e-6


def check_exact(y, y_ref, what):
    m = O.error_metrics(y, y_ref)
    say(f"  {what}: rel_fro={m['rel_fro']:.3e} max/rms={m['max_over_rms']:.3e}")
    assert m["rel_fro"] <= parity.REL_FRO and m["max_over_rms"] <= parity.MAX_OVER_RMS, (what, m)
    return m


def check_emulated(y, terms, rms, what):
    r = parity.emulation_ratio(y, terms, rms)
    m = O.error_metrics(y, terms["y"])
    say(f"  {what}: emulation bound ratio {r:.3f} (max/rms vs emulation {m['max_over_rms']:.2e}, "
        f"rel_fro {m['rel_fro']:.2e})")
    assert r <= 1.0, (what, r)


def unperm8(a):
    a = np.asarray(a)
    r = a.reshape(*a.shape[:-1], -1, 8)
    out = np.empty_like(r)
    out[..., PERM8] = r
    return out.reshape(a.shape)


def ws_fp16(ws, off, shape):
    n = int(np.prod(shape))
    t = ws[off:off + 2 * n].view(torch.float16)
    return t.cpu().numpy().astype(np.float64).reshape(shape)


def gamma(K):
    """Worst-case relative accumulation bound of an fp32 MFMA dot product of
    length K: K/32 steps of 32-term products added to the accumulator."""
    return (K / 32 + 32) * 2.0 ** -24


def check_h_stage(h_gpu, X16, gu16, what):
    f = gu16.shape[0] // 2
    a = X16 @ gu16.T
    sab = np.abs(X16) @ np.abs(gu16).T
    g, u = a[:, :f], a[:, f:]
    silu = g / (1.0 + np.exp(-g))
    h = silu * u
    K = gu16.shape[1]
    dh = 1.1 * np.abs(u) * gamma(K) * sab[:, :f] + np.abs(silu) * gamma(K) * sab[:, f:] + 1e-6 * np.abs(h)
    bound = 0.5 * O.ulp_fp16(np.abs(h) + dh) + dh
    err = np.abs(h_gpu - h)
    worst = float(np.max(err / bound))
    exact = float(np.mean(h_gpu == O.round_fp16(h)))
    assert worst <= 1.0, (what, worst)
    return worst, exact


def check_o_stage(o_gpu, H, dn16, what):
    o = H @ dn16.T
    do = gamma(dn16.shape[1]) * (np.abs(H) @ np.abs(dn16).T) + 1e-6 * np.abs(o)
    bound = 0.5 * O.ulp_fp16(np.abs(o) + do) + do
    worst = float(np.max(np.abs(o_gpu - o) / bound))
    exact = float(np.mean(o_gpu == O.round_fp16(o)))
    assert worst <= 1.0, (what, worst)
    return worst, exact


def stage_checks_prefill(moe, p, layer, ws, y, routing, cache):
    """x16, h, o and y of a prefill-form call against exact stage values."""
    T, sh = p.T, p.shape
    d, f, E, k, fs = sh.d, sh.f, sh.E, sh.k, sh.f_sh
    lay = moe.workspace_layout(T, layer)
    assert lay["decode_form"] == 0
    X = O.bf16_value(p.x)
    x16 = unperm8(ws_fp16(ws, lay["x16"], (T, d)))
    assert np.array_equal(x16, O.round_fp16(X)), "x16 is not round_fp16(x)"
    h = unperm8(ws_fp16(ws, lay["h"], (T * k, f)))
    o = ws_fp16(ws, lay["o"], (T * k, d))
    offs = routing["offsets"].cpu().numpy()
    st = routing["sorted_token"].cpu().numpy()
    worst_h = worst_o = 0.0
    n_eq_h = n_eq_o = 0.0

    def weights(e):
        key = (e, "fp16")
        if key not in cache:
            cache[key] = O.expert_weights(p.layer, e, "fp16")
        return cache[key]

    for e in range(E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            continue
        gu16, dn16 = weights(e)
        wh, eh = check_h_stage(h[lo:hi], x16[st[lo:hi]], gu16, f"h expert {e}")
        wo, eo = check_o_stage(o[lo:hi], h[lo:hi], dn16, f"o expert {e}")
        worst_h, worst_o = max(worst_h, wh), max(worst_o, wo)
        n_eq_h += eh * (hi - lo)
        n_eq_o += eo * (hi - lo)
    rows = T * k
    o_sh = None
    if fs > 0:
        gu16, dn16 = weights("sh")
        h_sh = unperm8(ws_fp16(ws, lay["h_sh"], (T, fs)))
        o_sh = ws_fp16(ws, lay["o_sh"], (T, d))
        wh, eh = check_h_stage(h_sh, x16, gu16, "h shared")
        wo, eo = check_o_stage(o_sh, h_sh, dn16, "o shared")
        worst_h, worst_o = max(worst_h, wh), max(worst_o, wo)
        n_eq_h += eh * T
        n_eq_o += eo * T
        rows += T
    frac_h, frac_o = n_eq_h / rows, n_eq_o / rows
    # y over the GPU's own gates and expert outputs
    gts = routing["topk_w"].cpu().numpy().astype(np.float64)
    pp = routing["pair_pos"].cpu().numpy().reshape(T, k)
    yr = np.zeros((T, d))
    mag = np.zeros((T, d))
    for j in range(k):
        term = gts[:, j, None] * o[pp[:, j]]
        yr += term
        mag += np.abs(term)
    if o_sh is not None:
        yr += o_sh
        mag += np.abs(o_sh)
    worst_y = float(np.max(np.abs(y - yr) / ((k + 2) * 2.0 ** -24 * mag + 1e-30)))
    say(f"  stages: h worst {worst_h:.2f} of bound, {100 * frac_h:.2f}% exact; "
        f"o worst {worst_o:.2f}, {100 * frac_o:.2f}% exact; y worst {worst_y:.2f}")
    assert frac_h >= MIN_EXACT_FRACTION and frac_o >= MIN_EXACT_FRACTION, (frac_h, frac_o)
    assert worst_y <= 1.0, worst_y


def stage_checks_decode(moe, p, layer, ws, y, routing, cache):
    """h per (token, slot) and y of a decode-form call."""
    T, sh = p.T, p.shape
    d, f, k, fs = sh.d, sh.f, sh.k, sh.f_sh
    lay = moe.workspace_layout(T, layer)
    assert lay["decode_form"] == 1
    fmax = max(f, fs)
    hd = unperm8(ws_fp16(ws, lay["dec_h"], (T, k + 1, fmax)))
    X16 = O.round_fp16(O.bf16_value(p.x))
    ids = routing["topk_ids"].cpu().numpy()
    gts = routing["topk_w"].cpu().numpy().astype(np.float64)

    def weights(e):
        key = (e, "fp16")
        if key not in cache:
            cache[key] = O.expert_weights(p.layer, e, "fp16")
        return cache[key]

    yr = np.zeros((T, d))
    dy = np.zeros((T, d))
    mag = np.zeros((T, d))
    worst_h = 0.0
    for t in range(T):
        slots = [(j, int(ids[t, j]), gts[t, j]) for j in range(k)] + ([(k, "sh", 1.0)] if fs > 0 else [])
        for j, e, gj in slots:
            gu16, dn16 = weights(e)
            hh = hd[t, j, :gu16.shape[0] // 2][None, :]
            wh, _ = check_h_stage(hh, X16[t:t + 1], gu16, f"decode h t={t} slot {j}")
            worst_h = max(worst_h, wh)
            o = (hh @ dn16.T)[0]
            yr[t] += gj * o
            dy[t] += abs(gj) * gamma(dn16.shape[1]) * (np.abs(hh) @ np.abs(dn16).T)[0]
            mag[t] += np.abs(gj * o)
    worst_y = float(np.max(np.abs(y - yr) / (dy + (k + 3) * 2.0 ** -24 * mag + 1e-30)))
    say(f"  decode stages: h worst {worst_h:.2f} of bound; y worst {worst_y:.2f}")
    assert worst_y <= 1.0, worst_y


def run_layer(moe, p, layer, x, lg):
    ws = moe.alloc_workspace(moe.workspace_bytes(p.T, layer))
    routing = moe.alloc_routing(p.T, p.shape.E, p.shape.k)
    y = moe.layer_forward(layer, x, lg, routing=routing, ws=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64), routing, ws


@pytest.mark.timeout(900)
@pytest.mark.parametrize("index", [0, 1, 2])
def test_layer_config_every_row(moe, index):
    p = S.make_problem(index)
    k = p.shape.k
    say(f"config {index}: T={p.T}, every output row; emulation bound; stage checks")
    layer, x, lg = upload(p, moe)
    y, routing, ws = run_layer(moe, p, layer, x, lg)
    check_routing(routing, O.route(p.logits, k))
    cache = {}
    m = check_exact(y, O.moe_forward(p.layer, p.x, p.logits, k, weight_cache=cache), f"config {index} exact")
    check_emulated(y, O.moe_forward_terms(p.layer, p.x, p.logits, k, emulate="fp16", weight_cache=cache),
                   m["rms"], f"config {index}")
    stage_checks_prefill(moe, p, layer, ws, y, routing, cache)


EDGE_SHAPES = [
    # T, d, f, E, k, f_sh  (prefill form; T > 8)
    (65, 64, 64, 3, 1, 0),
    (129, 320, 192, 8, 8, 64),
    (33, 2048, 512, 256, 8, 512),
    (300, 512, 320, 12, 3, 192),
    (50, 2560, 192, 4, 2, 64),
    (40, 448, 576, 5, 2, 0),
    (256, 1024, 256, 64, 4, 256),
    (130, 1536, 1024, 6, 2, 1024),
    (192, 512, 512, 2, 1, 512),
    (60, 512, 512, 4, 2, 1024),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("T,d,f,E,k,f_sh", EDGE_SHAPES)
def test_edge_shapes_emulation_and_stages(moe, T, d, f, E, k, f_sh):
    p = S.make_custom(T, S.LayerShape(d=d, f=f, E=E, k=k, f_sh=f_sh), seed=T + d + f)
    say(f"edge T={T} d={d} f={f} E={E} k={k} f_sh={f_sh}: emulation bound; stage checks")
    layer, x, lg = upload(p, moe)
    y, routing, ws = run_layer(moe, p, layer, x, lg)
    check_routing(routing, O.route(p.logits, k))
    cache = {}
    m = check_exact(y, O.moe_forward(p.layer, p.x, p.logits, k, weight_cache=cache), "exact")
    check_emulated(y, O.moe_forward_terms(p.layer, p.x, p.logits, k, emulate="fp16", weight_cache=cache),
                   m["rms"], "edge")
    stage_checks_prefill(moe, p, layer, ws, y, routing, cache)


DECODE_SHAPES = [
    # T, E, k, f_sh  (d = 2048, f = 512: the few-token form)
    (1, 256, 8, 512),
    (4, 256, 8, 512),
    (3, 64, 4, 0),
    (8, 1024, 8, 512),
    (8, 16, 8, 0),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("T,E,k,f_sh", DECODE_SHAPES)
def test_decode_emulation_and_stages(moe, T, E, k, f_sh):
    p = S.make_custom(T, S.LayerShape(d=2048, f=512, E=E, k=k, f_sh=f_sh), seed=200 + T + E + k)
    say(f"decode T={T} E={E} k={k} f_sh={f_sh}: emulation bound; stage checks")
    layer, x, lg = upload(p, moe)
    y, routing, ws = run_layer(moe, p, layer, x, lg)
    check_routing(routing, O.route(p.logits, k))
    cache = {}
    m = check_exact(y, O.moe_forward(p.layer, p.x, p.logits, k, weight_cache=cache), "exact")
    check_emulated(y, O.moe_forward_terms(p.layer, p.x, p.logits, k, emulate="fp16", weight_cache=cache),
                   m["rms"], "decode")
    stage_checks_decode(moe, p, layer, ws, y, routing, cache)


@pytest.mark.timeout(900)
def test_chunked_config3_every_row(moe):
    """Config 3 through moe_prefill_chunked: every output row against the
    exact oracle and the emulation bound, and y equal bit for bit to
    per-chunk moe_layer_forward calls whose routing outputs (the routing
    the chunked driver runs) match the oracle's per-chunk routing."""
    p = S.make_problem(3)
    k, C = p.shape.k, 2048
    say("config 3: T=8192 in 2048-token chunks (skewed), every row")
    layer, x, lg = upload(p, moe)
    y = moe.prefill_chunked(layer, x, lg, chunk=C)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    ref_chunks = O.route_chunks(p.logits, k, C)
    ws = moe.alloc_workspace(moe.workspace_bytes(C, layer))
    for c, ref in enumerate(ref_chunks):
        r = moe.alloc_routing(C, p.shape.E, k)
        yc = moe.layer_forward(layer, x[c * C:(c + 1) * C].contiguous(), lg[c * C:(c + 1) * C].contiguous(),
                               routing=r, ws=ws)
        torch.cuda.synchronize()
        check_routing(r, ref)
        assert np.array_equal(yc.cpu().numpy(), y[c * C:(c + 1) * C]), f"chunk {c} differs from the chunked call"
        say(f"  chunk {c}: touched experts {int((ref['counts'] > 0).sum())}, max rows {int(ref['counts'].max())}")
    cache = {}
    m = check_exact(y, O.moe_forward(p.layer, p.x, p.logits, k, weight_cache=cache), "config 3 exact")
    check_emulated(y, O.moe_forward_terms(p.layer, p.x, p.logits, k, emulate="fp16", weight_cache=cache),
                   m["rms"], "config 3")


@pytest.mark.timeout(300)
def test_chunked_ragged_tail_switches_form(moe):
    """17 tokens in chunks of 9: the 8-token tail takes the few-token form in
    the middle of the driver, on the workspace sized for the first chunk."""
    p = S.make_custom(17, S.LayerShape(d=2048, f=512, E=64, k=8, f_sh=512), seed=17)
    say("chunked 17 tokens in chunks of 9")
    layer, x, lg = upload(p, moe)
    ws = moe.alloc_workspace(moe.workspace_bytes(9, layer))
    y = moe.prefill_chunked(layer, x, lg, chunk=9, ws=ws)
    torch.cuda.synchronize()
    check_exact(y.cpu().numpy(), O.moe_forward(p.layer, p.x, p.logits, 8), "chunked 9+8")
