"""Pins of the oracle's fp16 storage emulation and of the acceptance metrics,
and a CPU demonstration that the element-wise emulation bound catches an
indexing mistake the exact-oracle tolerance lets through. CPU only.

Pages cited (titles as published):
  Lily-ES  "Perplexity open sources Lily: un motor de inferencia ... para
           Qwen3.6-35B-A3B en Apple Silicon" (7minutos.es), section
           "Precarga: mantenga los pesos empaquetados, siga enrutando en la
           GPU": 64-weight groups, one bf16 scale and one bf16 bias, FP32
           accumulation.
"""
import json
import math
import os
import struct

import numpy as np
import pytest

import parity
from oracle import moe_oracle as O
from synth import moe_inputs as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


def test_round_fp16_ieee_facts():
    for x, r, _why in gold("fp16_rounding.json")["round"]:
        got = float(O.round_fp16(np.array([float(x)]))[0])
        assert got == float(r), (x, r, got)


def test_ulp_fp16_ieee_facts():
    for x, u in gold("fp16_rounding.json")["ulp"]:
        assert float(O.ulp_fp16(np.array([float(x)]))[0]) == float(u), (x, u)


def _fp16(v: float) -> float:
    """IEEE binary16 round trip through the struct module's 'e' format."""
    return struct.unpack("<e", struct.pack("<e", v))[0]


def test_emulation_brute_force_tiny():
    """Pure-Python loops with struct-module fp16 rounding and exact sums
    (math.fsum) against the oracle's emulate="fp16" on a tiny layer."""
    shape = S.LayerShape(d=128, f=64, E=3, k=2, f_sh=64)
    p = S.make_custom(4, shape, seed=21)
    lay = p.layer
    y_or = O.moe_forward(lay, p.x, p.logits, 2, emulate="fp16")
    ids = O.topk(p.logits, 2)
    g = O.gates(p.logits, ids)

    def weight_rows(q, s, b):
        rows = []
        for n in range(q.shape[0]):
            row = []
            for c in range(q.shape[1]):
                word = int(q[n, c])
                for i in range(8):
                    kk = 8 * c + i
                    sv = float(O.bf16_value(s[n, kk // 64]))
                    bv = float(O.bf16_value(b[n, kk // 64]))
                    row.append(_fp16(sv * ((word >> (4 * i)) & 15) + bv))
            rows.append(row)
        return rows

    def ffn(xrow, gu, dn):
        f = len(gu) // 2
        a = [math.fsum(w * v for w, v in zip(gu[n], xrow)) for n in range(2 * f)]
        h = [_fp16(a[n] / (1.0 + math.exp(-a[n])) * a[f + n]) for n in range(f)]
        return [_fp16(math.fsum(w * v for w, v in zip(dn[m], h))) for m in range(len(dn))]

    W = {e: (weight_rows(lay["gu_q"][e], lay["gu_s"][e], lay["gu_b"][e]),
             weight_rows(lay["dn_q"][e], lay["dn_s"][e], lay["dn_b"][e])) for e in range(3)}
    W["sh"] = (weight_rows(lay["sh_gu_q"], lay["sh_gu_s"], lay["sh_gu_b"]),
               weight_rows(lay["sh_dn_q"], lay["sh_dn_s"], lay["sh_dn_b"]))
    for t in range(4):
        xrow = [_fp16(float(v)) for v in O.bf16_value(p.x[t])]
        y = [0.0] * shape.d
        for j in range(2):
            o = ffn(xrow, *W[int(ids[t, j])])
            y = [a + g[t, j] * b for a, b in zip(y, o)]
        o = ffn(xrow, *W["sh"])
        y = [a + b for a, b in zip(y, o)]
        assert np.allclose(y_or[t], y, rtol=0, atol=1e-12 * max(1.0, max(abs(v) for v in y))), t


def test_emulation_terms_recombine():
    """y of the terms form equals sum_j g_j o_j + o_sh in slot order, and the
    exact (non-emulated) y is unchanged by asking for the terms."""
    p = S.make_problem(0)
    t = O.moe_forward_terms(p.layer, p.x, p.logits, 2, emulate="fp16")
    y = t["g"][:, 0, None] * t["o"][:, 0] + t["g"][:, 1, None] * t["o"][:, 1] + t["o_sh"]
    assert np.array_equal(y, t["y"])
    assert np.array_equal(O.moe_forward_terms(p.layer, p.x, p.logits, 2)["y"],
                          O.moe_forward(p.layer, p.x, p.logits, 2))


def test_emulated_weights_are_fp16_values():
    """Every emulated weight is an fp16 number within half a spacing of the
    exact w = s*q + b."""
    p = S.make_problem(0)
    gu, dn = O.expert_weights(p.layer, 3, "fp16")
    gx, dx = O.expert_weights(p.layer, 3)
    for w16, w in ((gu, gx), (dn, dx)):
        assert np.array_equal(w16.astype(np.float16).astype(np.float64), w16)
        assert np.all(np.abs(w16 - w) <= 0.5 * O.ulp_fp16(w))


# ------------------------------------------- the emulation bound at work ---
def _fp32_storage16_forward(layer, x_bits, logits, k, mutate=None):
    """The layer as a GPU path computes it: weights, x, h and o stored in
    fp16, products accumulated in fp32 (numpy float32 matrix products), gates
    and the combine in fp32. mutate(e, gu16, dn16) may replace an expert's
    weights (a planted mistake)."""
    L = np.asarray(logits, np.float32)
    X = O.round_fp16(O.bf16_value(x_bits)).astype(np.float32)
    ids = O.topk(L, k)
    g = O.gates(L, ids).astype(np.float32)
    Y = np.zeros((L.shape[0], X.shape[1]), np.float32)

    def ffn(rows, e):
        gu, dn = O.expert_weights(layer, e, "fp16")
        if mutate is not None:
            gu, dn = mutate(e, gu, dn)
        gu, dn = gu.astype(np.float32), dn.astype(np.float32)
        f = gu.shape[0] // 2
        a = X[rows] @ gu.T
        h = a[:, :f] / (np.float32(1) + np.exp(-a[:, :f])) * a[:, f:]
        h16 = O.round_fp16(h).astype(np.float32)
        return O.round_fp16(h16 @ dn.T).astype(np.float32)

    for j in range(k):
        for e in np.unique(ids[:, j]):
            rows = np.nonzero(ids[:, j] == e)[0]
            Y[rows] += g[rows, j][:, None] * ffn(rows, int(e))
    if "sh_gu_q" in layer:
        Y += ffn(np.arange(L.shape[0]), "sh")
    return Y.astype(np.float64)


@pytest.fixture(scope="module")
def mid_problem():
    shape = S.LayerShape(d=2048, f=512, E=16, k=2, f_sh=512)
    p = S.make_custom(128, shape, seed=3)
    cache = {}
    exact = O.moe_forward(p.layer, p.x, p.logits, 2, weight_cache=cache)
    emul = O.moe_forward_terms(p.layer, p.x, p.logits, 2, emulate="fp16", weight_cache=cache)
    return p, exact, emul


def test_fp32_accumulation_meets_emulation_bound(mid_problem):
    p, exact, emul = mid_problem
    y = _fp32_storage16_forward(p.layer, p.x, p.logits, 2)
    m = O.error_metrics(y, exact)
    assert m["rel_fro"] <= parity.REL_FRO and m["max_over_rms"] <= parity.MAX_OVER_RMS
    assert parity.emulation_ratio(y, emul, m["rms"]) <= 1.0


def test_planted_scale_misindex_passes_tolerance_but_not_emulation(mid_problem):
    """One gate/up weight column of the first token's first expert reads the
    scale of the next 64-group for one of its groups: the exact-oracle
    tolerance (5e-3 / 2e-2) passes, the element-wise emulation bound fails by
    a wide margin."""
    p, exact, emul = mid_problem
    e0 = int(O.topk(p.logits, 2)[0, 0])

    def misindex(e, gu, dn, n=7, grp=3):
        if e != e0:
            return gu, dn
        s = p.layer["gu_s"][e].copy()
        s[n, grp] = s[n, grp + 1]
        return O.round_fp16(O.dequant(p.layer["gu_q"][e], s, p.layer["gu_b"][e])), dn

    y = _fp32_storage16_forward(p.layer, p.x, p.logits, 2, mutate=misindex)
    m = O.error_metrics(y, exact)
    assert m["rel_fro"] <= parity.REL_FRO and m["max_over_rms"] <= parity.MAX_OVER_RMS, m
    assert parity.emulation_ratio(y, emul, m["rms"]) > 20.0


# ------------------------------------------------- acceptance metrics ---
def test_error_metrics_hand_values():
    for c in gold("error_metrics.json")["cases"]:
        m = O.error_metrics(np.array(c["test"]), np.array(c["ref"]))
        for key in ("rel_fro", "max_over_rms", "rms"):
            assert math.isclose(m[key], c[key], rel_tol=1e-12), (key, m[key], c[key])


def _metrics_rms_of_test(y_test, y_ref):
    yt, yr = np.asarray(y_test, float), np.asarray(y_ref, float)
    rms = np.linalg.norm(yt) / math.sqrt(yt.size)
    d = yt - yr
    return dict(rel_fro=np.linalg.norm(d) / np.linalg.norm(yr), max_over_rms=np.max(np.abs(d)) / rms, rms=rms)


def _metrics_no_abs(y_test, y_ref):
    yt, yr = np.asarray(y_test, float), np.asarray(y_ref, float)
    rms = np.linalg.norm(yr) / math.sqrt(yr.size)
    d = yt - yr
    return dict(rel_fro=np.linalg.norm(d) / np.linalg.norm(yr), max_over_rms=np.max(d) / rms, rms=rms)


def _metrics_swapped(y_test, y_ref):
    return _orig_metrics(y_ref, y_test)


def _metrics_rms_of_diff(y_test, y_ref):
    yt, yr = np.asarray(y_test, float), np.asarray(y_ref, float)
    d = yt - yr
    rms = np.linalg.norm(d) / math.sqrt(d.size)
    return dict(rel_fro=np.linalg.norm(d) / np.linalg.norm(yr), max_over_rms=np.max(np.abs(d)) / rms, rms=rms)


_orig_metrics = O.error_metrics


@pytest.mark.parametrize("fn", [_metrics_rms_of_test, _metrics_no_abs, _metrics_swapped, _metrics_rms_of_diff])
def test_planted_metric_mistakes_are_caught(monkeypatch, fn):
    monkeypatch.setattr(O, "error_metrics", fn)
    with pytest.raises(AssertionError):
        test_error_metrics_hand_values()


def _round_via_fp32(a):
    return np.asarray(a, np.float64).astype(np.float32).astype(np.float16).astype(np.float64)


def _round_toward_zero(a):
    a = np.asarray(a, np.float64)
    r = a.astype(np.float16).astype(np.float64)
    over = np.abs(r) > np.abs(a)
    step = O.ulp_fp16(r) * np.where(np.abs(r) == 2.0 ** np.floor(np.log2(np.maximum(np.abs(r), 1e-300))), 0.5, 1.0)
    return np.where(over, r - np.sign(r) * step, r)


@pytest.mark.parametrize("fn", [_round_via_fp32, _round_toward_zero])
def test_planted_rounding_mistakes_are_caught(monkeypatch, fn):
    monkeypatch.setattr(O, "round_fp16", fn)
    with pytest.raises(AssertionError):
        test_round_fp16_ieee_facts()
