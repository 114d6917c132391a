"""Pins for the CPU oracle: each step is checked against something other than
the oracle's own code (hand-derived fixtures, brute force, library routines on
special cases, closed forms, identities and invariants). CPU only.

Pages cited (titles as published):
  Lily-EN  "Perplexity Open Sources Lily: A Rust + Metal Inference Engine for
           Qwen3.6-35B-A3B on Apple Silicon" (insight.aitobox.com)
  Lily-ES  "Perplexity open sources Lily: un motor de inferencia ... para
           Qwen3.6-35B-A3B en Apple Silicon" (7minutos.es)
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

from oracle import moe_oracle as O
from synth import moe_inputs as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


def bf16(v):
    """bf16 bits of a float exactly representable in bf16."""
    bits = S.f32_to_bf16_bits(np.float32(v)).reshape(-1)[0]
    assert float(O.bf16_value(bits)) == float(np.float32(v))
    return int(bits)


# ------------------------------------------------------------ P1 dequant ---
def test_unpack_hand_words():
    g = gold("dequant_words.json")
    q = O.unpack_int4(np.array(g["words"], np.uint32))
    assert q.reshape(len(g["words"]), 8).tolist() == g["codes"]


def test_dequant_hand_values():
    g = gold("dequant_words.json")
    words = np.array([g["words"][0], g["words"][1]] * 4, np.uint32)[None, :]  # 64 weights
    s = np.array([[g["scale_bits"]]], np.uint16)
    b = np.array([[g["bias_bits"]]], np.uint16)
    w = O.dequant(words, s, b)[0]
    assert w[:8].tolist() == g["weights_word0"]
    assert w[8:16].tolist() == g["weights_word1"]


def test_dequant_group_boundaries():
    """Scale and bias change exactly at multiples of 64 along the input axis."""
    K = 256
    words = np.full((2, K // 8), 0x33333333, np.uint32)  # q = 3 everywhere
    s = np.array([[bf16(2.0 ** -(g + 3)) for g in range(4)],
                  [bf16(2.0 ** -(g + 5)) for g in range(4)]], np.uint16)
    b = np.array([[bf16(-(g + 1) * 2.0 ** -8) for g in range(4)],
                  [bf16((g + 1) * 2.0 ** -9) for g in range(4)]], np.uint16)
    w = O.dequant(words, s, b)
    for n in range(2):
        for kk in range(K):
            g = kk // 64
            sc = 2.0 ** -(g + 3) if n == 0 else 2.0 ** -(g + 5)
            bi = -(g + 1) * 2.0 ** -8 if n == 0 else (g + 1) * 2.0 ** -9
            assert w[n, kk] == 3 * sc + bi


def test_format_bits_match_checkpoint_size():
    g = gold("checkpoint_size.json")
    bits = 4 + 2 * 16 / g["group"]  # code + (scale + bias) shared by a group
    assert bits == 4.5
    est = g["bf16_gb"] * bits / 16
    assert abs(est - g["int4_gb"]) / g["int4_gb"] < g["rel_tol"]
    shape = S.LayerShape(d=2048, f=512, E=256, k=8, f_sh=512)
    assert S.bytes_per_expert(shape) * 8 == 3 * 2048 * 512 * 4.5


# ---------------------------------------------------- P7 affine identity ---
def test_affine_identity_random():
    """sum_k (s q_k + b) x_k = s * sum q_k x_k + b * sum x_k per 64-group,
    evaluated with integer code sums and math.fsum, independent of dequant."""
    rng = np.random.default_rng(7)
    N, K = 5, 192
    words = rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint32)
    s = S.f32_to_bf16_bits(rng.uniform(0.005, 0.02, (N, K // 64)).astype(np.float32))
    b = S.f32_to_bf16_bits(rng.uniform(-0.2, 0.0, (N, K // 64)).astype(np.float32))
    x = S.f32_to_bf16_bits(rng.standard_normal(K).astype(np.float32))
    xv = [float(v) for v in S.bf16_bits_to_f32(x)]
    W = O.dequant(words, s, b)
    for n in range(N):
        direct = math.fsum(W[n, kk] * xv[kk] for kk in range(K))
        ident = []
        for g in range(K // 64):
            codes = [(int(words[n, (g * 64 + i) // 8]) // 16 ** ((g * 64 + i) % 8)) % 16 for i in range(64)]
            sq = math.fsum(c * xv[g * 64 + i] for i, c in enumerate(codes))
            sx = math.fsum(xv[g * 64:(g + 1) * 64])
            ident.append(float(S.bf16_bits_to_f32(s[n, g])) * sq + float(S.bf16_bits_to_f32(b[n, g])) * sx)
        assert math.isclose(direct, math.fsum(ident), rel_tol=1e-12, abs_tol=1e-12)


# ------------------------------------------------------------ P2 top-k -----
def test_topk_golden_ties():
    for c in gold("topk_ties.json")["cases"]:
        row = np.array([float(v) for v in c["logits"]], np.float32)[None, :]
        assert O.topk(row, c["k"])[0].tolist() == c["ids"], c


def _beats(L, a, e):
    return L[a] > L[e] or (L[a] == L[e] and a < e)


def test_topk_bruteforce_small():
    """Expert e is picked iff fewer than k experts beat it; slot order is the
    rank. Heavy ties (values from a 3-element set including +-0.0)."""
    rng = np.random.default_rng(11)
    vals = np.array([-0.0, 0.0, 1.0], np.float32)
    for _ in range(200):
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, E + 1))
        L = vals[rng.integers(0, 3, E)]
        ids = O.topk(L[None, :], k)[0].tolist()
        rank = {e: sum(_beats(L, a, e) for a in range(E)) for e in range(E)}
        assert sorted(ids) == sorted(e for e in range(E) if rank[e] < k)
        assert [rank[e] for e in ids] == list(range(k))


def test_topk_matches_stable_sort():
    """Library special case: np.lexsort on (index, -logit) gives the same
    total order (both treat -0.0 == +0.0)."""
    rng = np.random.default_rng(3)
    L = rng.standard_normal((50, 16)).astype(np.float32)
    L[:, 5] = L[:, 9]  # forced exact ties
    ids = O.topk(L, 4)
    for t in range(50):
        order = np.lexsort((np.arange(16), -L[t]))
        assert ids[t].tolist() == order[:4].tolist()


# ------------------------------------------------------------ P4 gates -----
def test_gates_properties():
    rng = np.random.default_rng(5)
    L = rng.standard_normal((40, 12)).astype(np.float32)
    for k in (1, 3, 12):
        ids = O.topk(L, k)
        g = O.gates(L, ids)
        assert np.allclose(g.sum(1), 1.0, rtol=0, atol=1e-15)
        full = scipy.special.softmax(L.astype(np.float64), axis=1)
        sel = np.take_along_axis(full, ids.astype(np.int64), 1)
        assert np.allclose(g, sel / sel.sum(1, keepdims=True), rtol=1e-13, atol=0)
        if k == 1:
            assert np.all(g == 1.0)
        if k == 12:  # textbook softmax over all experts, in slot order
            assert np.allclose(g, sel, rtol=1e-13, atol=0)


# ------------------------------------------ P3 histogram / scan / scatter ---
def test_histogram_scan_scatter_invariants():
    rng = np.random.default_rng(9)
    T, E, k = 300, 24, 5
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[:, 3] += 2.0          # a hot expert
    L[:, 7] -= 50.0         # an (almost surely) empty expert
    r = O.route(L, k)
    ids = r["topk_ids"]
    assert r["counts"].sum() == T * k
    assert r["counts"].tolist() == np.bincount(ids.ravel(), minlength=E).tolist()
    assert r["offsets"].tolist() == [0] + np.cumsum(r["counts"]).tolist()
    assert np.all(np.diff(r["offsets"]) >= 0) and r["offsets"][-1] == T * k
    stable = np.argsort(ids.ravel(), kind="stable")
    assert r["sorted_pair"].tolist() == stable.tolist()
    assert sorted(r["sorted_pair"].tolist()) == list(range(T * k))
    assert np.all(r["sorted_token"] == r["sorted_pair"] // k)
    assert np.all(r["pair_pos"][r["sorted_pair"]] == np.arange(T * k))
    for e in range(E):
        seg = r["sorted_token"][r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)  # strictly increasing tokens per expert
        assert np.all(ids.ravel()[r["sorted_pair"][r["offsets"][e]:r["offsets"][e + 1]]] == e)


# ------------------------------------------------------------ P5 block map --
def test_block_map_golden_edges():
    g = gold("block_map_edges.json")
    cnt = np.array(g["counts"], np.int32)
    offs = O.offsets(cnt)
    bm, nb = O.block_map(cnt, offs, g["T"], g["k"])
    assert bm.shape == (g["max_blocks"], 3)
    assert nb == len(g["blocks"])
    assert bm[:nb].tolist() == g["blocks"]
    assert bm[nb:].tolist() == [[-1, 0, 0]] * (g["max_blocks"] - nb)


def test_block_map_invariants():
    rng = np.random.default_rng(13)
    for _ in range(50):
        E = int(rng.integers(1, 20))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 200))
        L = rng.standard_normal((T, E)).astype(np.float32)
        r = O.route(L, k)
        bm, nb = r["block_map"], int(r["num_blocks"])
        assert nb == sum(-(-int(c) // 32) for c in r["counts"]) <= bm.shape[0] == O.max_blocks(T, k, E)
        assert bm[:nb, 2].sum() == T * k and np.all((bm[:nb, 2] >= 1) & (bm[:nb, 2] <= 32))
        rows = np.concatenate([np.arange(b[1], b[1] + b[2]) for b in bm[:nb]])
        assert rows.tolist() == list(range(T * k))
        for b in bm[:nb]:
            assert r["offsets"][b[0]] <= b[1] and b[1] + b[2] <= r["offsets"][b[0] + 1]


# ---------------------------------------------------- closed-form layers ---
def _const_rows_layer(d, f, E, f_sh, row_spec):
    """A layer where every row of every matrix holds one repeated code, with
    bf16-exact scale and bias per row. row_spec(kind, e, n) -> (q, s, b)."""
    def mat(kind, e, n_rows, kdim):
        q = np.empty((n_rows, kdim // 8), np.uint32)
        s = np.empty((n_rows, kdim // 64), np.uint16)
        b = np.empty_like(s)
        for n in range(n_rows):
            qq, ss, bb = row_spec(kind, e, n)
            q[n] = qq * 0x11111111
            s[n] = bf16(ss)
            b[n] = bf16(bb)
        return q, s, b
    lay = {}
    gu = [mat("gu", e, 2 * f, d) for e in range(E)]
    dn = [mat("dn", e, d, f) for e in range(E)]
    lay["gu_q"], lay["gu_s"], lay["gu_b"] = (np.stack([m[i] for m in gu]) for i in range(3))
    lay["dn_q"], lay["dn_s"], lay["dn_b"] = (np.stack([m[i] for m in dn]) for i in range(3))
    if f_sh:
        lay["sh_gu_q"], lay["sh_gu_s"], lay["sh_gu_b"] = mat("gu", "sh", 2 * f_sh, d)
        lay["sh_dn_q"], lay["sh_dn_s"], lay["sh_dn_b"] = mat("dn", "sh", d, f_sh)
    return lay


def _spec(kind, e, n):
    ee = 3 if e == "sh" else e
    if kind == "gu":
        if n < 64:  # gate rows
            return (n + ee) % 16, 2.0 ** -6, -((n + ee) % 3) * 2.0 ** -5
        return (3 * n + 1 + ee) % 16, 2.0 ** -7, 2.0 ** -6
    return (5 * n + 2 + ee) % 16, 2.0 ** -8, -(2.0 ** -5)


def _closed_form_y(c, ee_list, gates_, d=64, f=64):
    """Closed form for constant rows and x = c * ones(d): a_n = d * c * w_n."""
    y = np.zeros(d)
    for ee, g in zip(ee_list, gates_):
        hsum = 0.0
        for n in range(f):
            q, s, b = _spec("gu", ee, n)
            a = d * c * (s * q + b)
            q, s, b = _spec("gu", ee, f + n)
            u = d * c * (s * q + b)
            hsum += a / (1 + math.exp(-a)) * u
        for m in range(d):
            q, s, b = _spec("dn", ee, m)
            y[m] += g * (s * q + b) * hsum
    return y


def test_closed_form_swiglu_layer():
    d, f, E, k = 64, 64, 3, 2
    lay = _const_rows_layer(d, f, E, 64, _spec)
    cs = [1.0, 0.5, -1.0, 2.0]
    x = np.array([[bf16(c)] * d for c in cs], np.uint16)
    # token t picks experts (2, 0) with logits 1.0 and 0.0, expert 1 is lowest
    logits = np.array([[0.0, -4.0, 1.0]] * len(cs), np.float32)
    y = O.moe_forward(lay, x, logits, k)
    g0 = math.e / (1 + math.e)
    for t, c in enumerate(cs):
        exp = _closed_form_y(c, [2, 0, "sh"], [g0, 1 - g0, 1.0])
        assert np.allclose(y[t], exp, rtol=1e-12, atol=1e-12)


def test_zero_input_gives_zero_output():
    p = S.make_problem(0)
    x = np.zeros_like(p.x)
    y = O.moe_forward(p.layer, x, p.logits[:8], p.shape.k, tokens=range(8))
    assert np.all(y == 0.0)


def test_brute_force_tiny_layer():
    """Pure-Python loops with a separate code extraction (integer division)
    and math.fsum, on a tiny random layer."""
    shape = S.LayerShape(d=64, f=64, E=3, k=2, f_sh=64)
    p = S.make_custom(T=3, shape=shape, seed=21)
    lay = p.layer
    y = O.moe_forward(lay, p.x, p.logits, shape.k)

    def code(word, i):
        return (int(word) // 16 ** i) % 16

    def wval(qm, sm, bm, n, kk):
        s = float(S.bf16_bits_to_f32(sm[n, kk // 64]))
        b = float(S.bf16_bits_to_f32(bm[n, kk // 64]))
        return s * code(qm[n, kk // 8], kk % 8) + b

    def ffn(gq, gs, gb, dq, ds, db, xv):
        a = [math.fsum(wval(gq, gs, gb, n, kk) * xv[kk] for kk in range(64)) for n in range(128)]
        h = [a[n] / (1 + math.exp(-a[n])) * a[64 + n] for n in range(64)]
        return [math.fsum(wval(dq, ds, db, m, n) * h[n] for n in range(64)) for m in range(64)]

    for t in range(3):
        xv = [float(v) for v in S.bf16_bits_to_f32(p.x[t])]
        lg = [float(v) for v in p.logits[t]]
        order = sorted(range(3), key=lambda e: (-lg[e], e))[:2]
        ex = [math.exp(lg[e] - lg[order[0]]) for e in order]
        yt = [0.0] * 64
        for e, w in zip(order, ex):
            o = ffn(lay["gu_q"][e], lay["gu_s"][e], lay["gu_b"][e], lay["dn_q"][e], lay["dn_s"][e], lay["dn_b"][e], xv)
            yt = [yt[m] + w / sum(ex) * o[m] for m in range(64)]
        o = ffn(lay["sh_gu_q"], lay["sh_gu_s"], lay["sh_gu_b"], lay["sh_dn_q"], lay["sh_dn_s"], lay["sh_dn_b"], xv)
        yt = [yt[m] + o[m] for m in range(64)]
        assert np.allclose(y[t], yt, rtol=1e-11, atol=1e-12)


# ------------------------------------------------- P9 / P12 / P11 / forms ---
def test_down_projection_linearity():
    p = S.make_problem(0)
    lay2 = dict(p.layer)
    for key in ("dn_s", "dn_b", "sh_dn_s", "sh_dn_b"):
        v = S.bf16_bits_to_f32(p.layer[key]) * np.float32(2.0)  # exact
        lay2[key] = S.f32_to_bf16_bits(v)
    tok = range(16)
    y1 = O.moe_forward(p.layer, p.x, p.logits, p.shape.k, tokens=tok)
    y2 = O.moe_forward(lay2, p.x, p.logits, p.shape.k, tokens=tok)
    assert np.array_equal(y2, 2.0 * y1)


def test_token_permutation_equivariance():
    p = S.make_problem(0)
    perm = np.random.default_rng(1).permutation(p.T)
    y = O.moe_forward(p.layer, p.x, p.logits, p.shape.k)
    yp = O.moe_forward(p.layer, p.x[perm], p.logits[perm], p.shape.k)
    assert np.allclose(yp, y[perm], rtol=1e-13, atol=1e-13)
    r, rp = O.route(p.logits, p.shape.k), O.route(p.logits[perm], p.shape.k)
    assert np.array_equal(rp["topk_ids"], r["topk_ids"][perm])
    assert np.array_equal(rp["counts"], r["counts"])


def test_chunking_matches_full():
    p = S.make_problem(0)
    y = O.moe_forward(p.layer, p.x, p.logits, p.shape.k)
    for lo in range(0, p.T, 24):
        yc = O.moe_forward(p.layer, p.x[lo:lo + 24], p.logits[lo:lo + 24], p.shape.k)
        assert np.allclose(yc, y[lo:lo + 24], rtol=1e-13, atol=1e-13)
    parts = O.route_chunks(p.logits, p.shape.k, 24)
    assert [int(c["counts"].sum()) for c in parts] == [24 * 2, 24 * 2, 16 * 2]


def test_sorted_form_matches_token_form():
    """Combining through sorted rows and pair_pos equals the per-token form,
    and both equal the dense masked form sum_e G[t,e] FFN_e(x_t) with G the
    renormalised softmax restricted to the picked experts."""
    p = S.make_problem(0)
    y_tok = O.moe_forward(p.layer, p.x, p.logits, p.shape.k)
    y_sorted = O.moe_forward_sorted(p.layer, p.x, p.logits, p.shape.k)
    assert np.allclose(y_sorted, y_tok, rtol=1e-12, atol=1e-12)
    X = O.bf16_value(p.x)
    full = scipy.special.softmax(p.logits.astype(np.float64), axis=1)
    thresh = np.sort(p.logits, axis=1)[:, -p.shape.k][:, None]
    G = np.where(p.logits >= thresh, full, 0.0)
    G /= G.sum(1, keepdims=True)
    y_dense = np.zeros_like(X)
    for e in range(p.shape.E):
        gu, dn = O.expert_weights(p.layer, e)
        y_dense += G[:, e:e + 1] * O.swiglu_ffn(X, gu, dn)
    gu, dn = O.expert_weights(p.layer, "sh")
    y_dense += O.swiglu_ffn(X, gu, dn)
    assert np.allclose(y_dense, y_tok, rtol=1e-12, atol=1e-12)


# ------------------------------------------- planted mistakes are caught ---
PIN_TESTS = [test_unpack_hand_words, test_dequant_hand_values, test_dequant_group_boundaries,
             test_affine_identity_random, test_topk_golden_ties, test_topk_bruteforce_small,
             test_gates_properties, test_histogram_scan_scatter_invariants,
             test_block_map_golden_edges, test_closed_form_swiglu_layer,
             test_brute_force_tiny_layer, test_sorted_form_matches_token_form]


# ---------------------------------------------------------- P0 router ---
def test_router_one_hot_rows_pick_weight_columns():
    """x = e_j (one-hot) gives logits[e] = W_r[e][j] exactly."""
    d, E = 64, 12
    rng = np.random.default_rng(7)
    w = S.draw_router(E, d, rng)
    x = np.zeros((d, d), np.uint16)
    x[np.arange(d), np.arange(d)] = bf16(1.0)
    L = O.router_logits(x, w)
    assert np.array_equal(L, O.bf16_value(w).T)


def test_router_brute_force_exact():
    """A tiny case against exact rational arithmetic of the definition."""
    from fractions import Fraction
    x, w = S.make_router_problem(3, 32, 5, seed=11)
    L = O.router_logits(x, w)
    xv, wv = O.bf16_value(x), O.bf16_value(w)
    for t in range(3):
        for e in range(5):
            exact = sum(Fraction(float(xv[t, k])) * Fraction(float(wv[e, k])) for k in range(32))
            assert abs(L[t, e] - float(exact)) <= 1e-14 * max(1.0, abs(float(exact)))


def test_router_equivariance_and_scale():
    """Permuting experts permutes columns; a common permutation of the input
    dimension changes nothing (up to summation order); doubling x doubles the
    logits exactly; constant rows give d * c * sum."""
    x, w = S.make_router_problem(6, 64, 9, seed=12)
    L = O.router_logits(x, w)
    pe = np.random.default_rng(1).permutation(9)
    assert np.array_equal(O.router_logits(x, w[pe]), L[:, pe])
    pk = np.random.default_rng(2).permutation(64)
    assert np.allclose(O.router_logits(x[:, pk], w[:, pk]), L, rtol=1e-12, atol=1e-12)
    x2 = S.f32_to_bf16_bits(2.0 * O.bf16_value(x).astype(np.float32))
    assert np.array_equal(O.router_logits(x2, w), 2.0 * L)
    ones = np.full((2, 64), bf16(1.0), np.uint16)
    c = np.full((3, 64), bf16(0.125), np.uint16)
    assert np.array_equal(O.router_logits(ones, c), np.full((2, 3), 8.0))


PIN_TESTS += [test_router_one_hot_rows_pick_weight_columns, test_router_brute_force_exact,
              test_router_equivariance_and_scale]


def _some_pin_fails():
    for t in PIN_TESTS:
        try:
            t()
        except AssertionError:
            return True
    return False


def _mut_high_nibble_first(words):
    w = np.asarray(words, dtype=np.uint32)
    shifts = np.arange(28, -4, -4, dtype=np.uint32)
    return ((w[..., None] >> shifts) & np.uint32(0xF)).reshape(*w.shape[:-1], w.shape[-1] * 8).astype(np.int64)


def _mut_no_bias(words, s, b):
    return np.repeat(O.bf16_value(s), 64, axis=-1) * O.unpack_int4(words)


def _mut_group_mod(words, s, b):
    q = O.unpack_int4(words).astype(np.float64)
    K = q.shape[-1]
    gi = np.arange(K) % s.shape[-1]  # wrong group index
    return O.bf16_value(s)[..., gi] * q + O.bf16_value(b)[..., gi]


def _mut_tie_high_index(L, k):
    L = np.asarray(L, np.float32)
    return np.array([sorted(range(L.shape[1]), key=lambda e: (-float(L[t, e]), -e))[:k]
                     for t in range(L.shape[0])], np.int32)


def _mut_gate_up_swapped(X, gu_w):
    f = gu_w.shape[0] // 2
    a = X @ gu_w.T
    up, gate = a[:, :f], a[:, f:]
    return gate / (1 + np.exp(-gate)) * up


def _mut_unstable_scatter(ids, offs):
    sp, st, pp = O._orig_scatter(ids, offs)
    E = len(offs) - 1
    for e in range(E):  # reverse within each expert segment
        lo, hi = int(offs[e]), int(offs[e + 1])
        sp[lo:hi], st[lo:hi] = sp[lo:hi][::-1].copy(), st[lo:hi][::-1].copy()
    pp[sp] = np.arange(len(sp))
    return sp, st, pp


def _mut_block_16(cnt, offs, T, k):
    bm, n = O._orig_block_map(cnt, offs, T, k)
    return bm, n + (1 if n else 0)


def _mut_router_drops_last_input(x_bits, w_bits):
    return O.bf16_value(x_bits)[:, :-1] @ O.bf16_value(w_bits)[:, :-1].T


def _mut_router_expert_shift(x_bits, w_bits):
    return O.bf16_value(x_bits) @ np.roll(O.bf16_value(w_bits), 1, axis=0).T


@pytest.mark.parametrize("name,fn", [
    ("router_logits", _mut_router_drops_last_input),
    ("router_logits", _mut_router_expert_shift),
    ("unpack_int4", _mut_high_nibble_first),
    ("dequant", _mut_no_bias),
    ("dequant", _mut_group_mod),
    ("topk", _mut_tie_high_index),
    ("swiglu_h", _mut_gate_up_swapped),
    ("scatter", _mut_unstable_scatter),
    ("block_map", _mut_block_16),
])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(O, "_orig_scatter", O.scatter, raising=False)
    monkeypatch.setattr(O, "_orig_block_map", O.block_map, raising=False)
    monkeypatch.setattr(O, name, fn)
    assert _some_pin_fails(), f"no pin caught a planted mistake in {name}"


def test_planted_gate_mistakes_are_caught(monkeypatch):
    def softmax_all_minus_max(L, ids):  # forgets to renormalise over the k picked
        Lf = np.asarray(L, np.float64)
        full = np.exp(Lf - Lf.max(1, keepdims=True))
        full /= full.sum(1, keepdims=True)
        return np.take_along_axis(full, ids.astype(np.int64), 1)
    monkeypatch.setattr(O, "gates", softmax_all_minus_max)
    assert _some_pin_fails()

    def no_shared(*a, **kw):
        lay = dict(a[0])
        for key in [k for k in lay if k.startswith("sh_")]:
            del lay[key]
        return orig(lay, *a[1:], **kw)
    monkeypatch.undo()
    orig = O.moe_forward
    monkeypatch.setattr(O, "moe_forward", no_shared)
    assert _some_pin_fails()
