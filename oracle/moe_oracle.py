"""CPU oracle for the grouped int4-dequant MoE layer (fp64, plain and slow).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke entry point and the
benchmark's CPU-baseline leg may import this module. The GPU library never
calls it, and it shares no code with the GPU path: it reads the same seeded
inputs and nothing else.

What it computes, step by step, in the order the pages describe the layer
(pages keyed below):

  0. router     logits = x W_r^T from bf16 token activations and bf16 router
                weights (Lily-EN "Three Workload Shapes": the router scores
                every expert for each token); the layer itself takes logits
                as an input
  1. unpack     4-bit codes, eight per uint32, low nibble first
  2. dequant    w = s * q + b, one bf16 scale and one bf16 bias per 64
                consecutive input-dimension weights
                (Lily-ES "Precarga..."; Lily-HE prefill section; Lily-FR)
  3. top-k      the k largest router logits per token, ties to the lower
                expert index (Lily-EN "Three Workload Shapes": a router scores
                256 experts and picks 8)
  4. gates      softmax over the k selected logits
  5-8. routing  per-expert histogram, exclusive prefix scan, stable scatter of
                (token, slot) pairs into expert order, and the map of 32-row
                blocks (Lily-EN "Prefill: Keep Weights Packed, Keep Routing on
                the GPU"; Lily-ES "Precarga..." for the 32-row tiles)
  9. expert FFN SwiGLU: h = silu(W_gate x) * (W_up x), o = W_down h
  10. shared    the same FFN for the shared expert, on every token
  11. combine   y_t = sum_j g_tj * o_(t,j) + o_shared(t)

Readings where the pages are silent (each is listed with its reason in the
design notes): affine form w = s*q + b with unsigned q; groups run along the
input dimension; logits are an input; gates are the softmax over the k picked
logits; ties go to the lower expert index under IEEE equality (-0.0 == +0.0);
the shared expert is added with weight 1; the activation is SwiGLU with gate
rows first; the scatter is stable in ascending pair index t*k+j; the block map
holds (expert, first row, row count) triples over unpadded offsets.

Diagnostic mode (not part of the method): emulate="fp16" rounds to the
nearest fp16 exactly the values the GPU path stores in fp16 (the rebuilt
weights, x entering the matrix cores, h and each expert's output o) and keeps
everything else exact, so a correct GPU result is within a few fp16 roundings
of it element by element; tests use it to catch indexing mistakes that the
5e-3 relative tolerance against the exact result would hide.

Parity pins (tests/test_oracle_pins.py) tie every step to something other than
this code: hand-packed words, a brute-force top-k, library-routine special
cases, the per-group affine identity, closed-form SwiGLU layers, linearity,
equivariance, the dense masked form of the combine, hand-computed error
metrics, IEEE binary16 rounding facts and a pure-Python brute force of the
fp16 emulation. Full-size expert FFN values are pinned only through those
identities (parity unpinned beyond them).

Pages cited (titles as published):
  Lily-EN  "Perplexity Open Sources Lily: A Rust + Metal Inference Engine for
           Qwen3.6-35B-A3B on Apple Silicon" (insight.aitobox.com)
  Lily-ES  "Perplexity open sources Lily: un motor de inferencia ... para
           Qwen3.6-35B-A3B en Apple Silicon" (7minutos.es)
  Lily-FR  "Perplexity Open Sources Lily : un moteur d'inférence Rust + Metal
           pour Qwen3.6-35B-A3B sur Apple Silicon" (cmedia.click)
  Lily-HE  the agentnet.co.il article on Lily (Hebrew), prefill section
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

GROUP = 64
BLOCK_ROWS = 32


# ---------------------------------------------------------------- formats ---
def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def unpack_int4(words) -> np.ndarray:
    """Step 1. Packed uint32 [..., K/8] -> codes [..., K] with
    q[..., 8c+i] = (words[..., c] >> 4i) & 0xF (low nibble first)."""
    w = np.asarray(words, dtype=np.uint32)
    shifts = np.arange(0, 32, 4, dtype=np.uint32)
    q = (w[..., None] >> shifts) & np.uint32(0xF)
    return q.reshape(*w.shape[:-1], w.shape[-1] * 8).astype(np.int64)


def dequant(words, scale_bits, bias_bits) -> np.ndarray:
    """Step 2 (Lily-ES "Precarga..."; Lily-HE prefill section): groupwise
    affine 4-bit weights, 64 consecutive input-dimension weights sharing one
    bf16 scale and one bf16 bias: W[n][k] = s[n][k//64] * q[n][k] + b[n][k//64].
    Exact in float64."""
    q = unpack_int4(words).astype(np.float64)
    s = np.repeat(bf16_value(scale_bits), GROUP, axis=-1)
    b = np.repeat(bf16_value(bias_bits), GROUP, axis=-1)
    assert q.shape == s.shape == b.shape
    return s * q + b


# ---------------------------------------------------------------- routing ---
def router_logits(x_bits, w_bits) -> np.ndarray:
    """Step 0 (Lily-EN "Three Workload Shapes"): the router's score of every
    expert for every token, logits[t][e] = sum_k x[t][k] * W_r[e][k], from
    bf16 x [T][d] and bf16 W_r [E][d], in float64 (a library matrix product
    on exactly widened values)."""
    return bf16_value(x_bits) @ bf16_value(w_bits).T


def topk(logits, k: int) -> np.ndarray:
    """Step 3 (Lily-EN "Three Workload Shapes"): for every token the k experts
    with the largest logits, listed by (logit descending, expert ascending).
    Python float comparison is IEEE comparison, so -0.0 and +0.0 tie and the
    lower index wins."""
    L = np.asarray(logits, dtype=np.float32)
    T, E = L.shape
    assert 1 <= k <= E
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        row = [float(v) for v in L[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))
        ids[t] = order[:k]
    return ids


def gates(logits, ids) -> np.ndarray:
    """Step 4: g[t][j] = exp(L_j - L_0) / sum_i exp(L_i - L_0) over the k
    selected logits (L_0 the largest), in float64."""
    L = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, k = ids.shape
    g = np.empty((T, k), np.float64)
    for t in range(T):
        sel = [L[t, e] for e in ids[t]]
        ex = [math.exp(v - sel[0]) for v in sel]
        tot = math.fsum(ex)
        g[t] = [v / tot for v in ex]
    return g


def counts(ids, E: int) -> np.ndarray:
    """Step 5 (routing histogram, Lily-EN "Prefill..."): pairs per expert."""
    c = np.zeros(E, np.int64)
    for e in np.asarray(ids).ravel():
        c[e] += 1
    return c.astype(np.int32)


def offsets(cnt) -> np.ndarray:
    """Step 6 (prefix scan): offsets[e] = sum of counts of experts < e;
    offsets[E] = total pairs."""
    out = [0]
    for c in cnt:
        out.append(out[-1] + int(c))
    return np.asarray(out, np.int32)


def scatter(ids, offs) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Step 7 (scatter): visit pairs in ascending t*k+j; each goes to the next
    free row of its expert's segment. Returns sorted_pair[T*k],
    sorted_token[T*k] and pair_pos[T*k]."""
    T, k = ids.shape
    cursor = [int(o) for o in offs[:-1]]
    sorted_pair = np.full(T * k, -1, np.int32)
    sorted_token = np.full(T * k, -1, np.int32)
    pair_pos = np.full(T * k, -1, np.int32)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            pos = cursor[e]
            cursor[e] += 1
            sorted_pair[pos] = t * k + j
            sorted_token[pos] = t
            pair_pos[t * k + j] = pos
    return sorted_pair, sorted_token, pair_pos


def max_blocks(T: int, k: int, E: int) -> int:
    """Upper bound on 32-row blocks: ceil(T*k/32) + E (one partial block per
    expert at most)."""
    return -(-T * k // BLOCK_ROWS) + E


def block_map(cnt, offs, T: int, k: int) -> Tuple[np.ndarray, int]:
    """Step 8 (block map, 32-row tiles: Lily-ES "Precarga..."): for each expert
    with rows, in expert order, blocks b = 0..ceil(c/32)-1 as triples
    (e, offsets[e] + 32b, min(32, c - 32b)). Entries past the count hold
    (-1, 0, 0)."""
    E = len(cnt)
    mb = max_blocks(T, k, E)
    bm = np.zeros((mb, 3), np.int32)
    bm[:, 0] = -1
    n = 0
    for e in range(E):
        c = int(cnt[e])
        b = 0
        while BLOCK_ROWS * b < c:
            bm[n] = (e, int(offs[e]) + BLOCK_ROWS * b, min(BLOCK_ROWS, c - BLOCK_ROWS * b))
            n += 1
            b += 1
    return bm, n


def route(logits, k: int) -> Dict[str, np.ndarray]:
    """Steps 3-8 for one call (one chunk)."""
    L = np.asarray(logits, dtype=np.float32)
    T, E = L.shape
    ids = topk(L, k)
    g = gates(L, ids)
    cnt = counts(ids, E)
    offs = offsets(cnt)
    sp, st, pp = scatter(ids, offs)
    bm, nb = block_map(cnt, offs, T, k)
    return dict(topk_ids=ids, topk_w=g, counts=cnt, offsets=offs, sorted_pair=sp,
                sorted_token=st, pair_pos=pp, block_map=bm, num_blocks=np.int32(nb))


# -------------------------------------------------------------- expert FFN ---
def swiglu_h(X, gu_w) -> np.ndarray:
    """Step 9, first half, for a batch of rows of one expert: a = X W_gu^T
    (gate columns 0..f-1, up columns f..2f-1) and h = silu(gate) * up, with
    silu(z) = z / (1 + exp(-z)). X float64 [m, d]; gu_w float64 [2f, d]."""
    f = gu_w.shape[0] // 2
    a = np.asarray(X, np.float64) @ np.asarray(gu_w, np.float64).T
    gate, up = a[:, :f], a[:, f:]
    return gate / (1.0 + np.exp(-gate)) * up


def down_proj(h, dn_w) -> np.ndarray:
    """Step 9, second half: o = h W_dn^T. h float64 [m, f]; dn_w float64 [d, f]."""
    return np.asarray(h, np.float64) @ np.asarray(dn_w, np.float64).T


def swiglu_ffn(X, gu_w, dn_w) -> np.ndarray:
    """Step 9 for a batch of rows of one expert: o = (silu(X W_g^T) * X W_u^T) W_dn^T."""
    return down_proj(swiglu_h(X, gu_w), dn_w)


# ------------------------------------------------- fp16 storage emulation ---
# A diagnostic, not part of the method. The GPU path keeps four kinds of
# values in fp16: the rebuilt weights, the activations entering the matrix
# cores, the SwiGLU output h and each expert's output o (y stays fp32). With
# emulate="fp16" the oracle rounds exactly those values to the nearest fp16
# (ties to even) and computes everything else exactly, so its result differs
# from a correct GPU result only by the GPU's fp32 accumulation and by the
# occasional fp16 rounding that this accumulation sends the other way.
def round_fp16(a) -> np.ndarray:
    """Nearest fp16 value of float64 values (ties to even), as float64.
    Magnitudes of 65520 and above become infinite, as in IEEE binary16."""
    with np.errstate(over="ignore"):
        return np.asarray(a, np.float64).astype(np.float16).astype(np.float64)


def ulp_fp16(a) -> np.ndarray:
    """Spacing of fp16 numbers at |a|: 2^(e - 10) for 2^e <= |a| < 2^(e+1)
    with e >= -14, and 2^-24 (the subnormal spacing) below 2^-14."""
    av = np.abs(np.asarray(a, np.float64))
    m, e = np.frexp(av)  # |a| = m 2^e with 0.5 <= m < 1 (frexp gives e = 0 for 0)
    e = np.where(av == 0.0, -24 + 11, e)
    return np.ldexp(1.0, np.maximum(e - 11, -24))


def expert_weights(layer: Dict[str, np.ndarray], e, emulate: Optional[str] = None
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """Dequantised (gate/up, down) weights of routed expert e, or of the shared
    expert when e == "sh"; rounded to fp16 when emulate == "fp16"."""
    if e == "sh":
        ws = (dequant(layer["sh_gu_q"], layer["sh_gu_s"], layer["sh_gu_b"]),
              dequant(layer["sh_dn_q"], layer["sh_dn_s"], layer["sh_dn_b"]))
    else:
        ws = (dequant(layer["gu_q"][e], layer["gu_s"][e], layer["gu_b"][e]),
              dequant(layer["dn_q"][e], layer["dn_s"][e], layer["dn_b"][e]))
    if emulate == "fp16":
        return round_fp16(ws[0]), round_fp16(ws[1])
    if emulate is not None:
        raise ValueError(emulate)
    return ws


def moe_forward_terms(layer: Dict[str, np.ndarray], x_bits, logits, k: int,
                      tokens: Optional[Sequence[int]] = None,
                      emulate: Optional[str] = None,
                      weight_cache: Optional[dict] = None) -> Dict[str, np.ndarray]:
    """Steps 3, 4 and 9-11 for the listed tokens (all by default), with the
    terms of the combine kept: g [n][k] (gates), o [n][k][d] (routed expert
    outputs by slot), o_sh [n][d] (shared expert output, None without one) and
    y [n][d] = sum_j g_j o_j + o_sh, the slots added in order j = 0..k-1.

    Tokens are independent, so any subset gives exactly the rows the full call
    would. Work is grouped by expert only to dequantise each expert once.
    emulate="fp16" rounds the weights, x, h and o to fp16 (diagnostic)."""
    L = np.asarray(logits, dtype=np.float32)
    T = L.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    X = bf16_value(np.asarray(x_bits)[tok])
    rnd = round_fp16 if emulate == "fp16" else (lambda v: v)
    X = rnd(X)
    ids = topk(L[tok], k)
    g = gates(L[tok], ids)
    n, d = X.shape
    cache = {} if weight_cache is None else weight_cache

    def weights(e):
        key = (e, emulate)
        if key not in cache:
            cache[key] = expert_weights(layer, e, emulate)
        return cache[key]

    def ffn(rows, e):
        gu, dn = weights(e)
        return rnd(down_proj(rnd(swiglu_h(X[rows], gu)), dn))

    o = np.zeros((n, k, d), np.float64)
    for j in range(k):
        for e in np.unique(ids[:, j]):
            rows = np.nonzero(ids[:, j] == e)[0]
            o[rows, j] = ffn(rows, int(e))
    Y = np.zeros((n, d), np.float64)
    for j in range(k):  # slot order
        Y += g[:, j][:, None] * o[:, j]
    o_sh = None
    if "sh_gu_q" in layer:  # step 10: shared expert, weight 1
        o_sh = ffn(np.arange(n), "sh")
        Y += o_sh
    return dict(y=Y, g=g, o=o, o_sh=o_sh)


def moe_forward(layer: Dict[str, np.ndarray], x_bits, logits, k: int,
                tokens: Optional[Sequence[int]] = None,
                emulate: Optional[str] = None,
                weight_cache: Optional[dict] = None) -> np.ndarray:
    """Steps 3, 4 and 9-11: y_t = sum_j g_tj * FFN_(e_tj)(x_t) + FFN_sh(x_t)
    for the listed tokens (all by default). Returns float64 [len(tokens), d]."""
    return moe_forward_terms(layer, x_bits, logits, k, tokens, emulate, weight_cache)["y"]


def moe_forward_sorted(layer: Dict[str, np.ndarray], x_bits, logits, k: int) -> np.ndarray:
    """The same layer evaluated the way the grouped form orders it: rows in
    sorted (expert-major) order through the scatter, then combined back with
    pair_pos (steps 7, 9, 11). Used to pin the routing tensors against the
    per-token form on small inputs."""
    L = np.asarray(logits, dtype=np.float32)
    T, E = L.shape
    r = route(L, k)
    X = bf16_value(x_bits)
    O = np.zeros((T * k, X.shape[1]))
    offs = r["offsets"]
    for e in range(E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi > lo:
            gu, dn = expert_weights(layer, e)
            O[lo:hi] = swiglu_ffn(X[r["sorted_token"][lo:hi]], gu, dn)
    Y = np.zeros_like(X)
    for t in range(T):
        for j in range(k):
            Y[t] += r["topk_w"][t, j] * O[r["pair_pos"][t * k + j]]
    if "sh_gu_q" in layer:
        gu, dn = expert_weights(layer, "sh")
        Y += swiglu_ffn(X, gu, dn)
    return Y


def route_chunks(logits, k: int, chunk: int) -> List[Dict[str, np.ndarray]]:
    """Bounded-chunk prefill (Lily-ES "Precarga..."; Lily-HE prefill section):
    routing tensors are produced per chunk of at most `chunk` tokens, each
    chunk routed on its own."""
    L = np.asarray(logits, dtype=np.float32)
    return [route(L[i:i + chunk], k) for i in range(0, L.shape[0], chunk)]


def error_metrics(y_test, y_ref) -> Dict[str, float]:
    """Acceptance metrics of a result against the reference:
    rel_fro = ||y_test - y_ref||_F / ||y_ref||_F and
    max_over_rms = max |y_test - y_ref| / rms(y_ref), where
    rms(y_ref) = ||y_ref||_F / sqrt(number of elements)."""
    yt = np.asarray(y_test, np.float64)
    yr = np.asarray(y_ref, np.float64)
    fro = float(np.linalg.norm(yr))
    rms = fro / math.sqrt(yr.size)
    diff = yt - yr
    return dict(rel_fro=float(np.linalg.norm(diff)) / fro,
                max_over_rms=float(np.max(np.abs(diff))) / rms,
                rms=rms)
