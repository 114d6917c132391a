"""Seeded synthetic inputs for the grouped int4-dequant MoE layer.

This module only draws random numbers and stores them in the layer's input
formats. It holds none of the layer's arithmetic (no dequantisation, routing,
GEMM or activation), so both the CPU oracle and the GPU path may consume its
output without sharing any code of the method.

Storage formats produced here:
  * bf16 values as uint16 bit patterns, rounded from float32 by
    round-to-nearest-even;
  * fp32 router logits;
  * 4-bit weight codes packed eight to a uint32 word, low nibble first. Eight
    independent uniform codes in 0..15 packed this way form exactly one uniform
    32-bit word, so the packed words are drawn directly.

Shapes follow the Qwen3.6-35B-A3B mixture-of-experts layer the Lily pages
describe (Lily-EN "Three Workload Shapes": 256 routed experts, 8 picked per
token, one shared expert seeing every token; Lily-ES "Precarga: mantenga los
pesos empaquetados, siga enrutando en la GPU": 4-bit codes in groups of 64 that
share one bf16 scale and one bf16 bias). The pages give no hidden or expert
sizes; d=2048 and f=512 are assumed.

Pages cited (titles as published):
  Lily-EN  "Perplexity Open Sources Lily: A Rust + Metal Inference Engine for
           Qwen3.6-35B-A3B on Apple Silicon" (insight.aitobox.com)
  Lily-ES  "Perplexity open sources Lily: un motor de inferencia ... para
           Qwen3.6-35B-A3B en Apple Silicon" (7minutos.es)

Generation order for one layer (one numpy Generator per layer): for each routed
expert 0..E-1, then the shared expert: gate/up codes, scales, biases, then down
codes, scales, biases. Token inputs follow the weights: logits, then x.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Iterator, Optional

import numpy as np

GROUP = 64  # weights per quantisation group (one bf16 scale + one bf16 bias)


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact). Used only to derive the bias
    draw from the already rounded scale, as the recipe states."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


@dataclasses.dataclass(frozen=True)
class LayerShape:
    d: int        # hidden size (K of gate/up, N of down)
    f: int        # routed expert intermediate size
    E: int        # routed experts
    k: int        # experts picked per token
    f_sh: int     # shared expert intermediate size (0: no shared expert)


@dataclasses.dataclass(frozen=True)
class Config:
    index: int
    name: str
    T: int
    shape: LayerShape
    seed: int
    logits: str = "normal"      # "normal" or "zipf"
    chunk: Optional[int] = None  # bounded-chunk size for long prompts
    steps: int = 1               # decode steps (fresh logits and x per step)


_QWEN = LayerShape(d=2048, f=512, E=256, k=8, f_sh=512)

CONFIGS: Dict[int, Config] = {
    0: Config(0, "tiny", 64, LayerShape(d=256, f=128, E=16, k=2, f_sh=128), seed=0),
    1: Config(1, "prefill512", 512, _QWEN, seed=1),
    2: Config(2, "prefill2048", 2048, _QWEN, seed=2),
    3: Config(3, "skew8192", 8192, _QWEN, seed=3, logits="zipf", chunk=2048),
    4: Config(4, "decode", 1, _QWEN, seed=4, steps=1000),
}


def _draw_matrix(rng: np.random.Generator, n: int, kdim: int):
    """One quantised [n, kdim] matrix: packed codes, scales, biases."""
    assert kdim % GROUP == 0
    q = rng.integers(0, 2 ** 32, size=(n, kdim // 8), dtype=np.uint32)
    s_f32 = rng.uniform(0.005, 0.02, size=(n, kdim // GROUP)).astype(np.float32)
    s = f32_to_bf16_bits(s_f32)
    s_val = bf16_bits_to_f32(s).astype(np.float64)
    b_f64 = -8.0 * s_val * (1.0 + rng.uniform(-0.1, 0.1, size=s.shape))
    b = f32_to_bf16_bits(b_f64.astype(np.float32))
    return q, s, b


def make_layer(shape: LayerShape, rng: np.random.Generator) -> Dict[str, np.ndarray]:
    """All weights of one layer, row-major, in the library's layout:
    gu_* [E][2f][...] (rows 0..f-1 gate, f..2f-1 up), dn_* [E][d][...],
    sh_gu_* [2f_sh][...], sh_dn_* [d][...]."""
    d, f, E = shape.d, shape.f, shape.E
    gu_q = np.empty((E, 2 * f, d // 8), np.uint32)
    gu_s = np.empty((E, 2 * f, d // GROUP), np.uint16)
    gu_b = np.empty_like(gu_s)
    dn_q = np.empty((E, d, f // 8), np.uint32)
    dn_s = np.empty((E, d, f // GROUP), np.uint16)
    dn_b = np.empty_like(dn_s)
    for e in range(E):
        gu_q[e], gu_s[e], gu_b[e] = _draw_matrix(rng, 2 * f, d)
        dn_q[e], dn_s[e], dn_b[e] = _draw_matrix(rng, d, f)
    layer = dict(gu_q=gu_q, gu_s=gu_s, gu_b=gu_b, dn_q=dn_q, dn_s=dn_s, dn_b=dn_b)
    if shape.f_sh > 0:
        layer["sh_gu_q"], layer["sh_gu_s"], layer["sh_gu_b"] = _draw_matrix(rng, 2 * shape.f_sh, d)
        layer["sh_dn_q"], layer["sh_dn_s"], layer["sh_dn_b"] = _draw_matrix(rng, d, shape.f_sh)
    return layer


def zipf_expert_bias(E: int, rng: np.random.Generator, s: float = 1.1, amp: float = 1.5) -> np.ndarray:
    """Per-expert logit offset giving Zipf-skewed loads: expert e gets rank
    r_e = 1 + perm(e) and offset amp * ln(r_e^-s / sum_i i^-s)."""
    perm = rng.permutation(E)
    ranks = 1.0 + perm.astype(np.float64)
    norm = sum(i ** -s for i in range(1, E + 1))
    return amp * np.log(ranks ** -s / norm)


def draw_tokens(T: int, shape: LayerShape, rng: np.random.Generator,
                expert_bias: Optional[np.ndarray] = None):
    """Router logits fp32 [T][E] (N(0,1) plus an optional per-expert offset,
    summed in float64 then rounded once), then x bf16 bits [T][d] (N(0,1))."""
    lg = rng.standard_normal((T, shape.E))
    if expert_bias is not None:
        lg = lg + expert_bias[None, :]
    logits = lg.astype(np.float32)
    x = f32_to_bf16_bits(rng.standard_normal((T, shape.d)).astype(np.float32))
    return logits, x


def draw_router(E: int, d: int, rng: np.random.Generator) -> np.ndarray:
    """Router weights bf16 bits [E][d], N(0, 1/d): with x ~ N(0,1) the logits
    come out about N(0,1), the distribution the layer workloads draw directly."""
    return f32_to_bf16_bits((rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32))


def make_router_problem(T: int, d: int, E: int, seed: int):
    """Seeded router-projection inputs: x bf16 bits [T][d] (N(0,1)), then W_r
    bf16 bits [E][d]."""
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    return x, draw_router(E, d, rng)


@dataclasses.dataclass
class Problem:
    config: Config
    T: int
    shape: LayerShape
    layer: Dict[str, np.ndarray]
    logits: np.ndarray  # fp32 [T][E]
    x: np.ndarray       # uint16 bf16 bits [T][d]


def make_problem(index: int, T: Optional[int] = None) -> Problem:
    """Inputs of one of the five configurations (seed = config index). For the
    decode configuration this returns step 0; use decode_steps for the rest.
    T overrides the token count (decode: 1 or 4)."""
    cfg = CONFIGS[index]
    rng = np.random.default_rng(cfg.seed)
    layer = make_layer(cfg.shape, rng)
    T = cfg.T if T is None else T
    bias = zipf_expert_bias(cfg.shape.E, rng) if cfg.logits == "zipf" else None
    logits, x = draw_tokens(T, cfg.shape, rng, bias)
    return Problem(cfg, T, cfg.shape, layer, logits, x)


def decode_steps(T: int, steps: Optional[int] = None, index: int = 4) -> Iterator[Problem]:
    """Decode stream: the layer's weights once, then per step fresh logits and
    x of T tokens, all from one Generator seeded with the config's seed."""
    cfg = CONFIGS[index]
    rng = np.random.default_rng(cfg.seed)
    layer = make_layer(cfg.shape, rng)
    for _ in range(cfg.steps if steps is None else steps):
        logits, x = draw_tokens(T, cfg.shape, rng)
        yield Problem(cfg, T, cfg.shape, layer, logits, x)


def make_custom(T: int, shape: LayerShape, seed: int,
                expert_bias: Optional[np.ndarray] = None) -> Problem:
    """Inputs of an arbitrary shape with the same value distributions."""
    rng = np.random.default_rng(seed)
    layer = make_layer(shape, rng)
    logits, x = draw_tokens(T, shape, rng, expert_bias)
    cfg = Config(-1, "custom", T, shape, seed)
    return Problem(cfg, T, shape, layer, logits, x)


def bytes_per_expert(shape: LayerShape, f: Optional[int] = None) -> int:
    """Packed codes + scales + biases of one expert (gate/up and down)."""
    f = shape.f if f is None else f
    n_w = 3 * shape.d * f
    return n_w // 2 + 2 * 2 * (n_w // GROUP)


def useful_flops_per_token(shape: LayerShape) -> int:
    """2 * (k routed + shared) * 3 * d * f multiply-adds counted as 2 flops."""
    return 2 * 3 * shape.d * (shape.k * shape.f + shape.f_sh)


assert bytes_per_expert(_QWEN) == 1_769_472
assert math.isclose(useful_flops_per_token(_QWEN) * 2048 / 1e9, 115.96, rel_tol=1e-3)
