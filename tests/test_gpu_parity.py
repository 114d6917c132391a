"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Routing tensors must match bit for bit; router weights within 1e-6; layer
outputs within relative Frobenius error 5e-3 and max abs error 2e-2 * rms of
the oracle output, every row (the full-size configurations and the
fp16-emulation and stage checks are in test_gpu_emulation.py)."""
import sys

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import moe_inputs as S

pytestmark = pytest.mark.gpu

REL_FRO = 5e-3
MAX_OVER_RMS = 2e-2
ROUTE_KEYS = ("topk_ids", "counts", "offsets", "sorted_pair", "sorted_token", "pair_pos",
              "block_map", "num_blocks")


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


def upload(p: S.Problem, moe):
    sh = p.shape
    layer = moe.Layer.from_numpy(sh.d, sh.f, sh.E, sh.k, sh.f_sh, p.layer)
    x = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).cuda()
    lg = torch.from_numpy(p.logits).cuda()
    return layer, x, lg


def check_routing(got, ref, T, k):
    for key in ROUTE_KEYS:
        g = got[key].cpu().numpy().reshape(-1)
        r = np.asarray(ref[key]).reshape(-1)
        assert np.array_equal(g, r), f"routing tensor {key} differs (T={T}, k={k})"
    w = got["topk_w"].cpu().numpy().astype(np.float64)
    assert np.max(np.abs(w - ref["topk_w"])) <= 1e-6


def check_output(y_gpu, y_ref, what=""):
    m = O.error_metrics(y_gpu, y_ref)
    say(f"  {what}: rel_fro={m['rel_fro']:.3e} max/rms={m['max_over_rms']:.3e}")
    assert m["rel_fro"] <= REL_FRO, (what, m)
    assert m["max_over_rms"] <= MAX_OVER_RMS, (what, m)
    return m


def run_layer(moe, p, with_routing=True):
    layer, x, lg = upload(p, moe)
    routing = moe.alloc_routing(p.T, p.shape.E, p.shape.k) if with_routing else None
    y = moe.layer_forward(layer, x, lg, routing=routing)
    torch.cuda.synchronize()
    return y.cpu().numpy(), routing


# ------------------------------------------------------------------ routing
def test_route_config0(moe):
    p = S.make_problem(0)
    say("route config 0")
    got = moe.route(torch.from_numpy(p.logits).cuda(), p.shape.k)
    torch.cuda.synchronize()
    check_routing(got, O.route(p.logits, p.shape.k), p.T, p.shape.k)


def _adversarial_cases():
    rng = np.random.default_rng(123)
    cases = []
    # exact ties including +-0.0
    L = rng.choice(np.array([-0.0, 0.0, 1.0, -1.0], np.float32), size=(100, 8))
    cases.append(("ties", L, 3))
    # ties at the k-th pick among many lanes and all four 64-expert rows of a
    # wave: half-step logits, whole rows of +-0.0, and k from 1 to 16
    L = np.round(rng.standard_normal((96, 256)).astype(np.float32) * 2.0) / 2.0
    L[::7] = 0.0
    L[::7, 1::3] = -0.0
    for kk in (1, 8, 13, 16):
        cases.append((f"ties_E256_k{kk}", L, kk))
    L = np.round(rng.standard_normal((64, 1024)).astype(np.float32) * 4.0) / 4.0
    cases.append(("ties_E1024", L, 8))
    # every logit equal: the k lowest expert indices
    cases.append(("all_equal", np.full((10, 200), 0.25, np.float32), 11))
    # all tokens on the same experts
    L = rng.standard_normal((130, 16)).astype(np.float32)
    L[:, :4] += 100.0
    cases.append(("same_experts", L, 4))
    # counts 31, 32, 33, 64 on experts 0..3 with k = 1 (others empty)
    L = np.full((160, 6), -5.0, np.float32)
    rows = np.repeat(np.arange(4), [31, 32, 33, 64])
    L[np.arange(160), rows] = 5.0
    cases.append(("edge_counts", L, 1))
    # k = E
    cases.append(("k_eq_E", rng.standard_normal((77, 8)).astype(np.float32), 8))
    # one token, large E
    cases.append(("one_token", rng.standard_normal((1, 1024)).astype(np.float32), 8))
    # ragged T, E = 256
    cases.append(("ragged", rng.standard_normal((1000, 256)).astype(np.float32), 8))
    # E not a multiple of 64
    cases.append(("E_odd", rng.standard_normal((300, 67)).astype(np.float32), 5))
    # 32768 pairs: the largest call whose scatter workgroups count every pair
    # themselves; one token more takes the per-sub-chunk count pass
    cases.append(("pairs_32768", rng.standard_normal((4096, 256)).astype(np.float32), 8))
    cases.append(("pairs_32776", rng.standard_normal((4097, 256)).astype(np.float32), 8))
    cases.append(("pairs_49152_T16384", rng.standard_normal((16384, 64)).astype(np.float32), 3))
    return cases


@pytest.mark.parametrize("name,L,k", _adversarial_cases(), ids=[c[0] for c in _adversarial_cases()])
def test_route_adversarial(moe, name, L, k):
    say(f"route adversarial {name} T={L.shape[0]} E={L.shape[1]} k={k}")
    got = moe.route(torch.from_numpy(L).cuda(), k)
    torch.cuda.synchronize()
    check_routing(got, O.route(L, k), L.shape[0], k)


def test_route_deterministic(moe):
    p = S.make_problem(2)
    say("route determinism T=2048 x10")
    lg = torch.from_numpy(p.logits).cuda()
    first = {k_: v.clone() for k_, v in moe.route(lg, 8).items()}
    for _ in range(10):
        again = moe.route(lg, 8)
        for key in first:
            assert torch.equal(first[key], again[key]), key


# ----------------------------------------------------------- grouped GEMM
@pytest.mark.parametrize("N,K,E,k,T", [(128, 256, 5, 2, 100), (192, 320, 3, 1, 70), (256, 2048, 4, 2, 40)])
def test_grouped_gemm_matches_oracle(moe, N, K, E, k, T):
    say(f"grouped gemm N={N} K={K} E={E} k={k} T={T}")
    rng = np.random.default_rng(N + K)
    Wq = rng.integers(0, 2 ** 32, size=(E, N, K // 8), dtype=np.uint32)
    Ws = S.f32_to_bf16_bits(rng.uniform(0.005, 0.02, (E, N, K // 64)).astype(np.float32))
    Wb = S.f32_to_bf16_bits((-8 * O.bf16_value(Ws) * (1 + rng.uniform(-0.1, 0.1, Ws.shape))).astype(np.float32))
    A = S.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    L = rng.standard_normal((T, E)).astype(np.float32)
    ref_r = O.route(L, k)
    r = moe.route(torch.from_numpy(L).cuda(), k)
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).cuda()
    C = torch.full((T * k, N), float("nan"), dtype=torch.float32, device="cuda")
    moe.grouped_gemm_int4(dev(A, np.int16).view(torch.bfloat16), r["sorted_token"], N, K,
                          dev(Wq, np.int32), dev(Ws, np.int16).view(torch.bfloat16),
                          dev(Wb, np.int16).view(torch.bfloat16), r["block_map"], r["num_blocks"], C)
    torch.cuda.synchronize()
    Cg = C.cpu().numpy()
    X = O.bf16_value(A)
    ref = np.zeros((T * k, N))
    for e in range(E):
        lo, hi = ref_r["offsets"][e], ref_r["offsets"][e + 1]
        W = O.dequant(Wq[e], Ws[e], Wb[e])
        ref[lo:hi] = X[ref_r["sorted_token"][lo:hi]] @ W.T
    check_output(Cg, ref, "grouped gemm")


def test_grouped_gemm_long_and_empty_blocks(moe):
    """Outside the block map contract (1..32 rows per block): of a block
    longer than the 96-row work unit only the first 96 rows are computed,
    and empty or negative blocks write nothing; every other row keeps its
    old contents."""
    N, K, E = 256, 512, 3
    say("grouped gemm with blocks of 200, 97, 96, 1, 0 and -5 rows")
    rng = np.random.default_rng(11)
    Wq = rng.integers(0, 2 ** 32, size=(E, N, K // 8), dtype=np.uint32)
    Ws = S.f32_to_bf16_bits(rng.uniform(0.005, 0.02, (E, N, K // 64)).astype(np.float32))
    Wb = S.f32_to_bf16_bits((-8 * O.bf16_value(Ws) * (1 + rng.uniform(-0.1, 0.1, Ws.shape))).astype(np.float32))
    rows = 420
    A = S.f32_to_bf16_bits(rng.standard_normal((rows, K)).astype(np.float32))
    a_row = rng.permutation(rows).astype(np.int32)
    # (expert, first row, rows); rows 394..399 are in no block
    blocks = np.array([[0, 0, 200], [2, 200, 97], [1, 297, 96], [2, 393, 1], [1, 400, 0], [0, 400, -5],
                       [1, 400, 20]], np.int32)
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).cuda()
    C = torch.full((rows, N), float("nan"), dtype=torch.float32, device="cuda")
    moe.grouped_gemm_int4(dev(A, np.int16).view(torch.bfloat16), dev(a_row, np.int32), N, K,
                          dev(Wq, np.int32), dev(Ws, np.int16).view(torch.bfloat16),
                          dev(Wb, np.int16).view(torch.bfloat16), dev(blocks, np.int32),
                          dev(np.array([len(blocks)], np.int32), np.int32), C)
    torch.cuda.synchronize()
    Cg = C.cpu().numpy()
    X = O.bf16_value(A)
    covered = np.zeros(rows, bool)
    for e, r0, n in blocks:
        n = min(n, 96)
        if n <= 0:
            continue
        W = O.dequant(Wq[e], Ws[e], Wb[e])
        ref = X[a_row[r0:r0 + n]] @ W.T
        check_output(Cg[r0:r0 + n], ref, f"block ({e}, {r0}, {n})")
        covered[r0:r0 + n] = True
    assert np.isnan(Cg[~covered]).all()


# ------------------------------------------------------------------ layer
def test_layer_config0(moe):
    p = S.make_problem(0)
    say("layer config 0 (T=64 d=256 f=128 E=16 k=2)")
    y, routing = run_layer(moe, p)
    check_routing(routing, O.route(p.logits, p.shape.k), p.T, p.shape.k)
    check_output(y, O.moe_forward(p.layer, p.x, p.logits, p.shape.k), "config 0")


EDGE_SHAPES = [
    # T, d, f, E, k, f_sh
    (1, 256, 128, 16, 2, 128),
    (65, 64, 64, 3, 1, 0),
    (129, 320, 192, 8, 8, 64),
    (200, 128, 64, 1, 1, 0),
    (33, 2048, 512, 256, 8, 512),
    (300, 512, 320, 12, 3, 192),
    (50, 2560, 192, 4, 2, 64),      # K = 2560: scale/bias table refilled every 1024 inputs, last chunk partial
    (40, 448, 576, 5, 2, 0),        # 7 groups along d: scalar table fill
    (50, 1024, 192, 4, 2, 0),       # 4 units (not a multiple of 8), all half-width: down in eight 128-column slices
    (50, 768, 192, 4, 2, 64),       # all units half-width; down in six 128-column slices over d = 768
    (256, 1024, 256, 64, 4, 256),   # 64 units: 32 full-width + 32 half-width (128-column) units
    # persistent streaming GEMM (K a multiple of 512, at most 2048)
    (40, 512, 512, 8, 2, 512),      # four steps per item, shared rows after routed rows
    (250, 1024, 512, 3, 2, 0),      # experts split into several units, no shared expert
    (130, 1536, 1024, 6, 2, 1024),  # 12 and 8 steps per item, partial last slice of d
    (97, 512, 512, 1, 1, 512),      # one expert over 97 rows: two units
    (192, 512, 512, 2, 1, 512),     # two full 96-row units per expert (six row blocks)
    (60, 512, 512, 4, 2, 1024),     # shared width differs from f: general kernel
]


@pytest.mark.parametrize("T,d,f,E,k,f_sh", EDGE_SHAPES)
def test_layer_edge_shapes(moe, T, d, f, E, k, f_sh):
    say(f"layer edge T={T} d={d} f={f} E={E} k={k} f_sh={f_sh}")
    p = S.make_custom(T, S.LayerShape(d=d, f=f, E=E, k=k, f_sh=f_sh), seed=T + d + f)
    y, routing = run_layer(moe, p)
    check_routing(routing, O.route(p.logits, k), T, k)
    check_output(y, O.moe_forward(p.layer, p.x, p.logits, k), f"edge {T},{d},{f},{E},{k},{f_sh}")


def test_layer_all_tokens_one_expert_set_streaming(moe):
    """All tokens on the same two experts, at a shape the streaming GEMM takes."""
    shape = S.LayerShape(d=512, f=512, E=16, k=2, f_sh=512)
    p = S.make_custom(300, shape, seed=6)
    p.logits[:, :2] += 100.0
    say("all tokens -> experts {0,1}, streaming shape")
    y, routing = run_layer(moe, p)
    check_routing(routing, O.route(p.logits, 2), 300, 2)
    check_output(y, O.moe_forward(p.layer, p.x, p.logits, 2), "one expert set (streaming)")


def test_layer_all_tokens_one_expert_set(moe):
    """Every token routed to the same k experts: each expert group is a dense GEMM."""
    shape = S.LayerShape(d=256, f=128, E=16, k=2, f_sh=128)
    p = S.make_custom(300, shape, seed=5)
    p.logits[:, 3] += 100.0
    p.logits[:, 11] += 100.0
    say("layer all tokens on experts 3 and 11")
    y, routing = run_layer(moe, p)
    check_routing(routing, O.route(p.logits, 2), 300, 2)
    check_output(y, O.moe_forward(p.layer, p.x, p.logits, 2), "dense special case")


@pytest.mark.timeout(300)
def test_layer_max_call_tokens(moe):
    """One moe_layer_forward call at the per-call maximum, T = 16384 tokens of
    the Qwen-shaped layer (131072 pairs: the count pass, work lists of
    thousands of units): routing bit-exact, and every 256th output row
    against the oracle (each token's output depends only on its own row)."""
    T = 16384  # MOE_MAX_CALL_TOKENS in include/moe_int4.h
    shape = S.LayerShape(d=2048, f=512, E=256, k=8, f_sh=512)
    p = S.make_custom(T, shape, seed=16384)
    say(f"layer at the call maximum T={T}")
    y, routing = run_layer(moe, p)
    check_routing(routing, O.route(p.logits, shape.k), T, shape.k)
    rows = np.arange(0, T, 256)
    check_output(y[rows], O.moe_forward(p.layer, p.x[rows], p.logits[rows], shape.k), f"T={T}, {len(rows)} rows")


@pytest.mark.parametrize("index", [1, 2])
def test_layer_bit_reproducible(moe, index):
    """Repeated calls on the same inputs give the same y bit for bit (every
    reduction has a fixed order; no atomics), whatever else ran between them."""
    p = S.make_problem(index)
    say(f"layer determinism config {index} T={p.T} x12")
    layer, x, lg = upload(p, moe)
    ws = moe.alloc_workspace(moe.workspace_bytes(p.T, layer))
    first = moe.layer_forward(layer, x, lg, ws=ws).clone()
    for r in range(12):
        y = torch.empty_like(first)
        for _ in range(1 + (7 * r) % 5):
            moe.layer_forward(layer, x, lg, y=y, ws=ws)
        torch.cuda.synchronize()
        diff = (y != first).sum().item()
        assert diff == 0, f"repeat {r}: {diff} output elements differ"


@pytest.mark.parametrize("keep", [(0, 1, 2, 3, 4), (2, 3), ()], ids=["all", "gate_up", "none"])
@pytest.mark.parametrize("index", [0, 1])
def test_layer_forward_timed_matches_plain(moe, index, keep):
    """moe_layer_forward_timed computes what moe_layer_forward computes, bit
    for bit, with all five events, with only the gate/up pair (the
    benchmark's timed calls) or with every entry null; each recorded pair
    spans a positive time."""
    import ctypes
    import bench
    from grouped_int4_dequant_amd import binding as B
    p = S.make_problem(index)
    say(f"timed forward config {index} T={p.T} events {keep}")
    layer, x, lg = upload(p, moe)
    ws = moe.alloc_workspace(moe.workspace_bytes(p.T, layer))
    ref = moe.layer_forward(layer, x, lg, ws=ws).clone()
    lib = B.load()
    lib.moe_layer_forward_timed.argtypes = [ctypes.POINTER(B.MoeLayerT), B._P, B._P, B._I32, B._P, B._P, B._P,
                                            ctypes.c_size_t, B._P, ctypes.POINTER(B._P)]
    lib.moe_layer_forward_timed.restype = ctypes.c_int
    hip = bench.hip_runtime()
    evs = [bench.HipEvent(hip) for _ in range(5)]
    arr = (B._P * 5)(*[evs[i].handle if i in keep else None for i in range(5)])
    y = torch.empty_like(ref)
    st = lib.moe_layer_forward_timed(ctypes.byref(layer.c), x.data_ptr(), lg.data_ptr(), p.T, y.data_ptr(), None,
                                     ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream, arr)
    assert st == 0, moe.status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    for i in range(4):
        if i in keep and i + 1 in keep:
            assert evs[i].elapsed_time(evs[i + 1]) > 0.0, (i, keep)


@pytest.mark.parametrize("T", [1, 4])
def test_decode_config4(moe, T):
    """Config 4's parity schedule: routing checked on every one of the 1000
    seeded steps, outputs on steps 0, 999 and every 20th step."""
    nsteps = S.CONFIGS[4].steps
    say(f"config 4 decode T={T}: {nsteps} steps")
    cache = {}
    layer = None
    ys, refs = [], []
    for step, p in enumerate(S.decode_steps(T)):
        if step % 200 == 0:
            say(f"  step {step}")
        if layer is None:
            layer, _, _ = upload(p, moe)
        x = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).cuda()
        lg = torch.from_numpy(p.logits).cuda()
        routing = moe.alloc_routing(T, p.shape.E, p.shape.k)
        y = moe.layer_forward(layer, x, lg, routing=routing)
        torch.cuda.synchronize()
        check_routing(routing, O.route(p.logits, p.shape.k), T, p.shape.k)
        if step % 20 == 0 or step == nsteps - 1:
            ys.append(y.cpu().numpy())
            refs.append(O.moe_forward(p.layer, p.x, p.logits, p.shape.k, weight_cache=cache))
    check_output(np.concatenate(ys), np.concatenate(refs), f"decode T={T}")


DECODE_SHAPES = [
    # T, E, k, f_sh  (d = 2048, f = 512: the two-kernel decode path)
    (2, 256, 8, 512),
    (3, 64, 4, 0),       # no shared expert, one key per lane
    (8, 1024, 8, 512),   # 16 keys per lane, eight tokens
    (5, 256, 1, 512),    # k = 1: gate 1
    (8, 16, 8, 0),       # 64 picks over 16 experts: every expert shared by several tokens
]


@pytest.mark.parametrize("T,E,k,f_sh", DECODE_SHAPES)
@pytest.mark.parametrize("with_routing", [False, True])
def test_decode_shapes(moe, T, E, k, f_sh, with_routing):
    p = S.make_custom(T, S.LayerShape(d=2048, f=512, E=E, k=k, f_sh=f_sh), seed=100 + T + E + k)
    say(f"decode T={T} E={E} k={k} f_sh={f_sh} routing={'yes' if with_routing else 'no'}")
    y, routing = run_layer(moe, p, with_routing=with_routing)
    if with_routing:
        check_routing(routing, O.route(p.logits, k), T, k)
    check_output(y, O.moe_forward(p.layer, p.x, p.logits, k), f"decode T={T} E={E} k={k}")


@pytest.mark.parametrize("T,d,E,k", [(1, 1024, 256, 8), (4, 1024, 64, 8), (1, 4096, 128, 4), (3, 4096, 256, 8)])
def test_decode_other_widths(moe, T, d, E, k):
    """Decode at d = 1024 and 4096 (two and eight gate/up waves, so the
    partial sums take the general reduction loop; k = 4 also in the down
    kernel's combine)."""
    p = S.make_custom(T, S.LayerShape(d=d, f=512, E=E, k=k, f_sh=512), seed=200 + T + d + E + k)
    say(f"decode T={T} d={d} E={E} k={k}")
    y, routing = run_layer(moe, p, with_routing=True)
    check_routing(routing, O.route(p.logits, k), T, k)
    check_output(y, O.moe_forward(p.layer, p.x, p.logits, k), f"decode T={T} d={d} E={E} k={k}")


@pytest.mark.parametrize("T,zero_row", [(4, 1), (1, None), (1, 0)])
def test_decode_tied_logits(moe, T, zero_row):
    """Exact ties (and -0.0 against +0.0) decide which experts the decode
    kernels' own top-k picks; a wrong tie rule changes y by a whole expert."""
    p = S.make_custom(T, S.LayerShape(d=2048, f=512, E=256, k=8, f_sh=512), seed=77)
    p.logits[:] = np.round(p.logits * 2.0) / 2.0
    if zero_row is not None:
        p.logits[zero_row, :] = 0.0
        p.logits[zero_row, 1::3] = -0.0
    say(f"decode tied logits T={T} zero row {zero_row}")
    y, _ = run_layer(moe, p, with_routing=False)
    check_output(y, O.moe_forward(p.layer, p.x, p.logits, 8), "decode ties")


# ------------------------------------------------------------------ router
def _router_bound(x_bits, w_bits):
    """Error bound of an fp32 sum of d exact products in any order:
    (d - 1) * 2^-24 * sum_k |x_k w_k| per logit (the bf16 products are exact
    in fp32)."""
    d = x_bits.shape[1]
    return (d - 1) * 2.0 ** -24 * (np.abs(O.bf16_value(x_bits)) @ np.abs(O.bf16_value(w_bits)).T)


@pytest.mark.parametrize("T,d,E", [(2048, 2048, 256), (37, 96, 20), (1, 32, 1), (130, 512, 1024), (45, 2080, 70),
                                   (1, 2048, 256), (16, 2048, 256), (17, 2048, 256), (9, 96, 20), (3, 2080, 1000)])
def test_router_logits_match_oracle(moe, T, d, E):
    say(f"router T={T} d={d} E={E}")
    x, w = S.make_router_problem(T, d, E, seed=T + d + E)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    lg = moe.router_logits(xt, wt)
    lg2 = moe.router_logits(xt, wt)
    torch.cuda.synchronize()
    got = lg.cpu().numpy().astype(np.float64)
    ref = O.router_logits(x, w)
    assert np.array_equal(got, lg2.cpu().numpy()), "router logits differ between calls"
    err = np.abs(got - ref)
    bound = _router_bound(x, w)
    say(f"  max err {err.max():.3e}, max err/bound {np.max(err / np.maximum(bound, 1e-30)):.3f}")
    assert np.all(err <= bound)


def test_router_then_route_matches_oracle_routing(moe):
    """Logits from the router kernel feed the routing kernels; the picks agree
    with the oracle's top-k of the exact logits wherever the k-th and
    (k+1)-th exact logits are further apart than the error bound, and are
    valid picks (within the bound of the k-th) everywhere."""
    T, d, E, k = 2048, 2048, 256, 8
    x, w = S.make_router_problem(T, d, E, seed=5)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    got = moe.route(moe.router_logits(xt, wt), k)
    torch.cuda.synchronize()
    ref = O.router_logits(x, w)
    bound = _router_bound(x, w)
    ids = got["topk_ids"].cpu().numpy()
    ref_sorted = -np.sort(-ref, axis=1)
    clear = (ref_sorted[:, k - 1] - ref_sorted[:, k]) > 2 * bound.max(axis=1)
    ref_ids = O.topk(ref.astype(np.float32), k)
    for t in range(T):
        if clear[t]:
            assert set(ids[t]) == set(ref_ids[t]), t
        picked = ref[t, ids[t]]
        assert np.all(picked >= ref_sorted[t, k - 1] - 2 * bound[t].max()), t
    say(f"  {int(clear.sum())} of {T} tokens with a clear k-th pick")


# ------------------------------------------------------------------ ablations
ABLATION_SHAPES = [
    # T, d, f, E, k, f_sh
    (64, 256, 128, 16, 2, 128),
    (1, 256, 128, 16, 2, 128),      # one token through the prefill form
    (129, 320, 192, 8, 8, 64),
    (256, 1024, 256, 64, 4, 256),
    (250, 1024, 512, 3, 2, 0),      # streaming GEMM, experts over several units
    (130, 1536, 1024, 6, 2, 1024),
]


@pytest.mark.parametrize("variant", ["tile16", "host_routing", "unfused"])
@pytest.mark.parametrize("T,d,f,E,k,f_sh", ABLATION_SHAPES)
def test_ablation_matches_oracle(moe, variant, T, d, f, E, k, f_sh):
    """The ablation forms (16-row work units; routing built on the host;
    weights expanded in memory before the GEMMs) compute the same layer:
    routing exact, outputs within the tolerance of the oracle and equal bit
    for bit to the default prefill form (same weights, same accumulation
    order, fixed combine order)."""
    p = S.make_custom(T, S.LayerShape(d=d, f=f, E=E, k=k, f_sh=f_sh), seed=T + d + f + E)
    say(f"ablation {variant} T={T} d={d} f={f} E={E} k={k} f_sh={f_sh}")
    layer, x, lg = upload(p, moe)
    routing = moe.alloc_routing(T, E, k)
    y = moe.layer_forward_ablation(layer, x, lg, variant, routing=routing)
    y_def = moe.layer_forward_ablation(layer, x, lg, "none")
    torch.cuda.synchronize()
    check_routing(routing, O.route(p.logits, k), T, k)
    y = y.cpu().numpy()
    check_output(y, O.moe_forward(p.layer, p.x, p.logits, k), f"{variant} {T},{d},{f},{E},{k},{f_sh}")
    assert np.array_equal(y, y_def.cpu().numpy()), f"{variant} differs from the default prefill form"


@pytest.mark.parametrize("variant", ["tile16", "host_routing", "unfused"])
def test_ablation_full_config(moe, variant):
    p = S.make_problem(1)
    say(f"ablation {variant} config 1 T={p.T} (every row)")
    layer, x, lg = upload(p, moe)
    routing = moe.alloc_routing(p.T, p.shape.E, p.shape.k)
    y = moe.layer_forward_ablation(layer, x, lg, variant, routing=routing)
    # the default form at T=512 runs the small-unit GEMM build (32-row units);
    # every ablation form runs the 96-row build: equal bit for bit
    y_def = moe.layer_forward(layer, x, lg)
    torch.cuda.synchronize()
    check_routing(routing, O.route(p.logits, p.shape.k), p.T, p.shape.k)
    check_output(y.cpu().numpy(), O.moe_forward(p.layer, p.x, p.logits, p.shape.k), f"{variant} config 1")
    assert np.array_equal(y.cpu().numpy(), y_def.cpu().numpy()), f"{variant} differs from the default form"


def test_zero_tokens_is_a_noop(moe):
    p = S.make_problem(0)
    layer, x, lg = upload(p, moe)
    y = torch.full((0, p.shape.d), 1.0, device="cuda")
    moe.layer_forward(layer, x[:0], lg[:0], y=y)
    torch.cuda.synchronize()


# ------------------------------------------------------ router fused with top-k
@pytest.mark.parametrize("T,d,E,k", [(2048, 2048, 256, 8), (37, 96, 20, 3), (1, 64, 256, 8), (130, 512, 128, 8),
                                     (64, 256, 16, 16), (70, 512, 300, 8), (45, 2080, 70, 4),
                                     (16, 2048, 256, 8), (5, 2080, 1000, 13)])
def test_router_topk_matches_own_logits(moe, T, d, E, k):
    """moe_router_topk: its logits equal moe_router_logits' bit for bit, its
    picks equal the oracle's top-k of those same fp32 logits bit for bit, its
    gates the oracle's gates of them within 1e-6."""
    say(f"router+topk T={T} d={d} E={E} k={k}")
    x, w = S.make_router_problem(T, d, E, seed=T + d + E + k)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids, g = moe.router_topk(xt, wt, k, logits=lg)
    ref_lg = moe.router_logits(xt, wt)
    torch.cuda.synchronize()
    L = lg.cpu().numpy()
    assert np.array_equal(L, ref_lg.cpu().numpy()), "fused logits differ from moe_router_logits"
    ref_ids = O.topk(L, k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.max(np.abs(g.cpu().numpy().astype(np.float64) - O.gates(L, ref_ids))) <= 1e-6
    err = np.abs(L.astype(np.float64) - O.router_logits(x, w))
    assert np.all(err <= _router_bound(x, w))


@pytest.mark.parametrize("T,E", [(2048, 256), (300, 64), (4, 256), (1, 256), (100, 300)])
def test_layer_forward_router_equals_logits_path(moe, T, E):
    """moe_layer_forward_router equals moe_layer_forward fed with
    moe_router_logits' output, bit for bit, routing tensors included (prefill
    and few-token forms); and it is within tolerance of the oracle on the
    router's logits."""
    shape = S.LayerShape(d=2048, f=512, E=E, k=8, f_sh=512)
    p = S.make_custom(T, shape, seed=40 + T + E)
    _, w = S.make_router_problem(1, 2048, E, seed=7 + E)
    say(f"layer from router weights T={T} E={E}")
    layer, x, _ = upload(p, moe)
    wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    r1 = moe.alloc_routing(T, E, 8)
    r2 = moe.alloc_routing(T, E, 8)
    y1 = moe.layer_forward_router(layer, x, wt, routing=r1)
    lg = moe.router_logits(x, wt)
    y2 = moe.layer_forward(layer, x, lg, routing=r2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), "layer from router weights differs from the logits path"
    for key in r1:
        assert torch.equal(r1[key], r2[key]), key
    if T <= 300:
        check_output(y1.cpu().numpy(), O.moe_forward(p.layer, p.x, lg.cpu().numpy(), 8), f"router layer T={T} E={E}")
