"""GPU: the prepared weight copy (moe_prepare_weights).

1. The bytes moe_prepare_weights writes equal a NumPy construction of the
   layout the header and prep_layout.h define, from the original arrays.
2. A layer with its prepared copy gives the same y, bit for bit, as the same
   layer without it (the GEMMs do the same arithmetic in the same order), on
   shapes with full and half-empty column slices, half-width items, several
   K steps and table refills, with and without a shared expert."""
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


def _row(t, c, N, swiglu):
    if swiglu:
        f = N // 2
        j = 128 * t + (c & 127)
        return (j if c < 128 else f + j) if j < f else -1
    n = 256 * t + c
    return n if n < N else -1


def _slices(N, swiglu):
    return (N // 2 + 127) // 128 if swiglu else (N + 255) // 256


def prep_codes_np(q, N, K, swiglu):
    """q [E][N][K/8] uint32 -> [E][S][steps][16 chunks][64 lanes][4 words]."""
    E, steps = q.shape[0], K // 128
    S_ = _slices(N, swiglu)
    out = np.zeros((E, S_, steps, 16, 64, 4), np.uint32)
    for t in range(S_):
        for chunk in range(16):
            w, b = divmod(chunk, 4)
            for c in range(16):
                if swiglu:
                    lc = (32 * w + 16 * b if b < 2 else 128 + 32 * w + 16 * (b - 2)) + c
                else:
                    lc = 64 * w + 16 * b + c
                n = _row(t, lc, N, swiglu)
                if n < 0:
                    continue
                for st in range(steps):
                    for qq in range(4):
                        out[:, t, st, chunk, 16 * qq + c, :] = q[:, n, 16 * st + 4 * qq:16 * st + 4 * qq + 4]
    return out.reshape(E, -1)


def prep_table_np(s_bits, b_bits, N, K, swiglu):
    """bf16 bits [E][N][K/64] -> packed (fp16 s * 2^20, fp16 b) [E][S][G][256]
    (the scales here are inside the range of that form)."""
    E, G = s_bits.shape[0], K // 64
    sf = S.bf16_bits_to_f32(s_bits).astype(np.float64)
    bf = S.bf16_bits_to_f32(b_bits).astype(np.float64)
    assert np.all(np.abs(sf) < 2.0 ** -4)
    lo = (sf * 2.0 ** 20).astype(np.float16)
    assert np.array_equal(lo.astype(np.float64), sf * 2.0 ** 20)  # exact
    hi = bf.astype(np.float16)
    assert np.array_equal(hi.astype(np.float64), bf)              # exact
    packed = lo.view(np.uint16).astype(np.uint32) | (hi.view(np.uint16).astype(np.uint32) << 16)
    S_ = _slices(N, swiglu)
    out = np.zeros((E, S_, G, 256), np.uint32)
    for t in range(S_):
        for c in range(256):
            n = _row(t, c, N, swiglu)
            if n >= 0:
                out[:, t, :, c] = packed[:, n, :]
    return out.reshape(E, -1)


@pytest.mark.parametrize("d,f,E,f_sh", [(256, 128, 3, 128), (384, 256, 2, 0)])
def test_prepared_bytes_follow_the_layout(moe, d, f, E, f_sh):
    say(f"prepared layout d={d} f={f} E={E} f_sh={f_sh}")
    p = S.make_custom(16, S.LayerShape(d=d, f=f, E=E, k=1, f_sh=f_sh), seed=d + f + E)
    layer = moe.Layer.from_numpy(d, f, E, 1, f_sh, p.layer)
    n = moe.prepared_bytes(layer)
    assert layer.c.prep and n > 0
    off = layer.c.prep - layer.prep.data_ptr()
    got = layer.prep[off:off + n].cpu().numpy().view(np.uint32)
    L = p.layer
    parts = [prep_codes_np(L["gu_q"], 2 * f, d, True), prep_table_np(L["gu_s"], L["gu_b"], 2 * f, d, True),
             prep_codes_np(L["dn_q"], d, f, False), prep_table_np(L["dn_s"], L["dn_b"], d, f, False)]
    if f_sh:
        parts += [prep_codes_np(L["sh_gu_q"][None], 2 * f_sh, d, True),
                  prep_table_np(L["sh_gu_s"][None], L["sh_gu_b"][None], 2 * f_sh, d, True),
                  prep_codes_np(L["sh_dn_q"][None], d, f_sh, False),
                  prep_table_np(L["sh_dn_s"][None], L["sh_dn_b"][None], d, f_sh, False)]
    flags = got[:4]
    assert flags.tolist() == [1, 1, 1 if f_sh else 0, 1 if f_sh else 0], flags
    at = 64  # after the 256-byte header of flags
    for i, ref in enumerate(parts):
        ref = ref.reshape(-1)
        assert np.array_equal(got[at:at + ref.size], ref), f"region {i}"
        at += (ref.size * 4 + 255) // 256 * 256 // 4
    assert at * 4 == n


PREP_SHAPES = [
    # T, d, f, E, k, f_sh
    (2048, 2048, 512, 256, 8, 512),   # the 2048-token workload
    (512, 2048, 512, 256, 8, 512),    # mostly one-block units, half-width tail
    (300, 384, 256, 12, 3, 128),      # down: a half-empty second column slice
    (129, 256, 128, 8, 8, 128),       # one K step of down, two of gate/up
    (200, 2560, 384, 5, 2, 0),        # gate/up: 20 K steps, table refilled at steps 8 and 16
    (96, 1024, 1024, 3, 2, 1024),     # several slices per unit, long shared expert
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("T,d,f,E,k,f_sh", PREP_SHAPES)
def test_prepared_equals_unprepared(moe, T, d, f, E, k, f_sh):
    say(f"prepared vs original weights T={T} d={d} f={f} E={E} k={k} f_sh={f_sh}")
    p = S.make_custom(T, S.LayerShape(d=d, f=f, E=E, k=k, f_sh=f_sh), seed=T + 7 * d + f)
    plain = moe.Layer.from_numpy(d, f, E, k, f_sh, p.layer, prepare=False)
    prep = moe.Layer(d, f, E, k, f_sh, plain.tensors, prepare=True)
    assert not plain.c.prep and prep.c.prep
    x = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).cuda()
    lg = torch.from_numpy(p.logits).cuda()
    y0 = moe.layer_forward(plain, x, lg)
    y1 = moe.layer_forward(prep, x, lg)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    assert torch.isfinite(y1).all()


def test_large_scale_projection_falls_back(moe):
    """A gate/up scale of 2^-4 or more keeps the gate/up flag at 0 (that GEMM
    reads the original arrays); the other projections stay prepared; y still
    equals the unprepared layer's."""
    T, d, f, E, k, f_sh = 200, 512, 256, 6, 2, 128
    p = S.make_custom(T, S.LayerShape(d=d, f=f, E=E, k=k, f_sh=f_sh), seed=77)
    lay = dict(p.layer)
    gs = lay["gu_s"].copy()
    gs[2, 5, 1] = S.f32_to_bf16_bits(np.array([0.0625], np.float32))[0]
    lay["gu_s"] = gs
    say("large scale in routed gate/up: prepared flags and outputs")
    plain = moe.Layer.from_numpy(d, f, E, k, f_sh, lay, prepare=False)
    prep = moe.Layer(d, f, E, k, f_sh, plain.tensors, prepare=True)
    off = prep.c.prep - prep.prep.data_ptr()
    flags = prep.prep[off:off + 16].cpu().numpy().view(np.uint32)
    assert flags.tolist() == [0, 1, 1, 1], flags
    x = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).cuda()
    lg = torch.from_numpy(p.logits).cuda()
    y0 = moe.layer_forward(plain, x, lg)
    y1 = moe.layer_forward(prep, x, lg)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
