"""Seeded random shapes through every entry point of the C ABI against the
float64 oracle: gqa_decode, gqa_decode_append, gqa_decode_paged,
gqa_decode_fp8 and gqa_decode_int8, with random group sizes, head dims,
context lengths (ragged, with empty and single-row sequences), new-token counts, page sizes, grid
sizes and merge modes -- so that tile ends, row windows, page windows and
split points fall at arbitrary rows; the fp16 entry points on the same
shapes.  Tolerance as for the fixed cases (bf16 inputs, fp32 accumulation:
2e-3 max abs; fp16: 2e-4; fp32: 1e-5)."""
import math

import numpy as np
import pytest
import torch

import gqa_inputs as gi

pytestmark = pytest.mark.gpu
TOL = {"bf16": 2e-3, "f16": 2e-4, "f32": 1e-5}
N_CASES = 24


@pytest.fixture(scope="module")
def gqa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_query_attention_decode_amd as m
    m.load_library()
    return m


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


def _shape(i):
    """Case i: a shape small enough for the oracle, drawn from seed 7000 + i."""
    rng = np.random.default_rng(7000 + i)
    G = int(rng.choice([1, 2, 4, 8]))
    rep = int(rng.choice([1, 2, 3, 4, 8, 16]))
    sq = int(rng.choice([1, 1, 1, 2, 3, 5]))
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 5))
    T = int(rng.integers(1, 700))
    lens = [int(v) for v in rng.integers(0, T + 1, size=B)]
    if B > 1 and rng.random() < 0.3:
        lens[int(rng.integers(0, B))] = int(rng.choice([0, 1]))
    P = int(rng.choice([0, 0, 1, 7, 64, 1000]))
    merge = int(rng.choice([0, 1, 2]))
    return dict(B=B, H=G * rep, G=G, D=D, T=T, sq=sq, lens=lens, P=P, merge=merge, seed=7100 + i)


def _err(got, want):
    got = got.double().cpu().numpy()
    assert np.isfinite(got).all()
    return float(np.abs(got - want).max()) if got.size else 0.0


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_decode(gqa, orc, i):
    c = _shape(i)
    dt = "f32" if i % 6 == 5 else "bf16"
    x = gi.make_custom(c["B"], c["H"], c["G"], c["D"], c["T"], c["sq"], dtype=dt, seed=c["seed"],
                       seq_lens=c["lens"])
    want = orc.decode_f64(x["q"], x["k"], x["v"], x["seq_lens"], 1.0 / math.sqrt(c["D"]))
    kw = dict(workgroups=c["P"])
    if dt == "bf16":
        kw["merge"] = c["merge"]
    got = gqa.decode(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), x["seq_lens"].cuda(), **kw)
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL[dt], c


@pytest.mark.parametrize("forced", [("GQA_RSPLIT", "0"), ("GQA_RSPLIT", "2"), ("GQA_MFX", "0")],
                         ids=["one_wave", "row_split_2", "no_32x32"])
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_decode_other_kernels(gqa, orc, monkeypatch, i, forced):
    """The same shapes (bf16) with the planner's development switches forcing
    the kernels the default plans do not pick for them: one-wave workgroups
    instead of row-split ones on small caches, two-wave row splits, and the
    16 x 16 kernels instead of the 32 x 32 one above 16 query rows."""
    if i % 6 == 5:
        pytest.skip("fp32 shapes run on the vector-ALU kernel only")
    c = _shape(i)
    monkeypatch.setenv(*forced)
    x = gi.make_custom(c["B"], c["H"], c["G"], c["D"], c["T"], c["sq"], dtype="bf16", seed=c["seed"],
                       seq_lens=c["lens"])
    want = orc.decode_f64(x["q"], x["k"], x["v"], x["seq_lens"], 1.0 / math.sqrt(c["D"]))
    got = gqa.decode(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), x["seq_lens"].cuda(),
                     workgroups=c["P"], merge=c["merge"])
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL["bf16"], (c, forced)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_f16(gqa, orc, i):
    """fp16 q/k/v on the same shapes: the default plan, or (every third
    case) the vector-ALU kernel forced."""
    c = _shape(i)
    x = gi.make_custom(c["B"], c["H"], c["G"], c["D"], c["T"], c["sq"], dtype="f16", seed=c["seed"],
                       seq_lens=c["lens"])
    want = orc.decode_f64(x["q"], x["k"], x["v"], x["seq_lens"], 1.0 / math.sqrt(c["D"]))
    path = gqa.PATH_VALU if i % 3 == 0 else gqa.PATH_AUTO
    kw = dict(workgroups=c["P"], path=path)
    if path == gqa.PATH_AUTO:
        kw["merge"] = c["merge"]
    got = gqa.decode(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), x["seq_lens"].cuda(), **kw)
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL["f16"], (c, path)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_append(gqa, orc, i, dt):
    c = _shape(i)
    B, G, D, T, sq = c["B"], c["G"], c["D"], c["T"], c["sq"]
    x = gi.make_custom(B, c["H"], G, D, T, sq, dtype=dt, seed=c["seed"], seq_lens=c["lens"])
    gen = torch.Generator().manual_seed(c["seed"] + 1)
    kn = torch.randn(B, G, sq, D, generator=gen).to(x["k"].dtype)
    vn = torch.randn(B, G, sq, D, generator=gen).to(x["k"].dtype)
    want, k_after, v_after = orc.decode_append_f64(x["q"], kn, vn, x["k"], x["v"], x["seq_lens"],
                                                   1.0 / math.sqrt(D), threads=8)
    kc, vc = x["k"].cuda(), x["v"].cuda()
    got = gqa.decode_append(x["q"].cuda(), kn.cuda(), vn.cuda(), kc, vc, x["seq_lens"].cuda(),
                            workgroups=c["P"], merge=c["merge"])
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL[dt], c
    assert np.array_equal(kc.double().cpu().numpy(), k_after), c
    assert np.array_equal(vc.double().cpu().numpy(), v_after), c


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_paged(gqa, orc, i, dt):
    c = _shape(i)
    B, G, D, T = c["B"], c["G"], c["D"], c["T"]
    ps = int(np.random.default_rng(c["seed"]).choice([16, 32, 64, 256]))
    n = (T + ps - 1) // ps
    x = gi.make_custom(B, c["H"], G, D, n * ps, c["sq"], dtype=dt, seed=c["seed"],
                       seq_lens=[min(L, n * ps) for L in c["lens"]])
    perm = np.random.default_rng(c["seed"] + 2).permutation(B * n)
    kp = torch.empty(B * n, G, ps, D, dtype=x["k"].dtype)
    vp = torch.empty_like(kp)
    bt = torch.empty(B, n, dtype=torch.int32)
    for b in range(B):
        for j in range(n):
            p = int(perm[b * n + j])
            kp[p] = x["k"][b, :, j * ps:(j + 1) * ps]
            vp[p] = x["v"][b, :, j * ps:(j + 1) * ps]
            bt[b, j] = p
    want = orc.decode_paged_f64(x["q"], kp, vp, bt, x["seq_lens"], threads=8)
    got = gqa.decode_paged(x["q"].cuda(), kp.cuda(), vp.cuda(), bt.cuda(), x["seq_lens"].cuda(),
                           workgroups=c["P"], merge=c["merge"])
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL[dt], (c, ps)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_fp8(gqa, orc, i):
    c = _shape(i)
    B, G, D, T = c["B"], c["G"], c["D"], c["T"]
    x = gi.make_custom(B, c["H"], G, D, T, c["sq"], dtype="bf16", seed=c["seed"], seq_lens=c["lens"])
    gen = torch.Generator().manual_seed(c["seed"] + 3)
    kc = torch.randint(0, 256, (B, G, T, D), generator=gen, dtype=torch.uint8)
    vc = torch.randint(0, 256, (B, G, T, D), generator=gen, dtype=torch.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x38     # no NaN codes
    vc[(vc & 0x7F) == 0x7F] = 0x38
    ks = (torch.rand(G, generator=gen) * 0.01 + 0.001).float()
    vs = (torch.rand(G, generator=gen) * 0.01 + 0.001).float()
    want = orc.decode_fp8_f64(x["q"], kc, vc, ks, vs, x["seq_lens"], threads=8)
    got = gqa.decode_fp8(x["q"].cuda(), kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(), x["seq_lens"].cuda(),
                         workgroups=c["P"], merge=c["merge"])
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL["bf16"], c


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_int8(gqa, orc, i):
    c = _shape(i)
    B, G, D, T = c["B"], c["G"], c["D"], c["T"]
    x = gi.make_custom(B, c["H"], G, D, T, c["sq"], dtype="bf16", seed=c["seed"], seq_lens=c["lens"])
    gen = torch.Generator().manual_seed(c["seed"] + 4)
    kc = torch.randint(-128, 128, (B, G, T, D), generator=gen, dtype=torch.int8)
    vc = torch.randint(-128, 128, (B, G, T, D), generator=gen, dtype=torch.int8)
    ks = (torch.rand(G, generator=gen) * 0.01 + 0.001).float()
    vs = (torch.rand(G, generator=gen) * 0.01 + 0.001).float()
    want = orc.decode_int8_f64(x["q"], kc, vc, ks, vs, x["seq_lens"], threads=8)
    got = gqa.decode_int8(x["q"].cuda(), kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(), x["seq_lens"].cuda(),
                          workgroups=c["P"], merge=c["merge"])
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL["bf16"], c
