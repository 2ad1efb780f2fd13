"""GPU parity of the fp8 E4M3 cache (gqa_decode_fp8) against the float64
oracle through the C ABI.  Tolerance as for bf16 inputs (2e-3 max abs):
the codes convert to bf16 exactly and accumulation is fp32.  With
power-of-two scales the dequantized cache is exactly a bf16 cache, and the
fp8 call must agree with gqa_decode on it to within REORDER_TOL: the score
product sums the head dim in a different order, and each weight p is
carried as bf16 hi + lo (about 16 significant bits), so a last-bit change
of a score moves a weight by up to ~2^-16 of itself and an output by
~1e-5; 1e-4 bounds that with room, 20x under TOL."""
import math

import numpy as np
import pytest
import torch

import gqa_inputs as gi

pytestmark = pytest.mark.gpu
TOL = 2e-3
REORDER_TOL = 1e-4


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


def _quantize(x, G):
    """Per-KV-head symmetric scale (amax / 448) and E4M3 codes of x [B,G,T,D]."""
    amax = x.float().abs().amax(dim=(0, 2, 3)).clamp_min(1e-6)
    sc = (amax / 448.0).float()
    codes = (x.float() / sc.view(1, G, 1, 1)).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), sc


FP8 = [
    # B, H, G, D, T, sq, seq_lens
    (3, 32, 8, 128, 700, 1, [700, 333, 1]),
    (2, 32, 8, 64, 400, 2, [400, 3]),
    (2, 32, 1, 128, 300, 1, [300, 150]),       # 32 rows
    (2, 32, 1, 128, 200, 2, [200, 64]),        # 64 rows, combine kernel
    (4, 8, 2, 128, 128, 1, [0, 1, 128, 500]),  # empty, one row, full, clamped
]


@pytest.mark.parametrize("case", FP8, ids=lambda c: "B%d_H%d_G%d_D%d_T%d_sq%d" % c[:6])
def test_fp8_matches_oracle(gqa, orc, case):
    B, H, G, D, T, sq, lens = case
    x = gi.make_custom(B, H, G, D, T, sq, dtype="bf16", seed=600 + T + D, seq_lens=lens)
    kc, ks = _quantize(x["k"], G)
    vc, vs = _quantize(x["v"], G)
    want = orc.decode_fp8_f64(x["q"], kc, vc, ks, vs, x["seq_lens"], threads=8)
    got = gqa.decode_fp8(x["q"].cuda(), kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(), x["seq_lens"].cuda())
    torch.cuda.synchronize()
    g = got.double().cpu().numpy()
    assert np.isfinite(g).all()
    assert float(np.abs(g - want).max()) <= TOL


@pytest.mark.parametrize("B,D,lens", [(1, 128, [4096]), (2, 64, [4096, 1234])])
def test_fp8_small_cache_default_plan(gqa, orc, B, D, lens):
    """A small fp8 cache runs the default plan with at least 256 cache rows
    per wave (B * 8 * 4096 / 256 workgroups) and matches the oracle."""
    G = 8
    x = gi.make_custom(B, 32, G, D, 4096, 1, dtype="bf16", seed=620 + B + D, seq_lens=lens)
    kc, ks = _quantize(x["k"], G)
    vc, vs = _quantize(x["v"], G)
    plan = gqa.plan(gqa.shape_of(x["q"], kc))
    assert plan["workgroups"] == B * G * 4096 // 256
    want = orc.decode_fp8_f64(x["q"], kc, vc, ks, vs, x["seq_lens"], threads=8)
    got = gqa.decode_fp8(x["q"].cuda(), kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(), x["seq_lens"].cuda())
    torch.cuda.synchronize()
    g = got.double().cpu().numpy()
    assert np.isfinite(g).all()
    assert float(np.abs(g - want).max()) <= TOL


def test_fp8_with_power_of_two_scales_is_a_bf16_cache(gqa, orc):
    B, H, G, D, T, sq = 3, 32, 8, 128, 500, 1
    x = gi.make_custom(B, H, G, D, T, sq, dtype="bf16", seed=610, seq_lens=[500, 257, 30])
    gen = torch.Generator().manual_seed(611)
    kc = torch.randint(0, 256, (B, G, T, D), generator=gen, dtype=torch.uint8)
    vc = torch.randint(0, 256, (B, G, T, D), generator=gen, dtype=torch.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x30     # no NaN codes
    vc[(vc & 0x7F) == 0x7F] = 0x30
    ks = torch.tensor([2.0 ** -e for e in range(8)], dtype=torch.float32) / 64
    vs = torch.tensor([2.0 ** -e for e in range(8)], dtype=torch.float32) / 32
    want = orc.decode_fp8_f64(x["q"], kc, vc, ks, vs, x["seq_lens"], threads=8)
    q, sl = x["q"].cuda(), x["seq_lens"].cuda()
    got = gqa.decode_fp8(q, kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(), sl)
    kd = (kc.view(torch.float8_e4m3fn).float() * ks.view(1, G, 1, 1)).to(torch.bfloat16)
    vd = (vc.view(torch.float8_e4m3fn).float() * vs.view(1, G, 1, 1)).to(torch.bfloat16)
    ref = gqa.decode(q, kd.cuda(), vd.cuda(), sl)
    torch.cuda.synchronize()
    assert float(np.abs(got.double().cpu().numpy() - want).max()) <= TOL
    # same values; the score product sums the head dim in another order
    assert (got - ref).abs().max().item() <= REORDER_TOL


def test_fp8_unit_scales_through_decode(gqa, orc):
    B, H, G, D, T = 2, 16, 4, 64, 300
    x = gi.make_custom(B, H, G, D, T, 1, dtype="bf16", seed=620, seq_lens=[300, 100])
    kc, _ = _quantize(x["k"], G)
    vc, _ = _quantize(x["v"], G)
    one = torch.ones(G)
    want = orc.decode_fp8_f64(x["q"], kc, vc, one, one, x["seq_lens"], scale=0.01, threads=8)
    got = gqa.decode(x["q"].cuda(), kc.cuda(), vc.cuda(), x["seq_lens"].cuda(), scale=0.01)
    torch.cuda.synchronize()
    assert float(np.abs(got.double().cpu().numpy() - want).max()) <= TOL


def test_fp8_split_invariance_and_determinism(gqa, orc):
    B, H, G, D, T = 4, 32, 8, 128, 777
    x = gi.make_custom(B, H, G, D, T, 1, dtype="bf16", seed=630, seq_lens=[777, 3, 400, 129])
    kc, ks = _quantize(x["k"], G)
    vc, vs = _quantize(x["v"], G)
    want = orc.decode_fp8_f64(x["q"], kc, vc, ks, vs, x["seq_lens"], threads=8)
    args = (x["q"].cuda(), kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(), x["seq_lens"].cuda())
    for P in (1, 5, 64, 300):
        for m in (gqa.MERGE_IN_KERNEL, gqa.MERGE_COMBINE):
            o = gqa.decode_fp8(*args, workgroups=P, merge=m)
            torch.cuda.synchronize()
            assert float(np.abs(o.double().cpu().numpy() - want).max()) <= TOL
            assert torch.equal(o, gqa.decode_fp8(*args, workgroups=P, merge=m))


def test_fp8_rejections(gqa):
    x = gi.make_custom(1, 8, 2, 64, 64, 1, dtype="bf16", seed=640)
    kc = torch.zeros(1, 2, 64, 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(gqa.GqaError) as ei:
        gqa.decode(x["q"].cuda(), kc, kc.clone(), path=gqa.PATH_VALU)
    assert ei.value.status == gqa.GQA_ERR_UNSUPPORTED
    sc = torch.ones(2, device="cuda")
    with pytest.raises(gqa.GqaError) as ei:
        # scales with a bf16 cache
        import ctypes
        lib = gqa.load_library()
        shape = gqa.shape_of(x["q"], x["k"])
        q, k = x["q"].cuda(), x["k"].cuda()
        out = torch.empty(q.shape, device="cuda")
        gqa._check(lib.gqa_decode_fp8(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), k.data_ptr(),
                                      sc.data_ptr(), sc.data_ptr(), None, ctypes.c_float(0.1),
                                      out.data_ptr(), None, ctypes.c_size_t(0), None, None))
    assert ei.value.status == gqa.GQA_ERR_INVALID_ARG
