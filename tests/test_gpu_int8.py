"""GPU parity of the int8 cache (gqa_decode_int8) against the float64
oracle through the C ABI.  Tolerance as for bf16 inputs (2e-3 max abs):
the codes convert to bf16 exactly (as c + 128, the offset leaving the scores
through the softmax and the outputs at the end) and accumulation is fp32.
With power-of-two scales the dequantized cache is exactly a bf16 cache, and
the int8 call must agree with gqa_decode on it to within REORDER_TOL: the
scores carry a per-row offset and the weighted sum runs over c + 128, so the
same sums round differently (each weight carries ~16 significant bits;
1e-4 bounds the reordering with room, as for the fp8 cache)."""
import ctypes

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
    """Per-KV-head symmetric scale (amax / 127) and int8 codes of x [B,G,T,D]."""
    amax = x.float().abs().amax(dim=(0, 2, 3)).clamp_min(1e-6)
    sc = (amax / 127.0).float()
    codes = torch.round(x.float() / sc.view(1, G, 1, 1)).clamp(-128, 127).to(torch.int8)
    return codes.contiguous(), sc


def _err(got, want):
    g = got.double().cpu().numpy()
    assert np.isfinite(g).all()
    return float(np.abs(g - want).max()) if g.size else 0.0


INT8 = [
    # B, H, G, D, T, sq, seq_lens
    (3, 32, 8, 128, 700, 1, [700, 333, 1]),
    (2, 32, 8, 64, 400, 2, [400, 3]),
    (2, 32, 1, 128, 300, 1, [300, 150]),       # 32 rows
    (2, 32, 1, 128, 200, 2, [200, 64]),        # 64 rows, combine kernel
    (4, 8, 2, 128, 128, 1, [0, 1, 128, 500]),  # empty, one row, full, clamped
    (2, 8, 4, 64, 50, 3, [2, 3]),              # rows that see nothing
]


@pytest.mark.parametrize("case", INT8, ids=lambda c: "B%d_H%d_G%d_D%d_T%d_sq%d" % c[:6])
def test_int8_matches_oracle(gqa, orc, case):
    B, H, G, D, T, sq, lens = case
    x = gi.make_custom(B, H, G, D, T, sq, dtype="bf16", seed=680 + T + D, seq_lens=lens)
    kc, ks = _quantize(x["k"], G)
    vc, vs = _quantize(x["v"], G)
    want = orc.decode_int8_f64(x["q"], kc, vc, ks, vs, x["seq_lens"], threads=8)
    got = gqa.decode_int8(x["q"].cuda(), kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(), x["seq_lens"].cuda())
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL, case


def test_int8_extreme_codes(gqa, orc):
    """Codes at the ends of the range (-128, 127) and large per-head scales
    in V (outputs in the hundreds): the offset of 128 comes off exactly."""
    B, H, G, D, T = 2, 32, 8, 128, 300
    gen = torch.Generator().manual_seed(690)
    x = gi.make_custom(B, H, G, D, T, 1, dtype="bf16", seed=691, seq_lens=[300, 40])
    kc = torch.randint(-128, 128, (B, G, T, D), generator=gen, dtype=torch.int8)
    vc = torch.where(torch.rand(B, G, T, D, generator=gen) < 0.5, -128, 127).to(torch.int8)
    ks = torch.full((G,), 0.01)
    vs = torch.linspace(0.5, 4.0, G)
    want = orc.decode_int8_f64(x["q"], kc, vc, ks, vs, x["seq_lens"], threads=8)
    got = gqa.decode_int8(x["q"].cuda(), kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(), x["seq_lens"].cuda())
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL * float(np.abs(want).max())


def test_int8_small_cache_default_plan(gqa, orc):
    """A small int8 cache plans as an fp8 one (at least 256 cache rows per
    wave) and matches the oracle."""
    B, G, D = 2, 8, 64
    x = gi.make_custom(B, 32, G, D, 4096, 1, dtype="bf16", seed=692, seq_lens=[4096, 1234])
    kc, ks = _quantize(x["k"], G)
    vc, vs = _quantize(x["v"], G)
    plan = gqa.plan(gqa.shape_of(x["q"], kc))
    assert plan["workgroups"] == B * G * 4096 // 256
    want = orc.decode_int8_f64(x["q"], kc, vc, ks, vs, x["seq_lens"], threads=8)
    got = gqa.decode_int8(x["q"].cuda(), kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(), x["seq_lens"].cuda())
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL


def test_int8_with_power_of_two_scales_is_a_bf16_cache(gqa, orc):
    B, H, G, D, T, sq = 3, 32, 8, 128, 500, 1
    x = gi.make_custom(B, H, G, D, T, sq, dtype="bf16", seed=693, seq_lens=[500, 257, 30])
    gen = torch.Generator().manual_seed(694)
    kc = torch.randint(-128, 128, (B, G, T, D), generator=gen, dtype=torch.int8)
    vc = torch.randint(-128, 128, (B, G, T, D), generator=gen, dtype=torch.int8)
    ks = torch.tensor([2.0 ** -e for e in range(8)], dtype=torch.float32) / 512
    vs = torch.tensor([2.0 ** -e for e in range(8)], dtype=torch.float32) / 64
    want = orc.decode_int8_f64(x["q"], kc, vc, ks, vs, x["seq_lens"], threads=8)
    q, sl = x["q"].cuda(), x["seq_lens"].cuda()
    got = gqa.decode_int8(q, kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(), sl)
    kd = (kc.float() * ks.view(1, G, 1, 1)).to(torch.bfloat16)
    vd = (vc.float() * vs.view(1, G, 1, 1)).to(torch.bfloat16)
    ref = gqa.decode(q, kd.cuda(), vd.cuda(), sl)
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL
    assert (got - ref).abs().max().item() <= REORDER_TOL


def test_int8_unit_scales_through_decode(gqa, orc):
    B, H, G, D, T = 2, 16, 4, 64, 300
    x = gi.make_custom(B, H, G, D, T, 1, dtype="bf16", seed=695, seq_lens=[300, 100])
    kc, _ = _quantize(x["k"], G)
    vc, _ = _quantize(x["v"], G)
    one = torch.ones(G)
    want = orc.decode_int8_f64(x["q"], kc, vc, one, one, x["seq_lens"], scale=0.001, threads=8)
    got = gqa.decode(x["q"].cuda(), kc.cuda(), vc.cuda(), x["seq_lens"].cuda(), scale=0.001)
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL * float(np.abs(want).max())


def test_int8_split_invariance_and_determinism(gqa, orc):
    B, H, G, D, T = 4, 32, 8, 128, 777
    x = gi.make_custom(B, H, G, D, T, 1, dtype="bf16", seed=696, seq_lens=[777, 3, 400, 129])
    kc, ks = _quantize(x["k"], G)
    vc, vs = _quantize(x["v"], G)
    want = orc.decode_int8_f64(x["q"], kc, vc, ks, vs, x["seq_lens"], threads=8)
    args = (x["q"].cuda(), kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(), x["seq_lens"].cuda())
    for P in (1, 5, 64, 300):
        for m in (gqa.MERGE_IN_KERNEL, gqa.MERGE_COMBINE):
            o = gqa.decode_int8(*args, workgroups=P, merge=m)
            torch.cuda.synchronize()
            assert _err(o, want) <= TOL, (P, m)
            assert torch.equal(o, gqa.decode_int8(*args, workgroups=P, merge=m))


def test_int8_rejections(gqa):
    """Another path, an int8 cache through the fp8 entry point (and the
    reverse), and an fp16 query with int8 codes are refused before any
    device work."""
    x = gi.make_custom(1, 8, 2, 64, 64, 1, dtype="bf16", seed=697)
    kc = torch.zeros(1, 2, 64, 64, dtype=torch.int8, device="cuda")
    q = x["q"].cuda()
    with pytest.raises(gqa.GqaError) as ei:
        gqa.decode(q, kc, kc.clone(), path=gqa.PATH_VALU)
    assert ei.value.status == gqa.GQA_ERR_UNSUPPORTED
    with pytest.raises(gqa.GqaError) as ei:
        gqa.decode_fp8(q, kc, kc.clone())
    assert ei.value.status == gqa.GQA_ERR_INVALID_ARG
    with pytest.raises(gqa.GqaError) as ei:
        gqa.decode_int8(q, kc.view(torch.uint8), kc.view(torch.uint8).clone())
    assert ei.value.status == gqa.GQA_ERR_INVALID_ARG
    with pytest.raises(gqa.GqaError) as ei:
        gqa.decode_int8(q.half(), kc, kc.clone())
    assert ei.value.status == gqa.GQA_ERR_UNSUPPORTED
    lib = gqa.load_library()
    assert ctypes.cast(lib.gqa_decode_int8, ctypes.c_void_p).value
