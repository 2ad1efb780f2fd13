"""GPU parity of gqa_decode_paged over page pools of 8-bit codes (fp8 E4M3
or int8, read with unit scales) against the float64 oracle, through the C
ABI.  A caller with one K scale and one V scale folds the K scale into the
score scale and multiplies the output by the V scale; with power-of-two
scales that is exact, so the tolerance is the bf16 cache's (2e-3 max abs:
codes convert to bf16 exactly, accumulation is fp32).  Paging changes only
where rows live: the same call on the contiguous cache (gqa_decode_fp8 /
gqa_decode_int8, same plan, same tiles) gives the same bits."""
import math

import numpy as np
import pytest
import torch

import gqa_inputs as gi

pytestmark = pytest.mark.gpu
TOL = 2e-3


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


def _codes(x, kind):
    """8-bit codes of x [B,G,T,D] and the one scale they carry: E4M3 of x
    itself (scale 1), or int8 round(x * 32) (scale 1/32)."""
    if kind == "fp8":
        return x.float().to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), 1.0
    return torch.round(x.float() * 32).clamp(-128, 127).to(torch.int8).contiguous(), 1.0 / 32


def _to_pages(c, ps, perm):
    B, G, T, D = c.shape
    n = T // ps
    pages = torch.empty(B * n, G, ps, D, dtype=c.dtype)
    bt = torch.empty(B, n, dtype=torch.int32)
    for b in range(B):
        for i in range(n):
            p = int(perm[b * n + i])
            pages[p] = c[b, :, i * ps:(i + 1) * ps]
            bt[b, i] = p
    return pages, bt


def _err(got, want):
    g = got.double().cpu().numpy()
    assert np.isfinite(g).all()
    return float(np.abs(g - want).max()) if g.size else 0.0


CASES = [
    # B, H, G, D, T, sq, page_size, seq_lens
    (3, 32, 8, 128, 512, 1, 16, [512, 300, 17]),
    (2, 32, 8, 64, 512, 2, 64, [512, 65]),
    (2, 32, 1, 128, 320, 2, 32, [320, 33]),      # 64 query rows per KV head
    (2, 8, 2, 128, 256, 64, 16, [256, 100]),     # 256 rows: four 64-row blocks
    (4, 8, 2, 64, 256, 1, 256, [0, 1, 256, 999]),  # empty, one row, full, clamped
]


@pytest.mark.parametrize("kind", ["fp8", "int8"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_H%d_G%d_D%d_T%d_sq%d_ps%d" % c[:7])
def test_paged_codes_match_oracle_and_contiguous(gqa, orc, case, kind):
    B, H, G, D, T, sq, ps, lens = case
    x = gi.make_custom(B, H, G, D, T, sq, dtype="bf16", seed=760 + T + ps + sq, seq_lens=lens)
    kc, ks = _codes(x["k"], kind)
    vc, vs = _codes(x["v"], kind)
    perm = np.random.default_rng(ps + sq).permutation(B * (T // ps))
    kp, bt = _to_pages(kc, ps, perm)
    vp, _ = _to_pages(vc, ps, perm)
    for b, L in enumerate(lens):
        bt[b, (min(L, T) + ps - 1) // ps:] = -7     # never read
    deq = orc.dequant_fp8 if kind == "fp8" else orc.dequant_int8
    one = torch.ones(G)
    want = orc.decode_paged_f64(x["q"], deq(kp, one * ks), deq(vp, one * vs), bt, x["seq_lens"],
                                scale=1.0 / math.sqrt(D), threads=8)
    q, sl = x["q"].cuda(), x["seq_lens"].cuda()
    s = ks / math.sqrt(D)
    got = gqa.decode_paged(q, kp.cuda(), vp.cuda(), bt.cuda(), sl, scale=s)
    contiguous = gqa.decode_fp8 if kind == "fp8" else gqa.decode_int8
    ref = contiguous(q, kc.cuda(), vc.cuda(), None, None, sl, scale=s)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), (case, kind)
    assert _err(got * vs, want) <= TOL, (case, kind)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
def test_paged_codes_splits_and_long_walk(gqa, orc, kind):
    """A sequence of 1100 pages of 16 rows (the block table through LDS in
    several windows) and short ones, over 1, 7 and 200 workgroups with both
    merge modes."""
    B, H, G, D, ps = 3, 8, 2, 128, 16
    T = 1100 * ps
    x = gi.make_custom(B, H, G, D, T, 1, dtype="bf16", seed=771, seq_lens=[T, 40, 1000])
    kc, ks = _codes(x["k"], kind)
    vc, vs = _codes(x["v"], kind)
    perm = np.random.default_rng(772).permutation(B * (T // ps))
    kp, bt = _to_pages(kc, ps, perm)
    vp, _ = _to_pages(vc, ps, perm)
    deq = orc.dequant_fp8 if kind == "fp8" else orc.dequant_int8
    one = torch.ones(G)
    want = orc.decode_paged_f64(x["q"], deq(kp, one * ks), deq(vp, one * vs), bt, x["seq_lens"],
                                scale=1.0 / math.sqrt(D), threads=8)
    args = (x["q"].cuda(), kp.cuda(), vp.cuda(), bt.cuda(), x["seq_lens"].cuda())
    for P in (1, 7, 200):
        for m in (gqa.MERGE_IN_KERNEL, gqa.MERGE_COMBINE):
            got = gqa.decode_paged(*args, scale=ks / math.sqrt(D), workgroups=P, merge=m)
            torch.cuda.synchronize()
            assert _err(got * vs, want) <= TOL, (kind, P, m)


def test_paged_codes_refusals(gqa):
    """An 8-bit pool with an fp16 query, or on the vector-ALU path, is
    refused before any device work; appended tokens still need a 16-bit
    cache."""
    x = gi.make_custom(1, 8, 2, 64, 64, 1, dtype="bf16", seed=773)
    kp = torch.zeros(4, 2, 16, 64, dtype=torch.int8, device="cuda")
    bt = torch.arange(4, dtype=torch.int32, device="cuda").view(1, 4)
    q = x["q"].cuda()
    with pytest.raises(gqa.GqaError) as ei:
        gqa.decode_paged(q.half(), kp, kp.clone(), bt)
    assert ei.value.status == gqa.GQA_ERR_UNSUPPORTED
    with pytest.raises(gqa.GqaError) as ei:
        gqa.decode_paged(q, kp.view(torch.uint8), kp.view(torch.uint8).clone(), bt, path=gqa.PATH_VALU)
    assert ei.value.status == gqa.GQA_ERR_UNSUPPORTED
    kc = torch.zeros(1, 2, 64, 64, dtype=torch.int8, device="cuda")
    kn = torch.zeros(1, 2, 1, 64, dtype=torch.int8, device="cuda")
    with pytest.raises(gqa.GqaError) as ei:
        gqa.decode_append(q, kn, kn.clone(), kc, kc.clone())
    assert ei.value.status == gqa.GQA_ERR_UNSUPPORTED


def test_paged_fp8_pool_as_float8_dtype(gqa):
    """A pool passed as torch.float8_e4m3fn is the same bytes as its uint8
    view: the same call, the same bits."""
    B, H, G, D, T, ps = 2, 16, 4, 128, 256, 32
    x = gi.make_custom(B, H, G, D, T, 1, dtype="bf16", seed=774, seq_lens=[256, 90])
    kc, _ = _codes(x["k"], "fp8")
    vc, _ = _codes(x["v"], "fp8")
    perm = np.random.default_rng(775).permutation(B * (T // ps))
    kp, bt = _to_pages(kc, ps, perm)
    vp, _ = _to_pages(vc, ps, perm)
    q, sl, kp, vp, bt = x["q"].cuda(), x["seq_lens"].cuda(), kp.cuda(), vp.cuda(), bt.cuda()
    a = gqa.decode_paged(q, kp, vp, bt, sl)
    b = gqa.decode_paged(q, kp.view(torch.float8_e4m3fn), vp.view(torch.float8_e4m3fn), bt, sl)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
def test_paged_codes_full_size_sampled(gqa, orc, kind):
    """The batched GQA-8 workload (B = 32, H = 32, G = 8, D = 128, ragged
    T <= 4096) as a randomly ordered pool of 16-row pages, in the launch the
    benchmark times: the whole batch on the GPU, sampled sequences against
    the oracle on the host, and the whole output against the contiguous
    8-bit call bit for bit."""
    w = gi.WORKLOADS[gi.HEADLINE]
    x = gi.make_inputs(w, device="cuda")
    B, G, T, D, ps = w.B, w.G, w.T, w.D, 16
    kc, ks = _codes(x["k"], kind)
    vc, vs = _codes(x["v"], kind)
    n = T // ps
    perm = torch.randperm(B * n, generator=torch.Generator().manual_seed(776)).cuda()
    kp = torch.empty(B * n, G, ps, D, dtype=kc.dtype, device="cuda")
    vp = torch.empty_like(kp)
    kp[perm] = kc.view(B, G, n, ps, D).transpose(1, 2).reshape(B * n, G, ps, D)
    vp[perm] = vc.view(B, G, n, ps, D).transpose(1, 2).reshape(B * n, G, ps, D)
    bt = perm.view(B, n).to(torch.int32).contiguous()
    s = ks / math.sqrt(D)
    got = gqa.decode_paged(x["q"], kp, vp, bt, x["seq_lens"], scale=s)
    contiguous = gqa.decode_fp8 if kind == "fp8" else gqa.decode_int8
    ref = contiguous(x["q"], kc, vc, None, None, x["seq_lens"], scale=s)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    fn = orc.decode_fp8_f64 if kind == "fp8" else orc.decode_int8_f64
    one = torch.ones(G)
    for b in (0, 17, 31):
        want = fn(x["q"][b:b + 1].cpu(), kc[b:b + 1].cpu(), vc[b:b + 1].cpu(), one * ks, one * vs,
                  x["seq_lens"][b:b + 1].cpu(), 1.0 / math.sqrt(D), threads=8)
        assert _err(got[b:b + 1] * vs, want) <= TOL, (kind, b)
    del x, kc, vc, kp, vp, got, ref
    torch.cuda.empty_cache()
