"""GPU parity of the two cache variants against the float64 oracle, through
the C ABI: gqa_decode_append (new tokens stored into the cache and attended
in one pass) and gqa_decode_paged (page pool + block table).

Tolerances as for gqa_decode (bf16 inputs, fp32 accumulation: 2e-3 max
abs).  The cache rows an append writes are compared bit for bit; a paged
decode is also compared bit for bit with gqa_decode on the cache it
describes where both run the same kernel on the same tiles, otherwise to
within REORDER_TOL, as is an append with gqa_decode on the appended cache.
REORDER_TOL: the same sums in another order -- each weight p is
carried as bf16 hi + lo (about 16 significant bits), so a change in the
last bit of a score can move a weight by ~2^-16 of itself and an output by
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


def _err(got, want):
    got = got.double().cpu().numpy()
    assert np.isfinite(got).all()
    return float(np.abs(got - want).max()) if got.size else 0.0


APPEND = [
    # B, H, G, D, T, sq, seq_lens
    (3, 32, 8, 128, 600, 1, [600, 257, 1]),
    (2, 32, 8, 64, 300, 2, [300, 2]),
    (2, 32, 1, 128, 200, 1, [200, 99]),          # MQA: 32 rows, two query blocks
    (2, 32, 1, 128, 150, 2, [150, 77]),          # 64 rows, combine kernel
    (2, 8, 2, 128, 400, 64, [400, 70]),          # 64 new tokens, 256 rows
    (2, 4, 1, 64, 90, 8, [90, 5]),               # L < sq: three tokens dropped
]


@pytest.mark.parametrize("case", APPEND, ids=lambda c: "B%d_H%d_G%d_D%d_T%d_sq%d" % c[:6])
def test_append_matches_oracle_and_decode(gqa, orc, case):
    B, H, G, D, T, sq, lens = case
    x = gi.make_custom(B, H, G, D, T, sq, dtype="bf16", seed=400 + T + sq, seq_lens=lens)
    gen = torch.Generator().manual_seed(401 + sq)
    kn = torch.randn(B, G, sq, D, generator=gen).to(torch.bfloat16)
    vn = torch.randn(B, G, sq, D, generator=gen).to(torch.bfloat16)
    want, k_after, v_after = orc.decode_append_f64(x["q"], kn, vn, x["k"], x["v"], x["seq_lens"],
                                                   1.0 / math.sqrt(D), threads=8)
    kc, vc = x["k"].cuda(), x["v"].cuda()
    q, sl = x["q"].cuda(), x["seq_lens"].cuda()
    got = gqa.decode_append(q, kn.cuda(), vn.cuda(), kc, vc, sl)
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL
    assert np.array_equal(kc.double().cpu().numpy(), k_after)
    assert np.array_equal(vc.double().cpu().numpy(), v_after)
    # the same as gqa_decode on the appended cache, to rounding
    again = gqa.decode(q, kc, vc, sl)
    torch.cuda.synchronize()
    assert (got - again).abs().max().item() <= REORDER_TOL


def test_append_splits_and_merge_modes(gqa, orc):
    B, H, G, D, T, sq = 4, 32, 8, 128, 777, 2
    x = gi.make_custom(B, H, G, D, T, sq, dtype="bf16", seed=410, seq_lens=[777, 3, 400, 129])
    gen = torch.Generator().manual_seed(411)
    kn = torch.randn(B, G, sq, D, generator=gen).to(torch.bfloat16)
    vn = torch.randn(B, G, sq, D, generator=gen).to(torch.bfloat16)
    want, _, _ = orc.decode_append_f64(x["q"], kn, vn, x["k"], x["v"], x["seq_lens"], threads=8)
    for P in (1, 7, 300):
        for m in (gqa.MERGE_IN_KERNEL, gqa.MERGE_COMBINE):
            kc, vc = x["k"].cuda(), x["v"].cuda()
            got = gqa.decode_append(x["q"].cuda(), kn.cuda(), vn.cuda(), kc, vc, x["seq_lens"].cuda(),
                                    workgroups=P, merge=m)
            torch.cuda.synchronize()
            assert _err(got, want) <= TOL, (P, m)


def _to_pages(k, ps, perm):
    B, G, T, D = k.shape
    n = T // ps
    pages = torch.empty(B * n, G, ps, D, dtype=k.dtype, device=k.device)
    bt = torch.empty(B, n, dtype=torch.int32)
    for b in range(B):
        for i in range(n):
            p = int(perm[b * n + i])
            pages[p] = k[b, :, i * ps:(i + 1) * ps]
            bt[b, i] = p
    return pages, bt


PAGED = [
    # B, H, G, D, T, sq, page_size, seq_lens
    (3, 32, 8, 128, 512, 1, 16, [512, 300, 17]),
    (2, 32, 8, 64, 512, 2, 64, [512, 65]),
    (2, 32, 1, 128, 256, 1, 256, [256, 255]),
    (2, 32, 1, 128, 320, 2, 32, [320, 33]),
    (2, 8, 2, 128, 256, 64, 16, [256, 100]),
]


@pytest.mark.parametrize("case", PAGED, ids=lambda c: "B%d_H%d_G%d_D%d_T%d_sq%d_ps%d" % c[:7])
def test_paged_matches_oracle_and_decode(gqa, orc, monkeypatch, case):
    B, H, G, D, T, sq, ps, lens = case
    x = gi.make_custom(B, H, G, D, T, sq, dtype="bf16", seed=500 + T + ps, seq_lens=lens)
    perm = np.random.default_rng(ps).permutation(B * (T // ps))
    kp, bt = _to_pages(x["k"], ps, perm)
    vp, _ = _to_pages(x["v"], ps, perm)
    # table entries past each sequence's length are never read
    for b, L in enumerate(lens):
        bt[b, (L + ps - 1) // ps:] = -7
    want = orc.decode_paged_f64(x["q"], kp, vp, bt, x["seq_lens"], threads=8)
    q, sl = x["q"].cuda(), x["seq_lens"].cuda()
    got = gqa.decode_paged(q, kp.cuda(), vp.cuda(), bt.cuda(), sl)
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL
    ref = gqa.decode(q, x["k"].cuda(), x["v"].cuda(), sl)
    torch.cuda.synchronize()
    if (H // G) * sq <= 16:
        # a small contiguous cache runs on row-split workgroups (the same
        # sums in another order) ...
        assert (got - ref).abs().max().item() <= REORDER_TOL
        # ... and with one-wave workgroups forced, the paged cache's kernel
        # over the same rows: the same bits
        monkeypatch.setenv("GQA_RSPLIT", "0")
        ref = gqa.decode(q, x["k"].cuda(), x["v"].cuda(), sl)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
    else:
        # a contiguous cache of more than 16 query rows per KV head runs on
        # the 32 x 32 matrix-core kernel, the paged cache on 16 x 16 tiles:
        # the same sums in another order
        assert (got - ref).abs().max().item() <= REORDER_TOL


def test_paged_piece_longer_than_page_window(gqa, orc):
    """One workgroup walks a sequence of 2100 pages of 16 rows: the block
    table goes through LDS in several windows."""
    B, H, G, D, ps = 1, 4, 1, 64, 16
    T = 2100 * ps
    x = gi.make_custom(B, H, G, D, T, 1, dtype="bf16", seed=520)
    perm = np.random.default_rng(5).permutation(T // ps)
    kp, bt = _to_pages(x["k"], ps, perm)
    vp, _ = _to_pages(x["v"], ps, perm)
    want = orc.decode_paged_f64(x["q"], kp, vp, bt, None, threads=8)
    got = gqa.decode_paged(x["q"].cuda(), kp.cuda(), vp.cuda(), bt.cuda(), None, workgroups=1)
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL


def test_variants_reject_fp32_and_bad_pages(gqa):
    x = gi.make_custom(1, 8, 2, 64, 64, 1, dtype="f32", seed=530)
    kn = torch.zeros(1, 2, 1, 64, device="cuda")
    with pytest.raises(gqa.GqaError) as ei:
        gqa.decode_append(x["q"].cuda(), kn, kn.clone(), x["k"].cuda(), x["v"].cuda())
    assert ei.value.status == gqa.GQA_ERR_UNSUPPORTED
    xb = gi.make_custom(1, 8, 2, 64, 64, 1, dtype="bf16", seed=531)
    kp = torch.zeros(4, 2, 24, 64, dtype=torch.bfloat16, device="cuda")     # page size 24
    bt = torch.zeros(1, 3, dtype=torch.int32, device="cuda")
    with pytest.raises(gqa.GqaError) as ei:
        gqa.decode_paged(xb["q"].cuda(), kp, kp.clone(), bt)
    assert ei.value.status == gqa.GQA_ERR_INVALID_ARG


@pytest.mark.parametrize("case", [(2, 32, 1, 128, 150, 2, [150, 77]), (2, 8, 2, 128, 400, 64, [400, 70])],
                         ids=["R64", "R256"])
def test_append_with_caller_workspace(gqa, orc, case):
    """gqa_append_workspace_bytes sizes a caller-owned workspace for
    gqa_decode_append (above 32 query rows per KV head the append plans other
    row blocks and grids than the plain decode); the result equals the one
    with the library's workspace bit for bit, and the counters come back
    zero so the buffer can be reused at once."""
    B, H, G, D, T, sq, lens = case
    x = gi.make_custom(B, H, G, D, T, sq, dtype="bf16", seed=410 + sq, seq_lens=lens)
    gen = torch.Generator().manual_seed(411 + sq)
    kn = torch.randn(B, G, sq, D, generator=gen).to(torch.bfloat16).cuda()
    vn = torch.randn(B, G, sq, D, generator=gen).to(torch.bfloat16).cuda()
    want, _, _ = orc.decode_append_f64(x["q"], kn.cpu(), vn.cpu(), x["k"], x["v"], x["seq_lens"],
                                       1.0 / math.sqrt(D), threads=8)
    q, sl = x["q"].cuda(), x["seq_lens"].cuda()
    need = gqa.append_workspace_bytes(gqa.shape_of(q, x["k"]))
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    outs = []
    for use_ws in (True, True, False):
        kc, vc = x["k"].cuda(), x["v"].cuda()
        outs.append(gqa.decode_append(q, kn, vn, kc, vc, sl, workspace=ws if use_ws else None))
    torch.cuda.synchronize()
    assert _err(outs[0], want) <= TOL
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    assert int(ws[: 1 << 20].view(torch.int32).abs().sum().item()) == 0
