"""GPU parity of fp16 q/k/v (fp32 out) against the float64 CPU oracle.

The matrix-core kernels take fp16 operands where they take bf16 ones
(v_mfma_f32_{16x16x32,16x16x16,32x32x16}_f16, fp32 accumulation) and the
vector-ALU kernel accumulates fp16 pairs in fp32 (v_dot2_f32_f16); the
softmax weights enter the V product as an fp16 pair hi + lo.  The appended-
token and paged entry points take fp16 on the one-block kernel.

Tolerance 2e-4 (max abs error), derived from the arithmetic: the q.k and
p.v products of fp16 values are exact in fp32 and the weights carry ~22
bits (hi + lo), so what remains is fp32 accumulation over <= 16384 rows
(~1e-5 on these N(0,1) fields).  The bar is tighter than the 2e-3 of bf16
on purpose: dropping the lo half of the weights (2^-12 relative) or
rounding any operand to bf16 (2^-9) moves outputs by 5e-4 or more.
"""
import math

import numpy as np
import pytest
import torch

import gqa_inputs as gi

pytestmark = pytest.mark.gpu

TOL = 2e-4


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


def _to(x, device):
    return {k: v.to(device) for k, v in x.items()}


def _run(gqa, x, scale=None, **kw):
    out = gqa.decode(x["q"], x["k"], x["v"], x["seq_lens"], scale, **kw)
    torch.cuda.synchronize()
    return out


def _compare(got, want, what, tol=TOL):
    got = got.double().cpu().numpy()
    assert np.isfinite(got).all(), what + ": non-finite output"
    err = np.abs(got - want).max() if got.size else 0.0
    assert err <= tol, "%s: max abs error %.3g > %.3g" % (what, err, tol)
    return err


CASES = [
    # B, H, G, D, T, sq, seq_lens
    (3, 32, 8, 128, 1000, 1, [1000, 999, 517]),       # one 16-row block (4 rows live)
    (3, 32, 8, 64, 777, 1, [777, 1, 64]),
    (4, 8, 2, 128, 64, 1, [0, 1, 64, 200]),           # empty, single row, full, clamped
    (2, 12, 4, 64, 200, 1, [200, 77]),                # R = 3
    (2, 32, 4, 128, 500, 2, [500, 311]),              # R = 16
    (2, 16, 1, 128, 401, 2, [401, 250]),              # R = 32: the 32 x 32 kernel, 4 waves
    (2, 32, 1, 64, 300, 2, [300, 123]),               # R = 64
    (2, 32, 1, 64, 200, 3, [200, 50]),                # R = 96 in a 128-row segment
    (1, 32, 8, 64, 200, 64, [200]),                   # R = 256, sq = 64
    (2, 8, 4, 64, 50, 3, [2, 3]),                     # rows that see nothing
    (1, 4, 2, 128, 1, 1, None),                       # T = 1
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_H%d_G%d_D%d_T%d_sq%d" % c[:6])
@pytest.mark.parametrize("path_name", ["auto", "valu"])
def test_f16_shapes(gqa, orc, case, path_name):
    B, H, G, D, T, sq, lens = case
    path = {"auto": gqa.PATH_AUTO, "valu": gqa.PATH_VALU}[path_name]
    x = gi.make_custom(B, H, G, D, T, sq, dtype="f16", seed=500 + T + sq, seq_lens=lens)
    assert x["k"].dtype == torch.float16
    want = orc.decode_f64(x["q"], x["k"], x["v"], x["seq_lens"], 1.0 / math.sqrt(D))
    xc = _to(x, "cuda")
    p = gqa.plan(gqa.shape_of(xc["q"], xc["k"]), path=path)
    assert p["path"] == (gqa.PATH_VALU if path_name == "valu" else gqa.PATH_MFMA)
    got = _run(gqa, xc, path=path)
    _compare(got, want, "%s %s" % (path_name, case))
    assert torch.equal(got, _run(gqa, xc, path=path))


def test_f16_exaone_layer_row_split(gqa, orc):
    """The Exaone layer's shape (B=1, H=32, G=8, D=64, T=4096) in fp16 runs
    the row-split workgroups (4 waves) and matches the oracle in full."""
    w = gi.WORKLOADS["exaone_b1_h32_g8_d64_t4096"].scaled(dtype="f16", seed=611)
    x = gi.make_inputs(w)
    want = orc.decode_f64(x["q"], x["k"], x["v"], x["seq_lens"], 1.0 / math.sqrt(w.D), threads=8)
    xc = _to(x, "cuda")
    p = gqa.plan(gqa.shape_of(xc["q"], xc["k"]))
    assert p["path"] == gqa.PATH_MFMA and p["waves_per_group"] == 4
    _compare(_run(gqa, xc), want, "exaone f16")


def test_f16_batched_one_block(gqa, orc):
    """The batched GQA-8 decode at full size (B=32, T=4096, ragged lengths)
    in fp16: one-wave workgroups of the one-block kernel; whole sampled
    sequences against the oracle, at the default grid and at small splits."""
    w = gi.WORKLOADS["batched_b32_h32_g8_d128_t4096_ragged"].scaled(dtype="f16", seed=612)
    x = gi.make_inputs(w, device="cuda")
    p = gqa.plan(gqa.shape_of(x["q"], x["k"]))
    assert p["path"] == gqa.PATH_MFMA and p["waves_per_group"] == 1 and p["row_block"] == 16
    got = _run(gqa, x)
    for b in (0, 13, 31):
        xb = {k: v[b:b + 1].cpu() for k, v in x.items()}
        want = orc.decode_f64(xb["q"], xb["k"], xb["v"], xb["seq_lens"], 1.0 / math.sqrt(w.D), threads=8)
        _compare(got[b:b + 1], want, "batched f16 row %d" % b)
    for P in (7, 100):
        o = _run(gqa, x, workgroups=P)
        assert (o - got).abs().max().item() <= TOL
    del x, got
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,rows", [("mqa_b64_h32_g1_d128_t8192", (0, 40)),
                                       ("multitoken_b8_h32_g8_d128_t4096_sq64", (2,))])
def test_f16_many_rows_full_size(gqa, orc, name, rows):
    """MQA (32 rows per KV head) and 64 new tokens (256 rows) in fp16 at
    full size: the 32 x 32 kernel; sampled whole sequences."""
    w = gi.WORKLOADS[name].scaled(dtype="f16", seed=613)
    x = gi.make_inputs(w, device="cuda")
    p = gqa.plan(gqa.shape_of(x["q"], x["k"]))
    assert p["path"] == gqa.PATH_MFMA and p["waves_per_group"] in (4, 8)
    got = _run(gqa, x)
    for b in rows:
        xb = {k: v[b:b + 1].cpu() for k, v in x.items()}
        want = orc.decode_f64(xb["q"], xb["k"], xb["v"], xb["seq_lens"], 1.0 / math.sqrt(w.D), threads=8)
        _compare(got[b:b + 1], want, "%s row %d" % (name, b))
    del x, got
    torch.cuda.empty_cache()


@pytest.mark.parametrize("H,G,sq", [(32, 8, 1), (32, 1, 1), (32, 1, 2)])
def test_f16_split_invariance_and_merge_modes(gqa, orc, H, G, sq):
    """Any split, with the in-kernel merge or the combine kernel, gives the
    oracle's result; the same plan gives the same bits every call."""
    x = gi.make_custom(4, H, G, 128, 777, sq, dtype="f16", seed=620 + G + sq, seq_lens=[777, 3, 400, 129])
    want = orc.decode_f64(x["q"], x["k"], x["v"], x["seq_lens"], 1.0 / math.sqrt(128))
    xc = _to(x, "cuda")
    for P in (1, 5, 64, 300):
        for m in (gqa.MERGE_IN_KERNEL, gqa.MERGE_COMBINE):
            kw = dict(workgroups=P, merge=m)
            o = _run(gqa, xc, **kw)
            _compare(o, want, "P=%d merge=%d" % (P, m))
            assert torch.equal(o, _run(gqa, xc, **kw))


def test_f16_values_bf16_cannot_hold(gqa, orc):
    """q, k and v hold values with 10-bit mantissas and a spread of
    exponents (2^-8 .. 2^6) that bf16 would round: any bf16 step in the
    kernels shows up as an error of 2^-9 relative, far above the bar."""
    B, H, G, D, T = 2, 32, 8, 128, 600
    g = torch.Generator().manual_seed(630)
    def field(shape, lo, hi):
        m = 1.0 + torch.randint(0, 1024, shape, generator=g).double() / 1024.0
        e = torch.randint(lo, hi + 1, shape, generator=g).double()
        s = torch.where(torch.rand(shape, generator=g) < 0.5, -1.0, 1.0).double()
        return (s * m * torch.pow(2.0, e)).to(torch.float16)
    q = field((B, H, 1, D), -8, -2)
    k = field((B, G, T, D), -4, 1)
    v = field((B, G, T, D), -8, 6)
    lens = torch.tensor([600, 257], dtype=torch.int32)
    assert not torch.equal(v.to(torch.bfloat16).to(torch.float16), v)
    want = orc.decode_f64(q, k, v, lens, 1.0 / math.sqrt(D))
    tol = TOL * max(1.0, float(np.abs(want).max()))
    for path in (gqa.PATH_AUTO, gqa.PATH_VALU):
        got = gqa.decode(q.cuda(), k.cuda(), v.cuda(), lens.cuda(), path=path)
        torch.cuda.synchronize()
        _compare(got, want, "path %d" % path, tol=tol)


@pytest.mark.parametrize("path_name", ["auto", "valu"])
def test_f16_poisoned_tail_is_never_read(gqa, path_name):
    """Cache rows at or beyond seq_lens hold NaN: the output is finite and
    bit-identical to the run with ordinary values there."""
    path = {"auto": gqa.PATH_AUTO, "valu": gqa.PATH_VALU}[path_name]
    args = (3, 32, 8, 128, 700, 2)
    lens = [700, 333, 5]
    clean = _to(gi.make_custom(*args, dtype="f16", seed=9, seq_lens=lens), "cuda")
    dirty = _to(gi.make_custom(*args, dtype="f16", seed=9, seq_lens=lens, poison_tail=True), "cuda")
    a = _run(gqa, clean, path=path)
    b = _run(gqa, dirty, path=path)
    assert torch.isfinite(b).all()
    assert torch.equal(a, b)


def test_f16_unsupported_forms_refused(gqa):
    """fp16 has no scores-only matrix form and does not mix with an fp8
    cache: each is refused with GQA_ERR_UNSUPPORTED before any device work."""
    x = _to(gi.make_custom(2, 32, 8, 128, 64, 1, dtype="f16", seed=3, seq_lens=[10, 20]), "cuda")
    with pytest.raises(gqa.GqaError) as ei:
        gqa.decode(x["q"], x["k"], x["v"], x["seq_lens"], path=gqa.PATH_MFMA_QK)
    assert ei.value.status == gqa.GQA_ERR_UNSUPPORTED
    codes = torch.zeros(2, 8, 64, 128, dtype=torch.uint8, device="cuda")
    with pytest.raises(gqa.GqaError) as ei:
        gqa.decode_fp8(x["q"], codes, codes.clone(), seq_lens=x["seq_lens"])
    assert ei.value.status == gqa.GQA_ERR_UNSUPPORTED


APPEND = [
    # B, H, G, D, T, sq, seq_lens
    (3, 32, 8, 128, 600, 1, [600, 257, 1]),
    (2, 32, 8, 64, 300, 2, [300, 2]),
    (2, 32, 1, 128, 150, 2, [150, 77]),          # 64 rows, combine kernel
    (2, 8, 2, 128, 400, 64, [400, 70]),          # 64 new tokens, 256 rows
    (2, 4, 1, 64, 90, 8, [90, 5]),               # L < sq: three tokens dropped
]


@pytest.mark.parametrize("case", APPEND, ids=lambda c: "B%d_H%d_G%d_D%d_T%d_sq%d" % c[:6])
def test_f16_append(gqa, orc, case):
    """gqa_decode_append with fp16 q/k/v: the output against the oracle's
    append-then-attend, and the cache rows it writes bit for bit."""
    B, H, G, D, T, sq, lens = case
    x = gi.make_custom(B, H, G, D, T, sq, dtype="f16", seed=640 + T + sq, seq_lens=lens)
    gen = torch.Generator().manual_seed(641 + sq)
    kn = torch.randn(B, G, sq, D, generator=gen).to(torch.float16)
    vn = torch.randn(B, G, sq, D, generator=gen).to(torch.float16)
    want, k_after, v_after = orc.decode_append_f64(x["q"], kn, vn, x["k"], x["v"], x["seq_lens"],
                                                   1.0 / math.sqrt(D), threads=8)
    kc, vc = x["k"].cuda(), x["v"].cuda()
    got = gqa.decode_append(x["q"].cuda(), kn.cuda(), vn.cuda(), kc, vc, x["seq_lens"].cuda())
    torch.cuda.synchronize()
    _compare(got, want, "append %s" % (case,))
    assert np.array_equal(kc.double().cpu().numpy(), k_after)
    assert np.array_equal(vc.double().cpu().numpy(), v_after)
    assert kc.dtype == torch.float16


def _to_pages(k, ps, perm):
    B, G, T, D = k.shape
    n = T // ps
    pages = torch.empty(B * n, G, ps, D, dtype=k.dtype)
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
    (2, 32, 1, 128, 320, 2, 32, [320, 33]),
    (2, 8, 2, 128, 256, 64, 16, [256, 100]),
]


@pytest.mark.parametrize("case", PAGED, ids=lambda c: "B%d_H%d_G%d_D%d_T%d_sq%d_ps%d" % c[:7])
def test_f16_paged(gqa, orc, case):
    """gqa_decode_paged with fp16 q/k/v, pages in random order and table
    entries past each sequence's length poisoned, against the oracle."""
    B, H, G, D, T, sq, ps, lens = case
    x = gi.make_custom(B, H, G, D, T, sq, dtype="f16", seed=650 + T + ps, seq_lens=lens)
    perm = np.random.default_rng(ps + 1).permutation(B * (T // ps))
    kp, bt = _to_pages(x["k"], ps, perm)
    vp, _ = _to_pages(x["v"], ps, perm)
    for b, L in enumerate(lens):
        bt[b, (L + ps - 1) // ps:] = -7
    want = orc.decode_paged_f64(x["q"], kp, vp, bt, x["seq_lens"], threads=8)
    got = gqa.decode_paged(x["q"].cuda(), kp.cuda(), vp.cuda(), bt.cuda(), x["seq_lens"].cuda())
    torch.cuda.synchronize()
    _compare(got, want, "paged %s" % (case,))


@pytest.mark.parametrize("path_name", ["auto", "valu"])
def test_f16_large_magnitudes(gqa, orc, path_name):
    """fp16 fields far from N(0, 1): queries and keys ~ N(0, 8^2) (scores in
    the thousands, a sharply peaked softmax) and V up to 6e4 (near fp16's
    largest value).  The weights stay in (0, 2^8] and every product and sum
    is in fp32, so nothing overflows; the error bar scales with max |V|."""
    path = {"auto": gqa.PATH_AUTO, "valu": gqa.PATH_VALU}[path_name]
    B, H, G, D, T = 2, 32, 8, 128, 400
    g = torch.Generator().manual_seed(660)
    q = (8.0 * torch.randn(B, H, 1, D, generator=g)).to(torch.float16)
    k = (8.0 * torch.randn(B, G, T, D, generator=g)).to(torch.float16)
    v = (torch.rand(B, G, T, D, generator=g) * 1.2e5 - 6e4).to(torch.float16)
    lens = torch.tensor([400, 131], dtype=torch.int32)
    want = orc.decode_f64(q, k, v, lens, 1.0 / math.sqrt(D))
    got = gqa.decode(q.cuda(), k.cuda(), v.cuda(), lens.cuda(), path=path)
    torch.cuda.synchronize()
    _compare(got, want, "large %s" % path_name, tol=TOL * float(v.abs().max()))
