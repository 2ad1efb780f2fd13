"""Pins of the oracle's cache variants: tokens appended before attending,
and a paged cache read through a block table.  CPU only.

Both variants are the plain definition on the cache they describe ("GQA
(Grouped-Query Attention) 분석", section "동작 원리", items 2-3 for the
append; its section "장단점" for paging as a layout orthogonal to GQA).
The pins below fix them against literal small examples and against other
formulations: the token-by-token incremental decode loop, page-permutation
invariance and shared pages."""
import math

import numpy as np
import pytest
import torch

import gqa_inputs as gi


def test_append_rows_literal_example(oracle_mod):
    # B=2, G=1, T=4, D=1: cache rows hold 0..3 (b=0) and 100..103 (b=1)
    k = np.array([[[[0.], [1.], [2.], [3.]]], [[[100.], [101.], [102.], [103.]]]])
    v = -k
    kn = np.array([[[[10.], [11.]]], [[[20.], [21.]]]])     # [B, G, sq=2, D]
    vn = -kn
    kc, vc = oracle_mod.append_rows(kn, vn, k, v, seq_lens=[3, 1])
    # b=0: L=3, new tokens at rows 1 and 2; b=1: L=1, token 0 would be row -1
    # (dropped), token 1 goes to row 0
    want_k = np.array([[[[0.], [10.], [11.], [3.]]], [[[21.], [101.], [102.], [103.]]]])
    assert np.array_equal(kc, want_k)
    assert np.array_equal(vc, -want_k)
    assert np.array_equal(k[0, 0, :, 0], [0., 1., 2., 3.])      # inputs untouched


def test_append_then_attend_equals_token_by_token_loop(oracle_mod):
    """sq new tokens appended at once and attended causally == the
    incremental loop: for each token, append it, then attend over every row
    up to and including it."""
    B, H, G, D, T, sq = 2, 8, 2, 16, 40, 3
    x = gi.make_custom(B, H, G, D, T, sq, dtype="f32", seed=61, seq_lens=[40, 17])
    gen = torch.Generator().manual_seed(62)
    kn = torch.randn(B, G, sq, D, generator=gen)
    vn = torch.randn(B, G, sq, D, generator=gen)
    out, kc, vc = oracle_mod.decode_append_f64(x["q"], kn, vn, x["k"], x["v"], x["seq_lens"])
    k = x["k"].double().numpy().copy()
    v = x["v"].double().numpy().copy()
    for b, L in enumerate([40, 17]):
        for s in range(sq):
            row = L - sq + s
            k[b, :, row] = kn[b, :, s].double().numpy()
            v[b, :, row] = vn[b, :, s].double().numpy()
            q1 = x["q"][b:b + 1, :, s:s + 1]
            one = oracle_mod.decode_f64(q1, k[b:b + 1], v[b:b + 1], [row + 1])
            assert np.allclose(one[0, :, 0], out[b, :, s], rtol=0, atol=1e-12)
    assert np.array_equal(kc, k) and np.array_equal(vc, v)


def test_gather_pages_literal_example(oracle_mod):
    # pages [num_pages=4, G=1, page_size=2, D=1] holding 10p + row
    pages = np.array([[[[10. * p], [10. * p + 1]]] for p in range(4)])
    bt = np.array([[2, 0], [1, 3]], dtype=np.int32)
    got = oracle_mod.gather_pages(pages, bt, seq_lens=[4, 3])
    want = np.array([[[[20.], [21.], [0.], [1.]]], [[[10.], [11.], [30.], [31.]]]])
    assert np.array_equal(got, want)


def _paged_from_contiguous(k, ps, perm):
    """Cut [B,G,T,D] into pages of ps rows, store page (b, i) at physical
    index perm[b * (T // ps) + i]; return pages and the block table."""
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


@pytest.mark.parametrize("ps", [16, 32])
def test_paged_equals_contiguous_under_any_page_order(oracle_mod, ps):
    B, H, G, D, T, sq = 3, 8, 2, 32, 64, 2
    x = gi.make_custom(B, H, G, D, T, sq, dtype="bf16", seed=63, seq_lens=[64, 33, 5])
    want = oracle_mod.decode_f64(x["q"], x["k"], x["v"], x["seq_lens"])
    n = B * (T // ps)
    for seed in (0, 1):
        perm = np.random.default_rng(seed).permutation(n) if seed else np.arange(n)
        kp, bt = _paged_from_contiguous(x["k"], ps, perm)
        vp, bt2 = _paged_from_contiguous(x["v"], ps, perm)
        assert torch.equal(bt, bt2)
        got = oracle_mod.decode_paged_f64(x["q"], kp, vp, bt, x["seq_lens"])
        assert np.array_equal(got, want)


def test_shared_pages_and_unused_table_entries(oracle_mod):
    """Two sequences sharing their first page read the same rows; table
    entries past a sequence's length are never looked up (here -1)."""
    ps, G, D, H = 16, 1, 16, 4
    gen = torch.Generator().manual_seed(64)
    kp = torch.randn(3, G, ps, D, generator=gen)
    vp = torch.randn(3, G, ps, D, generator=gen)
    q = torch.randn(2, H, 1, D, generator=gen)
    bt = torch.tensor([[0, 1, -1], [0, 2, -1]], dtype=torch.int32)
    lens = [20, 32]
    got = oracle_mod.decode_paged_f64(q, kp, vp, bt, lens)
    k = torch.stack([torch.cat([kp[0], kp[1], kp[1]], 1), torch.cat([kp[0], kp[2], kp[2]], 1)])
    v = torch.stack([torch.cat([vp[0], vp[1], vp[1]], 1), torch.cat([vp[0], vp[2], vp[2]], 1)])
    want = oracle_mod.decode_f64(q, k, v, lens)
    assert np.array_equal(got, want)
    with pytest.raises(ValueError):
        oracle_mod.decode_paged_f64(q, kp, vp, bt, [20, 40])     # needs entry -1


# ---------------------------------------------------------------------------
# fp8 E4M3 cache
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x80, -0.0), (0x38, 1.0), (0xB8, -1.0), (0x3C, 1.5), (0x40, 2.0),
    (0x7E, 448.0), (0xFE, -448.0),                 # largest finite
    (0x08, 2.0 ** -6), (0x07, 7 * 2.0 ** -9),     # smallest normal, largest subnormal
    (0x01, 2.0 ** -9),                             # smallest subnormal
    (0x28, 0.25), (0x30, 0.5), (0x22, 0.15625),     # 2^-2; 2^-1; (1 + 2/8) * 2^-3
])
def test_fp8_e4m3_literal_codes(oracle_mod, code, value):
    got = oracle_mod.fp8_e4m3_value(code)
    assert got == value and np.signbit(got) == np.signbit(value)


def test_fp8_e4m3_nan_codes_and_library_agreement(oracle_mod):
    assert np.isnan(oracle_mod.fp8_e4m3_value(0x7F)) and np.isnan(oracle_mod.fp8_e4m3_value(0xFF))
    # every code, against torch's float8_e4m3fn (a library with the same definition)
    codes = torch.arange(256, dtype=torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).double().numpy()
    ours = np.array([oracle_mod.fp8_e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(lib), np.isnan(ours))
    ok = ~np.isnan(lib)
    assert np.array_equal(lib[ok], ours[ok])
    # monotone over the positive codes, symmetric in the sign bit
    pos = ours[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(ours[0x80:0xFF], -ours[:0x7F])


def test_fp8_decode_equals_decode_of_dequantized_cache(oracle_mod):
    """With power-of-two scales every dequantized value is exactly a bf16
    number, so the fp8 decode equals the bf16 decode of that cache."""
    B, H, G, D, T, sq = 2, 8, 2, 32, 50, 1
    gen = torch.Generator().manual_seed(70)
    kc = torch.randint(0, 256, (B, G, T, D), generator=gen, dtype=torch.uint8)
    vc = torch.randint(0, 256, (B, G, T, D), generator=gen, dtype=torch.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x38      # no NaN codes
    vc[(vc & 0x7F) == 0x7F] = 0x38
    ks = torch.tensor([0.25, 2.0 ** -10])
    vs = torch.tensor([1.0, 0.5])
    q = torch.randn(B, H, sq, D, generator=gen).to(torch.bfloat16)
    lens = [50, 9]
    kd = kc.view(torch.float8_e4m3fn).to(torch.float32) * ks.view(1, G, 1, 1)
    vd = vc.view(torch.float8_e4m3fn).to(torch.float32) * vs.view(1, G, 1, 1)
    assert torch.equal(kd.to(torch.bfloat16).to(torch.float32), kd)      # exact in bf16
    want = oracle_mod.decode_f64(q, kd.to(torch.bfloat16), vd.to(torch.bfloat16), lens)
    got = oracle_mod.decode_fp8_f64(q, kc, vc, ks, vs, lens)
    assert np.array_equal(got, want)
    # scaling V's scale scales the output; K's scale acts as a score scale
    got2 = oracle_mod.decode_fp8_f64(q, kc, vc, ks, 2 * vs, lens)
    assert np.array_equal(got2, 2 * got)
    got3 = oracle_mod.decode_fp8_f64(q, kc, vc, 2 * ks, vs, lens, scale=0.5 / math.sqrt(D))
    assert np.allclose(got3, oracle_mod.decode_fp8_f64(q, kc, vc, ks, vs, lens, scale=1 / math.sqrt(D)),
                       rtol=0, atol=1e-12)


def test_int8_dequant_literal_codes(oracle_mod):
    """Two's-complement codes times the KV head's scale, at the ends of the
    range (0x80 = -128, 0x7F = 127) and around zero."""
    codes = np.array([0, 1, -1, 127, -128, 64, -64, 5], dtype=np.int8).reshape(1, 2, 1, 4)
    sc = np.array([0.5, 2.0 ** -7])
    got = oracle_mod.dequant_int8(codes, sc)
    want = np.array([[0.0, 0.5, -0.5, 63.5], [-1.0, 0.5, -0.5, 5.0 / 128]]).reshape(1, 2, 1, 4)
    assert np.array_equal(got, want)
    with pytest.raises(ValueError):
        oracle_mod.dequant_int8(codes.astype(np.uint8), sc)


def test_int8_decode_equals_decode_of_dequantized_cache(oracle_mod):
    """Every int8 code times a power-of-two scale is exactly a bf16 number
    (at most 8 significant bits), so the int8 decode equals the bf16 decode
    of that cache; V's scale scales the output."""
    B, H, G, D, T, sq = 2, 8, 2, 32, 50, 2
    gen = torch.Generator().manual_seed(71)
    kc = torch.randint(-128, 128, (B, G, T, D), generator=gen, dtype=torch.int8)
    vc = torch.randint(-128, 128, (B, G, T, D), generator=gen, dtype=torch.int8)
    ks = torch.tensor([2.0 ** -5, 2.0 ** -9])
    vs = torch.tensor([1.0, 0.25])
    q = torch.randn(B, H, sq, D, generator=gen).to(torch.bfloat16)
    lens = [50, 9]
    kd = kc.to(torch.float32) * ks.view(1, G, 1, 1)
    vd = vc.to(torch.float32) * vs.view(1, G, 1, 1)
    assert torch.equal(kd.to(torch.bfloat16).to(torch.float32), kd)      # exact in bf16
    want = oracle_mod.decode_f64(q, kd.to(torch.bfloat16), vd.to(torch.bfloat16), lens)
    got = oracle_mod.decode_int8_f64(q, kc, vc, ks, vs, lens)
    assert np.array_equal(got, want)
    assert np.array_equal(oracle_mod.decode_int8_f64(q, kc, vc, ks, 2 * vs, lens), 2 * got)
