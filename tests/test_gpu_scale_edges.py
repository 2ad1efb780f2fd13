"""GPU parity at the edges of the work split: more sequences than the LDS
copy of seq_lens holds, a very long single sequence, negative and tiny
scales, head dim 64 for every cache variant.  Same tolerances as the other
parity tests (bf16 inputs: 2e-3 max abs)."""
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


def _err(got, want):
    g = got.double().cpu().numpy()
    assert np.isfinite(g).all()
    return float(np.abs(g - want).max())


def test_more_sequences_than_the_lds_length_window(gqa, orc):
    """300 ragged sequences: the schedule reads lengths past the first 256
    from memory."""
    B, H, G, D, T = 300, 8, 2, 64, 96
    lens = [int(x) for x in np.random.default_rng(3).integers(0, 97, size=B)]
    x = gi.make_custom(B, H, G, D, T, 1, dtype="bf16", seed=700, seq_lens=lens)
    want = orc.decode_f64(x["q"], x["k"], x["v"], x["seq_lens"], threads=8)
    for path in (gqa.PATH_MFMA, gqa.PATH_MFMA_QK):
        got = gqa.decode(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), x["seq_lens"].cuda(), path=path)
        torch.cuda.synchronize()
        assert _err(got, want) <= TOL
    # 32 query rows per KV head: the multi-wave kernel
    x = gi.make_custom(B, 32, 1, 64, T, 1, dtype="bf16", seed=701, seq_lens=lens)
    want = orc.decode_f64(x["q"], x["k"], x["v"], x["seq_lens"], threads=8)
    got = gqa.decode(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), x["seq_lens"].cuda())
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL


@pytest.mark.parametrize("B", [63, 64, 65, 129])
def test_batch_sizes_around_one_wave_of_sequences(gqa, orc, B):
    """Up to 64 sequences the split is planned in one pass over the wave (one
    sequence per lane); more take the loop over 64-sequence windows.  Ragged
    lengths with empty sequences, on every kernel family."""
    T = 80
    lens = [int(x) for x in np.random.default_rng(B).integers(0, T + 1, size=B)]
    lens[0], lens[-1] = 0, T
    for (H, G, dt, kw) in [(8, 2, "bf16", {}),                       # 4 rows: one-wave / row-split kernel
                           (8, 2, "bf16", {"path": gqa.PATH_MFMA_QK}),
                           (8, 2, "f32", {}),                        # vector-ALU kernel
                           (32, 1, "bf16", {})]:                     # 32 rows: 32 x 32 kernel
        x = gi.make_custom(B, H, G, 64, T, 1, dtype=dt, seed=710 + B, seq_lens=lens)
        want = orc.decode_f64(x["q"], x["k"], x["v"], x["seq_lens"], threads=8)
        got = gqa.decode(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), x["seq_lens"].cuda(), **kw)
        torch.cuda.synchronize()
        assert _err(got, want) <= (TOL if dt == "bf16" else 1e-5), (H, G, dt, kw)


def test_one_long_sequence(gqa, orc):
    """131072 cache rows in one (sequence, KV head): every workgroup holds a
    piece of the same two segments."""
    B, H, G, D, T = 1, 8, 2, 128, 131072
    x = gi.make_custom(B, H, G, D, T, 1, dtype="bf16", seed=702)
    want = orc.decode_f64(x["q"], x["k"], x["v"], None, threads=8)
    for m in (gqa.MERGE_IN_KERNEL, gqa.MERGE_COMBINE):
        got = gqa.decode(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), None, merge=m)
        torch.cuda.synchronize()
        assert _err(got, want) <= TOL


@pytest.mark.parametrize("scale", [-0.3, 1e-4, 0.0, 4.0])
def test_scales(gqa, orc, scale):
    x = gi.make_custom(2, 32, 8, 128, 300, 2, dtype="bf16", seed=703, seq_lens=[300, 77])
    want = orc.decode_f64(x["q"], x["k"], x["v"], x["seq_lens"], scale, threads=8)
    got = gqa.decode(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), x["seq_lens"].cuda(), scale=scale)
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL


def test_head_dim_64_variants(gqa, orc):
    B, H, G, D, T, sq = 2, 32, 8, 64, 256, 2
    x = gi.make_custom(B, H, G, D, T, sq, dtype="bf16", seed=704, seq_lens=[256, 50])
    # paged
    ps = 16
    n = T // ps
    perm = np.random.default_rng(1).permutation(B * n)
    kp = torch.empty(B * n, G, ps, D, dtype=torch.bfloat16)
    vp = torch.empty_like(kp)
    bt = torch.empty(B, n, dtype=torch.int32)
    for b in range(B):
        for i in range(n):
            kp[perm[b * n + i]] = x["k"][b, :, i * ps:(i + 1) * ps]
            vp[perm[b * n + i]] = x["v"][b, :, i * ps:(i + 1) * ps]
            bt[b, i] = int(perm[b * n + i])
    want = orc.decode_paged_f64(x["q"], kp, vp, bt, x["seq_lens"], threads=8)
    got = gqa.decode_paged(x["q"].cuda(), kp.cuda(), vp.cuda(), bt.cuda(), x["seq_lens"].cuda())
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL
    # append
    gen = torch.Generator().manual_seed(705)
    kn = torch.randn(B, G, sq, D, generator=gen).to(torch.bfloat16)
    vn = torch.randn(B, G, sq, D, generator=gen).to(torch.bfloat16)
    want, ka, va = orc.decode_append_f64(x["q"], kn, vn, x["k"], x["v"], x["seq_lens"], threads=8)
    kc, vc = x["k"].cuda(), x["v"].cuda()
    got = gqa.decode_append(x["q"].cuda(), kn.cuda(), vn.cuda(), kc, vc, x["seq_lens"].cuda())
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL
    assert np.array_equal(kc.double().cpu().numpy(), ka)
    # fp8
    ks = (x["k"].float().abs().amax(dim=(0, 2, 3)) / 448).float()
    vs = (x["v"].float().abs().amax(dim=(0, 2, 3)) / 448).float()
    kq = (x["k"].float() / ks.view(1, G, 1, 1)).to(torch.float8_e4m3fn).view(torch.uint8)
    vq = (x["v"].float() / vs.view(1, G, 1, 1)).to(torch.float8_e4m3fn).view(torch.uint8)
    want = orc.decode_fp8_f64(x["q"], kq, vq, ks, vs, x["seq_lens"], threads=8)
    got = gqa.decode_fp8(x["q"].cuda(), kq.cuda(), vq.cuda(), ks.cuda(), vs.cuda(), x["seq_lens"].cuda())
    torch.cuda.synchronize()
    assert _err(got, want) <= TOL
