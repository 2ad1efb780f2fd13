"""Pins for the float64 oracle: facts fixed by the pages and by mathematics.

Every check compares the oracle with something that is not the oracle:
a table printed on a page, a closed form, an invariant, a different
formulation written here from a page's description (repeat-then-MHA, the
Q-reshape batched form), or a library routine (torch's CPU scaled
dot-product attention in float64 with its grouped-query flag).
CPU only.
"""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import gqa_inputs as gi
from conftest import GOLDEN

TOL = 1e-12


def _draw(B, H, G, D, T, sq, seed, dtype="f32", seq_lens=None, poison=False):
    x = gi.make_custom(B, H, G, D, T, sq, dtype=dtype, seed=seed,
                       seq_lens=seq_lens, poison_tail=poison)
    return x["q"], x["k"], x["v"], x["seq_lens"]


def _visible(L, T, sq, s):
    """Last visible row index for query s (the causal, end-aligned reading)."""
    L = max(0, min(int(L), T))
    return L - sq + s


# ---------------------------------------------------------------------------
# 1. The head -> KV head mapping printed on the page
# ---------------------------------------------------------------------------
def test_head_table_matches_page(oracle_mod):
    # "Same GQA, Different Execution Cost Across Backends", section 1 table.
    rows = []
    with open(os.path.join(GOLDEN, "head_to_kv_h32_g8.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            heads, kv = line.rstrip("\n").split("\t")
            rows.append(([int(h) for h in heads.split(",")], int(kv)))
    assert len(rows) == 8
    seen = []
    for heads, kv in rows:
        for h in heads:
            assert oracle_mod.kv_head(h, 32, 8) == kv
            seen.append(h)
    assert sorted(seen) == list(range(32))


def test_mapping_axis_ends(oracle_mod):
    # "질의 헤드는 그대로, 키·값 헤드만 줄인다", table of the three names:
    # g=h gives one query head per KV head (MHA), g=1 gives all h (MQA),
    # in between h/g query heads per KV head.
    with open(os.path.join(GOLDEN, "mha_gqa_mqa_axis.txt")) as f:
        names = [ln.split("\t")[1] for ln in f if not ln.startswith("#") and ln.strip()]
    assert names == ["MHA", "GQA", "MQA"]
    for h_count in (1, 2, 8, 32, 64):
        assert [oracle_mod.kv_head(h, h_count, h_count) for h in range(h_count)] == \
            list(range(h_count))
        assert all(oracle_mod.kv_head(h, h_count, 1) == 0 for h in range(h_count))
    for H, G in ((32, 8), (32, 4), (12, 4), (64, 16), (6, 3)):
        per = [0] * G
        for h in range(H):
            per[oracle_mod.kv_head(h, H, G)] += 1
        assert per == [H // G] * G


def test_oracle_rejects_indivisible_heads(oracle_mod):
    q = torch.zeros(1, 6, 1, 4, dtype=torch.float64)
    k = torch.zeros(1, 4, 3, 4, dtype=torch.float64)
    with pytest.raises(ValueError):
        oracle_mod.decode_f64(q, k, k)


# ---------------------------------------------------------------------------
# 2. Independent formulations of the same result
# ---------------------------------------------------------------------------
def _mha_numpy(q, k, v, lens, scale):
    """Plain per-head attention (no grouping), numpy float64, with the
    end-aligned causal visibility; rows that see nothing are zero."""
    B, H, sq, D = q.shape
    T = k.shape[2]
    out = np.zeros((B, H, sq, D))
    for b in range(B):
        for h in range(H):
            for s in range(sq):
                last = _visible(lens[b], T, sq, s)
                if last < 0:
                    continue
                z = scale * (k[b, h, :last + 1] @ q[b, h, s])
                w = np.exp(z - z.max())
                out[b, h, s] = (w / w.sum()) @ v[b, h, :last + 1]
    return out


def _repeat_kv_expand_reshape(x, n_rep):
    """K/V physically repeated the way the HF eager path does it: insert a
    stride-0 repeat axis after the KV-head axis, then merge the two axes
    ("Same GQA, Different Execution Cost Across Backends", section 2)."""
    B, G, T, D = x.shape
    e = np.broadcast_to(x[:, :, None, :, :], (B, G, n_rep, T, D))
    return e.reshape(B, G * n_rep, T, D)


@pytest.mark.parametrize("B,H,G,D,T,sq,lens", [
    (1, 32, 8, 16, 37, 1, None),
    (2, 8, 2, 8, 20, 2, [20, 7]),
    (3, 12, 4, 8, 16, 1, [16, 1, 9]),
    (2, 6, 6, 4, 9, 3, [9, 5]),      # MHA
    (2, 6, 1, 4, 9, 2, [3, 9]),      # MQA
])
def test_group_indexed_equals_repeated_kv(oracle_mod, B, H, G, D, T, sq, lens):
    q, k, v, sl = _draw(B, H, G, D, T, sq, seed=7 + T, seq_lens=lens)
    scale = 1.0 / np.sqrt(D)
    n_rep = H // G
    kr = _repeat_kv_expand_reshape(k.double().numpy(), n_rep)
    vr = _repeat_kv_expand_reshape(v.double().numpy(), n_rep)
    # the repeat must agree with the reference semantics of SDPA's grouped
    # flag: repeat_interleave along the head axis (same page, section 3)
    assert np.array_equal(kr, k.double().repeat_interleave(n_rep, dim=1).numpy())
    ref = _mha_numpy(q.double().numpy(), kr, vr, sl.tolist(), scale)
    got = oracle_mod.decode_f64(q, k, v, sl, scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=TOL)


@pytest.mark.parametrize("B,H,G,D,T,sq,lens", [
    (1, 32, 8, 64, 64, 1, None),
    (2, 32, 8, 32, 40, 2, [40, 33]),
    (2, 16, 4, 16, 25, 4, [25, 10]),
])
def test_q_reshape_batched_form(oracle_mod, B, H, G, D, T, sq, lens):
    """Q folded to [B, G, n_rep*sq, D] rows, one batched product per KV head,
    with row r = (head within group) * sq + s; the mask is applied per new
    token s ("Same GQA, Different Execution Cost Across Backends", sections 6
    and 7)."""
    q, k, v, sl = _draw(B, H, G, D, T, sq, seed=11 + sq, seq_lens=lens)
    scale = 1.0 / np.sqrt(D)
    n_rep = H // G
    qf = q.double().numpy().reshape(B, G, n_rep * sq, D)
    kf, vf = k.double().numpy(), v.double().numpy()
    scores = scale * np.matmul(qf, np.swapaxes(kf, -1, -2))   # [B,G,R,T]
    rows_s = np.arange(n_rep * sq) % sq                        # s of row r
    out = np.zeros((B, G, n_rep * sq, D))
    for b in range(B):
        for r in range(n_rep * sq):
            last = _visible(sl[b], T, sq, rows_s[r])
            if last < 0:
                continue
            z = scores[b, :, r, :last + 1]
            w = np.exp(z - z.max(axis=-1, keepdims=True))
            p = w / w.sum(axis=-1, keepdims=True)
            out[b, :, r] = np.einsum("gt,gtd->gd", p, vf[b, :, :last + 1])
    ref = out.reshape(B, H, sq, D)
    got = oracle_mod.decode_f64(q, k, v, sl, scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=TOL)


@pytest.mark.parametrize("B,H,G,D,T,sq,lens,scale", [
    (1, 32, 8, 64, 256, 1, None, None),
    (3, 32, 8, 128, 70, 1, [70, 33, 1], None),
    (2, 32, 32, 16, 50, 2, [50, 2], 0.3),
    (2, 32, 1, 16, 50, 2, [31, 50], -0.7),
    (2, 8, 4, 8, 12, 3, [12, 6], 2.0),
])
def test_matches_torch_sdpa_grouped(oracle_mod, B, H, G, D, T, sq, lens, scale):
    """torch's CPU scaled_dot_product_attention in float64 with its
    grouped-query flag ("Same GQA, Different Execution Cost Across Backends",
    section 3) and an explicit boolean visibility mask."""
    q, k, v, sl = _draw(B, H, G, D, T, sq, seed=23 + B + T, seq_lens=lens)
    sc = (1.0 / np.sqrt(D)) if scale is None else scale
    mask = torch.zeros(B, 1, sq, T, dtype=torch.bool)
    for b in range(B):
        for s in range(sq):
            last = _visible(sl[b], T, sq, s)
            if last >= 0:
                mask[b, 0, s, :last + 1] = True
    ref = F.scaled_dot_product_attention(
        q.double(), k.double(), v.double(), attn_mask=mask, scale=sc,
        enable_gqa=True).numpy()
    got = oracle_mod.decode_f64(q, k, v, sl, sc)
    vis = mask.any(-1).expand(B, H, sq).numpy()
    np.testing.assert_allclose(got[vis], ref[vis], rtol=0, atol=TOL)
    assert np.all(got[~vis] == 0.0)


# ---------------------------------------------------------------------------
# 3. Closed forms, invariants and reductions
# ---------------------------------------------------------------------------
def test_softmax_rows_sum_to_one(oracle_mod):
    q, k, v, sl = _draw(3, 16, 4, 32, 40, 2, seed=5, seq_lens=[40, 17, 1])
    out, p = oracle_mod.decode_f64(q, k, v, sl, 0.2, return_probs=True)
    for b in range(3):
        for s in range(2):
            last = _visible(sl[b], 40, 2, s)
            sums = p[b, :, s].sum(-1)
            if last < 0:
                assert np.all(p[b, :, s] == 0)
            else:
                np.testing.assert_allclose(sums, 1.0, rtol=0, atol=TOL)
                assert np.all(p[b, :, s, last + 1:] == 0)
                assert np.all(p[b, :, s, :last + 1] > 0)


def test_constant_v_returns_constant(oracle_mod):
    B, H, G, D, T = 2, 32, 8, 16, 33
    q, k, v, sl = _draw(B, H, G, D, T, 1, seed=3, seq_lens=[33, 12])
    c = torch.randn(B, G, 1, D, dtype=torch.float64)
    vc = c.expand(B, G, T, D).contiguous()
    got = oracle_mod.decode_f64(q, k, vc, sl)
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(got[b, h, 0], c[b, h // (H // G), 0].numpy(),
                                       rtol=0, atol=TOL)


def test_single_row_returns_v(oracle_mod):
    q, k, v, sl = _draw(2, 8, 2, 16, 1, 1, seed=4)
    got = oracle_mod.decode_f64(q, k, v, sl)
    for b in range(2):
        for h in range(8):
            assert np.array_equal(got[b, h, 0], v[b, h // 4, 0].double().numpy())
    # L = 1 inside a larger cache behaves the same
    q, k, v, sl = _draw(2, 8, 2, 16, 9, 1, seed=4, seq_lens=[1, 1])
    got = oracle_mod.decode_f64(q, k, v, sl)
    for b in range(2):
        for h in range(8):
            assert np.array_equal(got[b, h, 0], v[b, h // 4, 0].double().numpy())


def test_scale_zero_gives_mean_of_visible_v(oracle_mod):
    B, H, G, D, T, sq = 2, 8, 2, 8, 21, 2
    q, k, v, sl = _draw(B, H, G, D, T, sq, seed=9, seq_lens=[21, 6])
    got = oracle_mod.decode_f64(q, k, v, sl, 0.0)
    vd = v.double().numpy()
    for b in range(B):
        for h in range(H):
            for s in range(sq):
                last = _visible(sl[b], T, sq, s)
                np.testing.assert_allclose(got[b, h, s], vd[b, h // 4, :last + 1].mean(0),
                                           rtol=0, atol=TOL)


def test_multi_token_rows_reduce_to_single_token_decode(oracle_mod):
    """With sq new tokens, query s equals a one-token decode over the first
    L - sq + s + 1 cache rows (the causal reading)."""
    B, H, G, D, T, sq = 2, 16, 4, 16, 30, 3
    q, k, v, sl = _draw(B, H, G, D, T, sq, seed=13, seq_lens=[30, 11])
    got = oracle_mod.decode_f64(q, k, v, sl, 0.25)
    for s in range(sq):
        one = oracle_mod.decode_f64(q[:, :, s:s + 1].contiguous(), k, v,
                                    torch.tensor([L - sq + s + 1 for L in sl.tolist()],
                                                 dtype=torch.int32), 0.25)
        assert np.array_equal(got[:, :, s], one[:, :, 0])


def test_zero_and_short_lengths(oracle_mod):
    q, k, v, sl = _draw(3, 4, 2, 8, 10, 2, seed=2, seq_lens=[0, 1, -5])
    got = oracle_mod.decode_f64(q, k, v, sl)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert np.all(got[1, :, 0] == 0)                        # sees nothing
    for h in range(4):
        assert np.array_equal(got[1, h, 1], v[1, h // 2, 0].double().numpy())
    # lengths beyond the capacity clamp to T
    q, k, v, _ = _draw(1, 4, 2, 8, 10, 1, seed=2)
    a = oracle_mod.decode_f64(q, k, v, torch.tensor([10], dtype=torch.int32))
    b = oracle_mod.decode_f64(q, k, v, torch.tensor([99], dtype=torch.int32))
    c = oracle_mod.decode_f64(q, k, v, None)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_rows_beyond_length_are_never_read(oracle_mod):
    args = (3, 8, 2, 16, 24, 2)
    clean = _draw(*args, seed=17, seq_lens=[24, 10, 3])
    dirty = _draw(*args, seed=17, seq_lens=[24, 10, 3], poison=True)
    assert torch.isnan(dirty[1]).any()
    a = oracle_mod.decode_f64(*clean)
    b = oracle_mod.decode_f64(*dirty)
    assert np.array_equal(a, b)


def test_joint_permutation_of_cache_rows(oracle_mod):
    q, k, v, sl = _draw(2, 8, 2, 16, 31, 1, seed=19)
    perm = torch.randperm(31, generator=torch.Generator().manual_seed(0))
    a = oracle_mod.decode_f64(q, k, v, sl)
    b = oracle_mod.decode_f64(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), sl)
    np.testing.assert_allclose(a, b, rtol=0, atol=TOL)


def test_split_and_logsumexp_merge_is_exact(oracle_mod):
    """Splitting the cache rows into chunks, normalising each chunk on its
    own and merging the chunks by their log-sum-exp weights gives the unsplit
    result for any chunking (the rewrite the GPU path relies on)."""
    B, H, G, D, T, sq = 2, 8, 2, 16, 53, 2
    q, k, v, sl = _draw(B, H, G, D, T, sq, seed=29, seq_lens=[53, 20])
    scale = 0.3
    ref = oracle_mod.decode_f64(q, k, v, sl, scale)
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    for chunk in (1, 5, 16, 53):
        out = np.zeros_like(ref)
        for b in range(B):
            for h in range(H):
                g = h // (H // G)
                for s in range(sq):
                    last = _visible(sl[b], T, sq, s)
                    parts = []
                    for c0 in range(0, last + 1, chunk):
                        c1 = min(c0 + chunk, last + 1)
                        z = scale * (kd[b, g, c0:c1] @ qd[b, h, s])
                        m = z.max()
                        w = np.exp(z - m)
                        parts.append((m + np.log(w.sum()), (w / w.sum()) @ vd[b, g, c0:c1]))
                    if not parts:
                        continue
                    M = max(p[0] for p in parts)
                    wts = np.array([np.exp(p[0] - M) for p in parts])
                    out[b, h, s] = sum(wi * p[1] for wi, p in zip(wts, parts)) / wts.sum()
        np.testing.assert_allclose(out, ref, rtol=0, atol=TOL)


def test_row_entry_matches_full_call(oracle_mod):
    B, H, G, D, T, sq = 3, 8, 2, 16, 29, 2
    q, k, v, sl = _draw(B, H, G, D, T, sq, seed=31, seq_lens=[29, 14, 2])
    full = oracle_mod.decode_f64(q, k, v, sl, 0.4)
    for b in range(B):
        for h in (0, 3, 7):
            for s in range(sq):
                row = oracle_mod.decode_row_f64(q[b, h, s], k[b], v[b], H, sq, h, s,
                                                int(sl[b]), 0.4)
                assert np.array_equal(row, full[b, h, s])


def test_threads_do_not_change_bits(oracle_mod):
    q, k, v, sl = _draw(4, 16, 4, 32, 50, 1, seed=37, seq_lens=(10, 50))
    a = oracle_mod.decode_f64(q, k, v, sl, threads=1)
    b = oracle_mod.decode_f64(q, k, v, sl, threads=5)
    assert np.array_equal(a, b)


def test_bf16_inputs_are_upcast_exactly(oracle_mod):
    """bf16 inputs reach the oracle as the exact stored values."""
    q, k, v, sl = _draw(1, 8, 2, 16, 12, 1, seed=41, dtype="bf16")
    assert q.dtype == torch.bfloat16
    a = oracle_mod.decode_f64(q, k, v, sl)
    b = oracle_mod.decode_f64(q.float(), k.float(), v.float(), sl)
    assert np.array_equal(a, b)


def test_f16_inputs_are_upcast_exactly(oracle_mod):
    """fp16 inputs reach the oracle as the exact stored values (fp32 holds
    every fp16 value, subnormals included)."""
    q, k, v, sl = _draw(1, 8, 2, 16, 12, 1, seed=42, dtype="f16")
    assert q.dtype == torch.float16
    k[0, 0, 0, :4] = torch.tensor([6e-8, -3e-5, 65504.0, -1.0 / 3.0], dtype=torch.float16)
    a = oracle_mod.decode_f64(q, k, v, sl)
    b = oracle_mod.decode_f64(q.float(), k.float(), v.float(), sl)
    assert np.array_equal(a, b)
    assert oracle_mod._f64(k)[0, 0, 0, 0] == float(torch.tensor(6e-8, dtype=torch.float16).double())
