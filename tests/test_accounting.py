"""The byte and FLOP accounting behind every roofline figure bench.py
reports, pinned to the sizes the pages print (tests/golden/sizes.txt) and
to a brute-force count of the multiplies.  CPU only."""
import os

import numpy as np
import pytest

import bench
from conftest import GOLDEN

MiB = 1 << 20
KiB = 1 << 10
UNIT = {"MiB": MiB, "KiB": KiB, "ratio": 1, "x": 1, "count": 1}


def _golden():
    vals = {}
    for line in open(os.path.join(GOLDEN, "sizes.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        key, val, unit, cite = line.rstrip("\n").split("\t")
        assert cite.strip(), key
        vals[key] = float(val) * UNIT[unit]
    return vals


G = _golden()

# The Exaone4-1.2B decode layer of "Same GQA, Different Execution Cost Across
# Backends" (sections 2 and 8): q [1, 32, 1, 64], K/V cache [1, 8, 4096, 64],
# 2-byte elements.
EX = dict(B=1, H=32, G=8, D=64, sq=1, L=4096)


def test_exaone_layer_sizes():
    kv = bench.kv_bytes(EX["G"], EX["D"], EX["L"], "bf16")
    assert kv == 2 * G["layer_k_or_v_bytes"] == 2 * G["k_cache_layer_bytes"]
    assert bench.q_bytes(EX["B"], EX["H"], EX["D"], EX["sq"], "bf16") == G["decode_q_bytes"]
    # repeat_kv's reshape materialises the 4x copy: 4 MiB -> 16 MiB
    rep = bench.repeat_kv_bytes(EX["B"], EX["H"], EX["D"], EX["L"], "bf16")
    assert rep == G["reshape_repeat_bytes"]
    assert rep == (EX["H"] // EX["G"]) * G["expand_view_bytes"]
    # the useful bytes of one step count K and V once, q in and fp32 out --
    # never the repeated copy
    ub = bench.useful_bytes(EX["B"], EX["H"], EX["G"], EX["D"], EX["sq"], EX["L"], "bf16")
    assert ub == 2 * G["layer_k_or_v_bytes"] + G["decode_q_bytes"] + 2 * G["decode_q_bytes"]
    assert ub < 2 * rep


def test_tile_outputs_of_the_old_graph():
    # 60 tile ops per call, each the repeated [1, 32, 4096, 64] 2-byte tensor
    per_tile = bench.repeat_kv_bytes(1, 32, 64, 4096, "bf16")
    assert G["tile_ops_per_call"] * per_tile == G["tile_output_per_decode_call"]
    assert G["tile_output_per_decode_call"] / 64 == G["tile_output_per_prefill_token_qlen64"]


@pytest.mark.parametrize("H", [8, 32])
def test_kv_ratios(H):
    mha = bench.kv_bytes(H, 128, 4096, "bf16")
    # GQA-8 over MHA at 32 query heads: 1/4
    if H == 32:
        assert bench.kv_bytes(8, 128, 4096, "bf16") / mha == G["gqa8_over_mha_kv_ratio"]
    # MQA keeps 1/h of MHA's cache
    assert mha / bench.kv_bytes(1, 128, 4096, "bf16") == G["mqa_kv_reduction_h%d" % H]


def test_flops_match_a_brute_force_multiply_count():
    """Scores and the weighted sum each take one multiply per (head, query
    token, cache row, head-dim element) -- the lesson page's count has no g
    term -- and 2 FLOP per multiply-add."""
    for H, D, sq, lens in ((4, 3, 1, [5]), (6, 2, 2, [4, 7]), (2, 4, 3, [3, 0, 6])):
        macs = 0
        for L in lens:
            for h in range(H):
                for s in range(sq):
                    for j in range(L):
                        for d in range(D):
                            macs += 1          # q . k
                        for d in range(D):
                            macs += 1          # p * v
        assert bench.flops(H, D, sq, sum(lens)) == 2 * macs


def test_headline_bytes_recomputed_by_hand():
    # batched GQA-8 decode with the seed's sum of lengths 80,681:
    # 2 * 80681 * 8 * 128 * 2 + 32*32*128*2 + 32*32*128*4
    assert bench.useful_bytes(32, 32, 8, 128, 1, 80681, "bf16") == 331255808


def test_code_cache_bytes_recomputed_by_hand():
    # the headline workload with an 8-bit cache: 2 * 80681 * 8 * 128 * 1 codes
    # + 32*32*128*2 (bf16 q) + 32*32*128*4 (fp32 out) + 2 * 8 * 4 (scales)
    assert bench.code_cache_bytes(32, 32, 8, 128, 1, 80681, scales=True) == 166021184
    assert bench.code_cache_bytes(32, 32, 8, 128, 1, 80681, scales=False) == 166021120
    # one byte less per K/V element than the bf16 cache, nothing else changes
    assert (bench.useful_bytes(32, 32, 8, 128, 1, 80681, "bf16")
            - bench.code_cache_bytes(32, 32, 8, 128, 1, 80681, scales=False)) == 2 * 80681 * 8 * 128


@pytest.mark.parametrize("ps", [16, 64, 256])
def test_page_table_bytes_count_the_pages_rows_touch(ps):
    """One int32 per page holding a row below L (clamped to [0, T]), counted
    here by walking every row."""
    rng = np.random.default_rng(ps)
    T = 4096
    lens = [0, 1, ps - 1, ps, ps + 1, T, T + 500, -3] + rng.integers(0, T + 1, 20).tolist()
    walked = sum(len({t // ps for t in range(min(max(L, 0), T))}) for L in lens)
    assert bench.page_table_bytes(lens, T, ps) == 4 * walked
