"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of the oracle's C source (a text
substitution), builds it with gcc into a temporary directory, and runs a
battery of pins against it: the page's head table, torch's float64 SDPA
with the grouped-query flag, constant V, the single-row closed form and
the multi-token reduction.  At least one pin must fail for every mutant,
and all of them must pass for the unmodified source.  CPU only.
"""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import gqa_inputs as gi
from conftest import GOLDEN

MUTANTS = {
    "modulo_mapping": ("return h / (H / G);", "return h % G;"),
    "dropped_scale": ("z[j] = scale * acc;", "z[j] = acc;"),
    "flipped_max_sign": ("z[j] = exp(z[j] - m);", "z[j] = exp(m - z[j]);"),
    "k_used_as_v": ("J->v + ((size_t)b * G + g)", "J->k + ((size_t)b * G + g)"),
    "causal_off_by_one": ("const long last = L - sq + s;", "const long last = L - sq + s - 1;"),
    "missing_normalisation": ("for (long j = 0; j <= last; ++j) z[j] /= Z;", "(void)Z;"),
    "transposed_query_rows": ("const size_t row = ((size_t)b * H + h) * sq + s;",
                              "const size_t row = ((size_t)b * sq + s) * H + h;"),
    "first_row_skipped": ("for (long j = 1; j <= last; ++j)\n        if (z[j] > m) m = z[j];\n    double Z = 0.0;\n    for (long j = 0; j <= last; ++j) {",
                          "for (long j = 1; j <= last; ++j)\n        if (z[j] > m) m = z[j];\n    double Z = 0.0;\n    z[0] = -1.0e300;\n    for (long j = 0; j <= last; ++j) {"),
}


def _battery(oracle, lib):
    """Run the pins against ``lib``; return the names of the pins that fail."""
    failed = []
    # head table printed on the page
    with open(os.path.join(GOLDEN, "head_to_kv_h32_g8.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            heads, kv = line.rstrip("\n").split("\t")
            if any(oracle.kv_head(int(h), 32, 8, lib=lib) != int(kv) for h in heads.split(",")):
                failed.append("head_table")
                break
    # torch SDPA, grouped flag, ragged + causal
    B, H, G, D, T, sq = 2, 8, 2, 16, 19, 2
    x = gi.make_custom(B, H, G, D, T, sq, dtype="f32", seed=3, seq_lens=[19, 8])
    q, k, v, sl = x["q"], x["k"], x["v"], x["seq_lens"]
    mask = torch.zeros(B, 1, sq, T, dtype=torch.bool)
    for b in range(B):
        for s in range(sq):
            mask[b, 0, s, :int(sl[b]) - sq + s + 1] = True
    ref = F.scaled_dot_product_attention(q.double(), k.double(), v.double(),
                                         attn_mask=mask, scale=0.37, enable_gqa=True).numpy()
    got = oracle.decode_f64(q, k, v, sl, 0.37, lib=lib)
    if not np.allclose(got, ref, rtol=0, atol=1e-12):
        failed.append("sdpa")
    # constant V
    c = torch.randn(B, G, 1, D, dtype=torch.float64)
    got = oracle.decode_f64(q, k, c.expand(B, G, T, D).contiguous(), sl, 0.37, lib=lib)
    want = c[:, torch.arange(H) // (H // G), 0].unsqueeze(2).expand(B, H, sq, D).numpy()
    if not np.allclose(got, want, rtol=0, atol=1e-12):
        failed.append("constant_v")
    # single visible row returns V
    x1 = gi.make_custom(1, 4, 2, 8, 5, 1, dtype="f32", seed=5, seq_lens=[1])
    got = oracle.decode_f64(x1["q"], x1["k"], x1["v"], x1["seq_lens"], lib=lib)
    want = x1["v"][0, torch.arange(4) // 2, 0].double().numpy()
    if not np.array_equal(got[0, :, 0], want):
        failed.append("single_row")
    return failed


@pytest.fixture(scope="module")
def oracle_src(oracle_mod):
    with open(oracle_mod.SOURCE_PATH) as f:
        return f.read()


def test_unmodified_oracle_passes_battery(oracle_mod):
    assert _battery(oracle_mod, None) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(oracle_mod, oracle_src, tmp_path, name):
    old, new = MUTANTS[name]
    assert oracle_src.count(old) == 1, "mutation anchor missing: " + name
    src = tmp_path / ("oracle_%s.c" % name)
    src.write_text(oracle_src.replace(old, new))
    so = oracle_mod.compile_c(str(src), str(tmp_path / ("liboracle_%s.so" % name)))
    lib = oracle_mod.load_library(so)
    failed = _battery(oracle_mod, lib)
    assert failed, "no pin caught the planted mistake '%s'" % name
